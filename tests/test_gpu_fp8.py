"""FP8 path: block quantization (bit for bit against the oracle) and the FP8
forward (against the oracle's exact attention of the dequantized tensors).

The forward's only departure from that reference is the rounding of P to E4M3
before P V (the oracle does not model it).  The kernel keeps the exact running
max, so every probability p = exp(S_ij - m) <= 1 relative to the max of its
tile's time and is stored as 2^8 p.  Where 2^8 p is an E4M3 normal (p >= 2^-14)
its rounding error is at most 2^-4 p (3 mantissa bits, half an ulp); below
that the subnormal spacing 2^-9 of the code gives at most 2^-18.  A later
rescale by alpha <= 1 only shrinks both.  Divided by the row sum Z_i (fp32,
from the unrounded p), the error of O_ic is therefore at most

    2^-4 (P |V|)_ic + 2^-18 sum_{j allowed, p_ij < 2^-14} |v_jc| / Z_i

with P and p from the final max, plus the bf16 output rounding (2^-8 |O|) and
fp32 accumulation noise.  (P |V|) is exact attention of |V_deq|, which the
oracle computes; the small second term is computed per row in numpy.  That
per-element bound is what the tests apply, together with the lse tolerance of
the bf16 path (the scores themselves are exact products of the codes).
"""
from __future__ import annotations

import math

import numpy as np
import pytest

import oracle
import workloads as W
from tests.gpu_cases import TOL_BF16, check, say, to_device, to_host64

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():  # pragma: no cover - CPU container
    pytest.skip("no GPU", allow_module_level=True)

import exact_io_aware_59_amd as fa  # noqa: E402

BLOCK = 64


def _signs(d, seed):
    return np.random.default_rng(seed).choice([-1.0, 1.0], size=d).astype(np.float32)


def _outliers(shape, seed):
    """bf16 N(0,1) draws with 0.1% of the entries replaced by N(0, 10^2) ones."""
    r = np.random.default_rng(seed)
    z = r.standard_normal(shape).astype(np.float32)
    m = r.random(shape) < 0.001
    z = np.where(m, r.standard_normal(shape).astype(np.float32) * 10, z)
    bits = W.f32_to_bf16_bits(z)
    return W.Tensor(W.bf16_bits_to_f32(bits), bits, "bf16")


def _subnormal_term(qd, kd, vd, scale, causal, rows):
    """2^-18 sum_{j allowed, p_ij < 2^-14} |v_jc| / Z_i for the given (bh, i) rows
    (fp64 numpy on the dequantized tensors; p_ij = exp(S_ij - max_j S_ij))."""
    BH = qd.shape[0] * qd.shape[1]
    N, d = qd.shape[2], qd.shape[3]
    q2, k2, v2 = (a.reshape(BH, N, d) for a in (qd, kd, vd))
    out = np.zeros((len(rows), d))
    for r, (bh, i) in enumerate(rows):
        n = i + 1 if causal else N
        s = scale * (k2[bh, :n] @ q2[bh, i])
        p = np.exp(s - s.max())
        out[r] = 2.0 ** -18 * (np.abs(v2[bh, :n])[p < 2.0 ** -14].sum(axis=0)) / p.sum()
    return out


def _fp8_bound(qd, kd, vd, scale, causal, o_ref, rows=None):
    """Per-element bound on |O - O_ref| (see the module docstring); rows = None
    means every row, in [B, H, N, d] layout, else [len(rows), d]."""
    B, H, N, d = qd.shape
    if rows is None:
        pv, _ = oracle.attn_fwd(qd, kd, np.abs(vd), scale, causal)
        all_rows = np.array([(bh, i) for bh in range(B * H) for i in range(N)])
        sub = _subnormal_term(qd, kd, vd, scale, causal, all_rows).reshape(B, H, N, d)
    else:
        pv, _ = oracle.attn_fwd_rows(qd, kd, np.abs(vd), scale, rows, causal)
        sub = _subnormal_term(qd, kd, vd, scale, causal, rows)
    return 2.0 ** -4 * pv + sub + 2.0 ** -8 * np.abs(o_ref) + 1e-5


QUANT = [
    # B, H, N, d, signs, k_side
    (1, 2, 150, 128, False, False),
    (1, 2, 150, 128, True, False),
    (1, 2, 150, 128, True, True),
    (2, 1, 64, 64, True, True),
    (1, 1, 1, 128, False, False),
    (1, 3, 333, 64, True, False),
]


@pytest.mark.parametrize("case", QUANT, ids=lambda c: "B{}H{}N{}d{}{}{}".format(
    c[0], c[1], c[2], c[3], "-signs" if c[4] else "", "-kside" if c[5] else ""))
def test_quantize_bit_exact(case):
    B, H, N, d, use_signs, k_side = case
    say(f"[fp8 quantize] B={B} H={H} N={N} d={d} signs={use_signs} k_side={k_side}")
    x = _outliers((B, H, N, d), 90 + N)
    x.values[0, 0, 0, :] = 0.0  # a zero row inside the first block
    x.bits[0, 0, 0, :] = 0
    sg = _signs(d, 91) if use_signs else None
    codes, exps = fa.quantize_fp8(to_device(x, "bf16"), None if sg is None else torch.from_numpy(sg).to("cuda:0"),
                                  k_side)
    torch.cuda.synchronize()
    rc, re = oracle.fp8_quantize(x.values, BLOCK, None if sg is None else sg.astype(np.float64), k_side)
    assert np.array_equal(exps.cpu().numpy(), re), "block exponents"
    got = codes.cpu().numpy()
    bad = np.count_nonzero(got != rc)
    assert bad == 0, f"{bad} of {rc.size} codes differ"


FWD = [
    # B, H, N, d, causal, signs, scale
    (1, 2, 256, 128, True, True, None),
    (1, 2, 200, 128, False, False, None),
    (2, 1, 333, 64, True, True, None),
    (1, 1, 130, 64, False, True, -0.2),
    (1, 2, 1000, 128, True, True, None),
]


def _fwd_case(B, H, N, d, causal, use_signs, sc, seed):
    scale = float(np.float32(1 / math.sqrt(d) if sc is None else sc))
    x = W.make_inputs(B, H, N, d, "bf16", seed=seed)
    sg = _signs(d, seed + 7) if use_signs else None
    q, k, v = (to_device(x[n], "bf16") for n in "qkv")
    o, lse = fa.forward_fp8(q, k, v, scale, causal, None if sg is None else torch.from_numpy(sg).to("cuda:0"))
    torch.cuda.synchronize()
    o_ref, l_ref, quant = oracle.attn_fp8_fwd(x["q"].values, x["k"].values, x["v"].values, scale, causal, BLOCK,
                                              None if sg is None else sg.astype(np.float64))
    deq = {n: oracle.fp8_dequantize(*quant[n], BLOCK) for n in "qkv"}
    return x, o, lse, o_ref, l_ref, deq, scale


@pytest.mark.parametrize("case", FWD, ids=lambda c: "B{}H{}N{}d{}{}{}{}".format(
    c[0], c[1], c[2], c[3], "c" if c[4] else "", "-signs" if c[5] else "", "" if c[6] is None else f"-s{c[6]}"))
def test_fwd_fp8(case):
    B, H, N, d, causal, use_signs, sc = case
    say(f"[fp8 fwd] B={B} H={H} N={N} d={d} causal={causal} signs={use_signs} scale={sc}")
    x, o, lse, o_ref, l_ref, deq, scale = _fwd_case(B, H, N, d, causal, use_signs, sc, seed=95)
    got = to_host64(o)
    bound = _fp8_bound(deq["q"], deq["k"], deq["v"], scale, causal, o_ref)
    err = np.abs(got - o_ref)
    rms = float(np.sqrt(np.mean(err ** 2)))
    say(f"    O: max|err| = {err.max():.3e}, rms {rms:.3e}, max err / per-element bound = "
        f"{(err / bound).max():.3f} (mean bound {bound.mean():.3e})")
    assert np.all(err <= bound), "O beyond the E4M3 rounding bound of P"
    check("lse", to_host64(lse), l_ref, TOL_BF16["lse"])


def test_fwd_fp8_deterministic():
    _, o1, l1, _, _, _, _ = _fwd_case(1, 2, 300, 128, True, True, None, seed=96)
    _, o2, l2, _, _, _, _ = _fwd_case(1, 2, 300, 128, True, True, None, seed=96)
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_incoherent_processing_lowers_error():
    """On inputs with rare large entries the FP8 forward with the incoherent map
    is closer to exact attention of the original bf16 inputs than without it
    (the pages: FP8 block quantization with incoherent processing has lower
    error than plain FP8)."""
    B, H, N, d = 1, 4, 512, 128
    scale = float(np.float32(1 / math.sqrt(d)))
    q, k, v = (_outliers((B, H, N, d), s) for s in (301, 302, 303))
    o_ex, _ = oracle.attn_fwd(q.values, k.values, v.values, scale, False)
    qd, kd, vd = (to_device(t, "bf16") for t in (q, k, v))
    sg = torch.from_numpy(_signs(d, 304)).to("cuda:0")
    o_inc, _ = fa.forward_fp8(qd, kd, vd, scale, False, sg)
    o_blk, _ = fa.forward_fp8(qd, kd, vd, scale, False, None)
    o_bf, _ = fa.forward(qd, kd, vd, scale, False)
    torch.cuda.synchronize()
    rms = {n: float(np.sqrt(np.mean((to_host64(t) - o_ex) ** 2))) for n, t in
           (("fp8 block + incoherent", o_inc), ("fp8 block", o_blk), ("bf16", o_bf))}
    say("    rms error vs exact fp64 attention: " + ", ".join(f"{n} {e:.3e}" for n, e in rms.items()))
    assert rms["fp8 block + incoherent"] < rms["fp8 block"]


def test_full_size_fp8_sampled_rows():
    w = W.WORKLOADS["fp8_causal_fwd_b2h16n4096d128"]
    say(f"[full fp8] {w.name}")
    x = W.workload_inputs(w, seed=0)
    sg = W.fp8_signs(w.d)
    q, k, v = (to_device(x[n], "bf16") for n in "qkv")
    o, lse = fa.forward_fp8(q, k, v, w.scale, w.causal, torch.from_numpy(sg).to("cuda:0"))
    torch.cuda.synchronize()
    sg64 = sg.astype(np.float64)
    qd = oracle.fp8_dequantize(*oracle.fp8_quantize(x["q"].values, BLOCK, sg64, False), BLOCK)
    kd = oracle.fp8_dequantize(*oracle.fp8_quantize(x["k"].values, BLOCK, sg64, True), BLOCK)
    vd = oracle.fp8_dequantize(*oracle.fp8_quantize(x["v"].values, BLOCK, None, False), BLOCK)
    rows = W.sample_rows(w.B * w.H, w.N, 512, seed=W.SEED_ROWS)
    o_ref, l_ref = oracle.attn_fwd_rows(qd, kd, vd, w.scale, rows, w.causal)
    idx0 = torch.from_numpy(rows[:, 0]).to("cuda:0")
    idx1 = torch.from_numpy(rows[:, 1]).to("cuda:0")
    got = to_host64(o.reshape(w.B * w.H, w.N, w.d)[idx0, idx1])
    bound = _fp8_bound(qd, kd, vd, w.scale, w.causal, o_ref, rows)
    err = np.abs(got - o_ref)
    say(f"    O rows: max|err| = {err.max():.3e}, rms {np.sqrt(np.mean(err ** 2)):.3e}, "
        f"max err / per-element bound = {(err / bound).max():.3f} (mean bound {bound.mean():.3e})")
    assert np.all(err <= bound)
    check("lse rows", to_host64(lse.reshape(w.B * w.H, w.N)[idx0, idx1]), l_ref, TOL_BF16["lse"])
