"""Head sizes other than 64 and 128, against the fp64 oracle.

"FlashAttention原理概览" section 3.4 requires the head size to be a multiple of
16 and "FlashAttention 深度解析" section 五 bounds it by 256.  The bf16 forward
takes every multiple of 16 up to 256 (rows shorter than the 64-, 128- or
256-wide tile are padded in LDS, with zero Q columns); the bf16 backward and
the fp32 path take every multiple of 16 up to 128, and reject larger sizes
as unsupported.  Small cases are compared element by element (ragged N,
causal, block masks, window and ALiBi, the four-wave launch); two full-size
workloads (d = 256 forward, d = 96 forward + backward) on sampled rows and
heads.
"""
from __future__ import annotations

import math

import numpy as np
import pytest

import oracle
import workloads as W
from tests.gpu_cases import TOL_BF16, TOL_F32, check, check_bf16_out, say, to_device, to_host64

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():  # pragma: no cover - CPU container
    pytest.skip("no GPU", allow_module_level=True)

import exact_io_aware_59_amd as fa  # noqa: E402


def _mask(kind, N, seed):
    if kind is None:
        return None
    return W.random_blockmask((N + 127) // 128, seed, p=0.6, keep_diag=True)


def _dev(m):
    return None if m is None else torch.from_numpy(np.ascontiguousarray(m)).to("cuda:0")


FWD = [
    # B, H, N, d, causal, mask
    (1, 2, 200, 16, True, None),
    (1, 1, 333, 32, False, None),
    (2, 1, 150, 48, True, None),
    (1, 2, 300, 80, False, "rand"),
    (1, 1, 777, 96, True, None),
    (1, 2, 260, 112, False, None),
    (1, 1, 390, 144, True, None),
    (1, 2, 200, 176, False, None),
    (1, 1, 520, 192, True, "rand"),
    (2, 1, 129, 224, False, None),
    (1, 1, 333, 240, True, None),
    (1, 2, 700, 256, True, None),
    (1, 1, 300, 256, False, "rand"),
    # at least 512 work items on the 256-CU part: the four-wave launch
    (1, 520, 130, 96, True, None),
    (1, 180, 300, 48, False, None),
]


@pytest.mark.parametrize("case", FWD, ids=lambda c: "B{}H{}N{}d{}{}{}".format(
    *c[:4], "c" if c[4] else "", "-" + c[5] if c[5] else ""))
def test_fwd_bf16_head_sizes(case):
    B, H, N, d, causal, mkind = case
    scale = float(np.float32(1 / math.sqrt(d)))
    say(f"[fwd bf16 head size] B={B} H={H} N={N} d={d} causal={causal} mask={mkind}")
    x = W.make_inputs(B, H, N, d, "bf16", seed=61)
    m = _mask(mkind, N, 8)
    q, k, v = (to_device(x[n], "bf16") for n in "qkv")
    o, lse = fa.forward(q, k, v, scale, causal, _dev(m))
    torch.cuda.synchronize()
    o_ref, lse_ref = oracle.attn_fwd(x["q"].values, x["k"].values, x["v"].values, scale, causal, m)
    check_bf16_out("O", to_host64(o), o_ref, TOL_BF16["o"])
    check("lse", to_host64(lse), lse_ref, TOL_BF16["lse"])


@pytest.mark.parametrize("d", [80, 208])
def test_fwd_bf16_head_sizes_window_alibi(d):
    B, H, N = 1, 2, 333
    scale = float(np.float32(1 / math.sqrt(d)))
    say(f"[fwd bf16 head size, window + ALiBi] B={B} H={H} N={N} d={d}")
    x = W.make_inputs(B, H, N, d, "bf16", seed=62)
    slopes = np.array([0.25, 0.0625], dtype=np.float32)
    q, k, v = (to_device(x[n], "bf16") for n in "qkv")
    o, lse = fa.forward(q, k, v, scale, True, None, window=(100, -1), alibi_slopes=torch.from_numpy(slopes).cuda())
    torch.cuda.synchronize()
    o_ref, lse_ref = oracle.attn_fwd(x["q"].values, x["k"].values, x["v"].values, scale, True, None,
                                     window=(100, -1), slopes=slopes.astype(np.float64))
    check_bf16_out("O", to_host64(o), o_ref, TOL_BF16["o"])
    check("lse", to_host64(lse), lse_ref, TOL_BF16["lse"])


BWD = [
    (1, 2, 200, 16, True, None),
    (1, 1, 300, 32, False, "rand"),
    (2, 1, 257, 48, True, None),
    (1, 1, 384, 80, False, None),
    (1, 2, 333, 96, True, None),
    (1, 1, 260, 112, True, "rand"),
]


@pytest.mark.parametrize("case", BWD, ids=lambda c: "B{}H{}N{}d{}{}{}".format(
    *c[:4], "c" if c[4] else "", "-" + c[5] if c[5] else ""))
def test_bwd_bf16_head_sizes(case):
    B, H, N, d, causal, mkind = case
    scale = float(np.float32(1 / math.sqrt(d)))
    say(f"[bwd bf16 head size] B={B} H={H} N={N} d={d} causal={causal} mask={mkind}")
    x = W.make_inputs(B, H, N, d, "bf16", seed=63, with_do=True)
    m = _mask(mkind, N, 9)
    q, k, v, do = (to_device(x[n], "bf16") for n in ("q", "k", "v", "do"))
    o, lse = fa.forward(q, k, v, scale, causal, _dev(m))
    dq, dk, dv = fa.backward(q, k, v, o, do, lse, scale, causal, _dev(m))
    torch.cuda.synchronize()
    rq, rk, rv = oracle.attn_bwd(x["q"].values, x["k"].values, x["v"].values, x["do"].values, scale, causal, m)
    check("dQ", to_host64(dq), rq, TOL_BF16["dq"])
    check("dK", to_host64(dk), rk, TOL_BF16["dk"])
    check("dV", to_host64(dv), rv, TOL_BF16["dv"])


def test_bwd_bf16_head_size_window_alibi():
    B, H, N, d = 1, 2, 300, 80
    scale = float(np.float32(1 / math.sqrt(d)))
    say(f"[bwd bf16 head size, window + ALiBi] B={B} H={H} N={N} d={d}")
    x = W.make_inputs(B, H, N, d, "bf16", seed=64, with_do=True)
    slopes = np.array([0.125, 0.5], dtype=np.float32)
    ts = torch.from_numpy(slopes).cuda()
    q, k, v, do = (to_device(x[n], "bf16") for n in ("q", "k", "v", "do"))
    o, lse = fa.forward(q, k, v, scale, False, None, window=(60, 30), alibi_slopes=ts)
    dq, dk, dv = fa.backward(q, k, v, o, do, lse, scale, False, None, window=(60, 30), alibi_slopes=ts)
    torch.cuda.synchronize()
    rq, rk, rv = oracle.attn_bwd(x["q"].values, x["k"].values, x["v"].values, x["do"].values, scale, False, None,
                                 window=(60, 30), slopes=slopes.astype(np.float64))
    check("dQ", to_host64(dq), rq, TOL_BF16["dq"])
    check("dK", to_host64(dk), rk, TOL_BF16["dk"])
    check("dV", to_host64(dv), rv, TOL_BF16["dv"])


@pytest.mark.parametrize("d", [16, 48, 80, 112])
def test_f32_head_sizes(d):
    B, H, N = 1, 2, 150
    scale = float(np.float32(1 / math.sqrt(d)))
    say(f"[f32 head size] B={B} H={H} N={N} d={d}")
    x = W.make_inputs(B, H, N, d, "f32", seed=65, with_do=True)
    q, k, v, do = (to_device(x[n], "f32") for n in ("q", "k", "v", "do"))
    o, lse = fa.forward(q, k, v, scale, True)
    dq, dk, dv = fa.backward(q, k, v, o, do, lse, scale, True)
    torch.cuda.synchronize()
    rq, rk, rv, ro, rl, _ = oracle.attn_bwd(x["q"].values, x["k"].values, x["v"].values, x["do"].values,
                                            scale, True, None, return_fwd=True)
    check("O", to_host64(o), ro, TOL_F32["o"])
    check("lse", to_host64(lse), rl, TOL_F32["lse"])
    check("dQ", to_host64(dq), rq, TOL_F32["dq"])
    check("dK", to_host64(dk), rk, TOL_F32["dk"])
    check("dV", to_host64(dv), rv, TOL_F32["dv"])


def test_unsupported_head_sizes_raise():
    """Larger than the path supports, or not a multiple of 16: an error, no launch."""
    x = W.make_inputs(1, 1, 64, 256, "bf16", seed=66, with_do=True)
    q, k, v, do = (to_device(x[n], "bf16") for n in ("q", "k", "v", "do"))
    o, lse = fa.forward(q, k, v, None, True)
    with pytest.raises(fa.FAError) as e:
        fa.backward(q, k, v, o, do, lse, None, True)
    assert e.value.status == 2
    y = torch.zeros((1, 1, 64, 72), dtype=torch.bfloat16, device="cuda:0")
    with pytest.raises(fa.FAError) as e:
        fa.forward(y, y, y, None, False)
    assert e.value.status == 2
    z = torch.zeros((1, 1, 64, 144), dtype=torch.float32, device="cuda:0")
    with pytest.raises(fa.FAError) as e:
        fa.forward(z, z, z, None, False)
    assert e.value.status == 2


@pytest.mark.parametrize("d", [256, 160])
def test_full_size_wide_fwd_sampled_rows(d):
    """Causal B=1 H=8 N=8192 forward at d = 256 (the benchmark workload) and
    d = 160 (a 192-wide tile with padded columns): 512 sampled rows."""
    w = W.WORKLOADS["bf16_causal_fwd_b1h8n8192d256"]
    say(f"[full fwd] B={w.B} H={w.H} N={w.N} d={d} causal")
    if d == w.d:
        x = W.workload_inputs(w, seed=0)
        scale = w.scale
    else:
        x = W.make_inputs(w.B, w.H, w.N, d, "bf16", seed=0)
        scale = float(np.float32(1 / math.sqrt(d)))
    q, k, v = (to_device(x[n], "bf16") for n in "qkv")
    o, lse = fa.forward(q, k, v, scale, w.causal)
    torch.cuda.synchronize()
    rows = W.sample_rows(w.B * w.H, w.N, 512, seed=W.SEED_ROWS)
    o_ref, l_ref = oracle.attn_fwd_rows(x["q"].values, x["k"].values, x["v"].values, scale, rows, w.causal)
    of = o.reshape(w.B * w.H, w.N, d)
    lf = lse.reshape(w.B * w.H, w.N)
    i0 = torch.from_numpy(rows[:, 0]).to("cuda:0")
    i1 = torch.from_numpy(rows[:, 1]).to("cuda:0")
    check("O rows", to_host64(of[i0, i1]), o_ref, TOL_BF16["o"], f"max|O| = {np.abs(o_ref).max():.3f}")
    check("lse rows", to_host64(lf[i0, i1]), l_ref, TOL_BF16["lse"])
    assert torch.isfinite(o).all() and torch.isfinite(lse).all()
    assert float(o.abs().max()) <= float(v.abs().max()) * (1 + 2 ** -7)


def test_full_size_d96_fwdbwd_sampled():
    w = W.WORKLOADS["bf16_causal_fwdbwd_b2h16n4096d96"]
    say(f"[full fwd+bwd] {w.name}")
    x = W.workload_inputs(w, seed=0)
    q, k, v, do = (to_device(x[n], "bf16") for n in ("q", "k", "v", "do"))
    o, lse = fa.forward(q, k, v, w.scale, w.causal)
    dq, dk, dv = fa.backward(q, k, v, o, do, lse, w.scale, w.causal)
    torch.cuda.synchronize()
    rows = W.sample_rows(w.B * w.H, w.N, 512, seed=W.SEED_ROWS)
    o_ref, l_ref = oracle.attn_fwd_rows(x["q"].values, x["k"].values, x["v"].values, w.scale, rows, w.causal)
    of = o.reshape(w.B * w.H, w.N, w.d)
    i0 = torch.from_numpy(rows[:, 0]).to("cuda:0")
    i1 = torch.from_numpy(rows[:, 1]).to("cuda:0")
    check("O rows", to_host64(of[i0, i1]), o_ref, TOL_BF16["o"])
    check("lse rows", to_host64(lse.reshape(w.B * w.H, w.N)[i0, i1]), l_ref, TOL_BF16["lse"])
    assert torch.isfinite(dq).all() and torch.isfinite(dk).all() and torch.isfinite(dv).all()
    for b, h in ((0, 3), (1, 12)):
        sl = (slice(b, b + 1), slice(h, h + 1))
        rq, rk, rv = oracle.attn_bwd(x["q"].values[sl], x["k"].values[sl], x["v"].values[sl],
                                     x["do"].values[sl], w.scale, w.causal)
        check("dQ", to_host64(dq[b:b + 1, h:h + 1]), rq, TOL_BF16["dq"])
        check("dK", to_host64(dk[b:b + 1, h:h + 1]), rk, TOL_BF16["dk"])
        check("dV", to_host64(dv[b:b + 1, h:h + 1]), rv, TOL_BF16["dv"])
