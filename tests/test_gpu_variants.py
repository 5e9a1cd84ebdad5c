"""Parity of the local-window and ALiBi variants (the _ex entry points) with the fp64 oracle.

Every output element of small shapes is compared: windows open on one side,
on both, of width zero (only the diagonal), together with causal and block
masks (including rows left with no key), ALiBi alone and combined, negative
and zero scales (scale 0 leaves only the bias), d = 64 and 128, ragged N.
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


def _mask_for(kind, N, seed):
    nb = (N + 127) // 128
    if kind is None:
        return None
    if kind == "rand":
        return W.random_blockmask(nb, seed, p=0.6, keep_diag=True)
    if kind == "rand_empty_rows":
        m = W.random_blockmask(nb, seed, p=0.5)
        m[-1, :] = 0
        return m
    raise ValueError(kind)


def _slopes(H, on):
    """The usual geometric ALiBi slopes 2^(-8 (h+1) / H) (fp32 values), or None;
    on = "strong" gives 0.5, 0.25, ... (nearly one-hot rows near the diagonal)."""
    if not on:
        return None
    if on == "strong":
        return np.array([0.5 ** (h + 1) for h in range(H)], dtype=np.float32)
    return np.array([2.0 ** (-8.0 * (h + 1) / H) for h in range(H)], dtype=np.float32)


def _dev(a, dtype=None):
    if a is None:
        return None
    return torch.from_numpy(np.ascontiguousarray(a)).to("cuda:0")


def _win(w):
    return None if w is None else (-1 if w[0] is None else w[0], -1 if w[1] is None else w[1])


def _id(c):
    B, H, N, d, causal, mk, win, al, sc = c
    return "B{}H{}N{}d{}{}{}-w{}{}{}".format(B, H, N, d, "c" if causal else "", "-" + mk if mk else "", win,
                                            "-alibi" if al else "", "" if sc is None else f"-s{sc}")


FWD = [
    # B, H, N, d, causal, mask, window (left, right; None = unbounded), alibi, scale (None = 1/sqrt(d))
    (1, 2, 333, 64, False, None, (100, 20), True, None),
    (1, 2, 300, 128, True, None, (64, None), False, None),
    (2, 2, 520, 128, False, None, (None, 0), True, None),
    (1, 3, 777, 64, False, None, None, True, None),
    (1, 2, 1000, 128, True, None, (250, None), True, None),
    (1, 1, 129, 64, False, None, (0, 0), False, None),
    (1, 1, 17, 128, False, None, (3, 5), True, None),
    (1, 2, 640, 64, False, "rand", (200, 100), True, None),
    (1, 1, 260, 128, False, "rand_empty_rows", (30, 30), False, None),
    (1, 1, 200, 128, True, None, (50, None), True, -0.09),
    (1, 1, 150, 64, False, None, (20, 20), True, 0.0),
    (1, 2, 700, 64, True, "rand", None, True, None),
    (1, 1, 300, 128, True, None, None, True, 0.0),
    (2, 2, 1100, 128, True, None, (400, None), True, None),
]
# At least 512 work items (the four-wave launch on a 256-CU MI355X; the cases
# above take the eight-wave tile-split one): non-causal window + ALiBi (the
# per-element path) and causal window + ALiBi (the linear-bias path).
FWD_FOUR_WAVE = [
    (1, 520, 130, 128, False, None, (50, 20), True, None),
    (1, 520, 130, 128, True, None, (40, None), True, None),
]
FWD = FWD + FWD_FOUR_WAVE


@pytest.mark.parametrize("case", FWD, ids=_id)
def test_fwd_variant_bf16(case):
    B, H, N, d, causal, mk, win, al, sc = case
    scale = float(np.float32(1 / math.sqrt(d) if sc is None else sc))
    say(f"[fwd variant bf16] B={B} H={H} N={N} d={d} causal={causal} mask={mk} window={win} alibi={al} "
        f"scale={scale}")
    x = W.make_inputs(B, H, N, d, "bf16", seed=31)
    m = _mask_for(mk, N, 7)
    sl = _slopes(H, al)
    q, k, v = (to_device(x[n], "bf16") for n in "qkv")
    o, lse = fa.forward(q, k, v, scale, causal, _dev(m), window=_win(win), alibi_slopes=_dev(sl))
    torch.cuda.synchronize()
    o_ref, lse_ref = oracle.attn_fwd(x["q"].values, x["k"].values, x["v"].values, scale, causal, m,
                                     window=_win(win), slopes=None if sl is None else sl.astype(np.float64))
    check_bf16_out("O", to_host64(o), o_ref, TOL_BF16["o"])
    check("lse", to_host64(lse), lse_ref, TOL_BF16["lse"])


BWD = [
    (1, 2, 333, 64, False, None, (100, 20), True, None),
    (1, 2, 300, 128, True, None, (64, None), True, None),
    (1, 1, 520, 128, False, None, (None, 0), True, None),
    (1, 2, 384, 128, True, "rand", (150, None), False, None),
    (1, 1, 260, 64, False, "rand_empty_rows", (30, 30), True, None),
    (1, 1, 256, 128, True, None, (40, None), True, -0.1),
    (1, 2, 640, 64, False, None, (0, 0), False, None),
    (1, 2, 1100, 128, True, None, (400, None), True, None),
    (1, 2, 900, 64, True, "rand", (300, None), True, None),
    (1, 1, 700, 128, True, None, None, True, None),
    (1, 1, 200, 64, True, None, None, True, 0.0),
    (1, 1, 600, 128, False, None, (200, 50), False, None),
]


def test_fwd_variant_bf16_strong_alibi():
    """Strong slopes (0.5, 0.25) with causal: rows near the diagonal are nearly
    one-hot (O_i close to V_i, up to ~4.5 in magnitude), the case the net rule
    for |O| >= 2 of check_bf16_out exists for."""
    B, H, N, d = 2, 2, 520, 128
    scale = float(np.float32(1 / math.sqrt(d)))
    x = W.make_inputs(B, H, N, d, "bf16", seed=33)
    sl = _slopes(H, "strong")
    q, k, v = (to_device(x[n], "bf16") for n in "qkv")
    o, lse = fa.forward(q, k, v, scale, True, None, window=(300, -1), alibi_slopes=_dev(sl))
    torch.cuda.synchronize()
    o_ref, lse_ref = oracle.attn_fwd(x["q"].values, x["k"].values, x["v"].values, scale, True, None,
                                     window=(300, -1), slopes=sl.astype(np.float64))
    check_bf16_out("O", to_host64(o), o_ref, TOL_BF16["o"])
    check("lse", to_host64(lse), lse_ref, TOL_BF16["lse"])


@pytest.mark.parametrize("case", BWD, ids=_id)
def test_bwd_variant_bf16(case):
    B, H, N, d, causal, mk, win, al, sc = case
    scale = float(np.float32(1 / math.sqrt(d) if sc is None else sc))
    say(f"[bwd variant bf16] B={B} H={H} N={N} d={d} causal={causal} mask={mk} window={win} alibi={al} "
        f"scale={scale}")
    x = W.make_inputs(B, H, N, d, "bf16", seed=41, with_do=True)
    m = _mask_for(mk, N, 8)
    sl = _slopes(H, al)
    q, k, v, do = (to_device(x[n], "bf16") for n in ("q", "k", "v", "do"))
    kw = dict(window=_win(win), alibi_slopes=_dev(sl))
    o, lse = fa.forward(q, k, v, scale, causal, _dev(m), **kw)
    dq, dk, dv = fa.backward(q, k, v, o, do, lse, scale, causal, _dev(m), **kw)
    torch.cuda.synchronize()
    rq, rk, rv = oracle.attn_bwd(x["q"].values, x["k"].values, x["v"].values, x["do"].values, scale, causal, m,
                                 window=_win(win), slopes=None if sl is None else sl.astype(np.float64))
    check("dQ", to_host64(dq), rq, TOL_BF16["dq"])
    check("dK", to_host64(dk), rk, TOL_BF16["dk"])
    check("dV", to_host64(dv), rv, TOL_BF16["dv"])


F32 = [
    (1, 2, 150, 64, False, None, (40, 10), True, None),
    (1, 1, 200, 128, True, None, (70, None), True, None),
    (1, 1, 260, 64, False, "rand_empty_rows", (30, 30), False, None),
]


@pytest.mark.parametrize("case", F32, ids=_id)
def test_variant_f32(case):
    B, H, N, d, causal, mk, win, al, sc = case
    scale = float(np.float32(1 / math.sqrt(d) if sc is None else sc))
    say(f"[variant f32] B={B} H={H} N={N} d={d} causal={causal} mask={mk} window={win} alibi={al}")
    x = W.make_inputs(B, H, N, d, "f32", seed=51, with_do=True)
    m = _mask_for(mk, N, 9)
    sl = _slopes(H, al)
    q, k, v, do = (to_device(x[n], "f32") for n in ("q", "k", "v", "do"))
    kw = dict(window=_win(win), alibi_slopes=_dev(sl))
    o, lse = fa.forward(q, k, v, scale, causal, _dev(m), **kw)
    dq, dk, dv = fa.backward(q, k, v, o, do, lse, scale, causal, _dev(m), **kw)
    torch.cuda.synchronize()
    sl64 = None if sl is None else sl.astype(np.float64)
    rq, rk, rv, ro, rl, _ = oracle.attn_bwd(x["q"].values, x["k"].values, x["v"].values, x["do"].values, scale,
                                            causal, m, return_fwd=True, window=_win(win), slopes=sl64)
    check("O", to_host64(o), ro, TOL_F32["o"])
    check("lse", to_host64(lse), rl, TOL_F32["lse"])
    check("dQ", to_host64(dq), rq, TOL_F32["dq"])
    check("dK", to_host64(dk), rk, TOL_F32["dk"])
    check("dV", to_host64(dv), rv, TOL_F32["dv"])


def test_variant_stages_equal_monolithic():
    """fa_bwd_prep + fa_bwd_main_ex + fa_bwd_dq_ex == fa_bwd_dq_first_ex + fa_bwd_main_ex == fa_bwd_ex,
    bit for bit."""
    B, H, N, d = 1, 2, 300, 128
    scale = float(np.float32(1 / math.sqrt(d)))
    x = W.make_inputs(B, H, N, d, "bf16", seed=61, with_do=True)
    q, k, v, do = (to_device(x[n], "bf16") for n in ("q", "k", "v", "do"))
    kw = dict(window=(90, 12), alibi_slopes=_dev(_slopes(H, True)))
    o, lse = fa.forward(q, k, v, scale, True, None, **kw)
    dq, dk, dv = fa.backward(q, k, v, o, do, lse, scale, True, None, **kw)
    ws = fa.workspace(B, H, N, d, q.device)
    dq2, dk2, dv2 = torch.empty_like(q), torch.empty_like(q), torch.empty_like(q)
    fa.fa_bwd_prep(o, do, lse, ws)
    fa.fa_bwd_main_ex(q, k, v, do, dk2, dv2, scale, True, None, workspace=ws, **kw)
    fa.fa_bwd_dq_ex(q, k, v, do, dq2, scale, True, None, workspace=ws, **kw)
    torch.cuda.synchronize()
    for a, b in ((dq, dq2), (dk, dk2), (dv, dv2)):
        assert torch.equal(a, b)
    # the other order: dQ first (with the preprocessing), then dK and dV
    dq3, dk3, dv3 = torch.empty_like(q), torch.empty_like(q), torch.empty_like(q)
    ws.fill_(7)
    fa.fa_bwd_dq_first_ex(q, k, v, o, do, lse, dq3, scale, True, None, workspace=ws, **kw)
    fa.fa_bwd_main_ex(q, k, v, do, dk3, dv3, scale, True, None, workspace=ws, **kw)
    torch.cuda.synchronize()
    for a, b in ((dq, dq3), (dk, dk3), (dv, dv3)):
        assert torch.equal(a, b)


def test_plain_equals_empty_variant():
    """A variant of {-1, -1, NULL} is the plain computation: identical bits."""
    B, H, N, d = 1, 2, 260, 64
    scale = float(np.float32(1 / math.sqrt(d)))
    x = W.make_inputs(B, H, N, d, "bf16", seed=71)
    q, k, v = (to_device(x[n], "bf16") for n in "qkv")
    o1, l1 = fa.forward(q, k, v, scale, True)
    o2, l2 = torch.empty_like(q), torch.empty_like(l1)
    fa.fa_fwd_ex(q, k, v, o2, l2, scale, True, None, window=(-1, -1))
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


# ----------------------------------------------------------------------------
# full-size window + ALiBi workload (benchmark launch configuration), sampled
# ----------------------------------------------------------------------------

def test_full_size_window_alibi():
    w = W.WORKLOADS["bf16_window_alibi_fwdbwd_b2h16n4096d128"]
    say(f"[full variant] {w.name}")
    x = W.workload_inputs(w, seed=0)
    win, sl = W.workload_variant(w)
    q, k, v, do = (to_device(x[n], "bf16") for n in ("q", "k", "v", "do"))
    kw = dict(window=win, alibi_slopes=_dev(sl))
    o, lse = fa.forward(q, k, v, w.scale, w.causal, **kw)
    dq, dk, dv = fa.backward(q, k, v, o, do, lse, w.scale, w.causal, **kw)
    torch.cuda.synchronize()
    for name, t in (("O", o), ("lse", lse), ("dQ", dq), ("dK", dk), ("dV", dv)):
        assert torch.isfinite(t).all(), name
    rows = W.sample_rows(w.B * w.H, w.N, 512, seed=W.SEED_ROWS)
    # slopes are per head: row (b*H + h, i) takes slope h
    o_ref, l_ref = oracle.attn_fwd_rows(x["q"].values, x["k"].values, x["v"].values, w.scale, rows, w.causal,
                                        None, window=win, slopes=sl.astype(np.float64))
    idx0 = torch.from_numpy(rows[:, 0]).to("cuda:0")
    idx1 = torch.from_numpy(rows[:, 1]).to("cuda:0")
    check("O rows", to_host64(o.reshape(w.B * w.H, w.N, w.d)[idx0, idx1]), o_ref, TOL_BF16["o"])
    check("lse rows", to_host64(lse.reshape(w.B * w.H, w.N)[idx0, idx1]), l_ref, TOL_BF16["lse"])
    for b, h in ((0, 0), (1, 15)):
        s = (slice(b, b + 1), slice(h, h + 1))
        rq, rk, rv = oracle.attn_bwd(x["q"].values[s], x["k"].values[s], x["v"].values[s], x["do"].values[s],
                                     w.scale, w.causal, None, window=win, slopes=sl[h:h + 1].astype(np.float64))
        say(f"  head b={b} h={h} slope={sl[h]:.5f}")
        check("dQ", to_host64(dq[b:b + 1, h:h + 1]), rq, TOL_BF16["dq"])
        check("dK", to_host64(dk[b:b + 1, h:h + 1]), rk, TOL_BF16["dk"])
        check("dV", to_host64(dv[b:b + 1, h:h + 1]), rv, TOL_BF16["dv"])
