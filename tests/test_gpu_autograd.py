"""The autograd wrapper ``attention``: its forward and backward are the C ABI's
fa_fwd / fa_bwd (bit for bit the same outputs as the direct calls) and match
the fp64 oracle, for the bf16 and fp32 kernels, with a mask, a window and
ALiBi, and with a non-contiguous incoming gradient."""
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


def _leaf(t):
    return t.detach().clone().requires_grad_(True)


@pytest.mark.parametrize("dtype,causal,masked", [("bf16", True, False), ("bf16", False, True), ("f32", True, False)],
                         ids=["bf16-causal", "bf16-mask", "f32-causal"])
def test_attention_autograd_matches_oracle_and_direct_calls(dtype, causal, masked):
    B, H, N, d = 1, 2, 200, 64
    scale = float(np.float32(1 / math.sqrt(d)))
    say(f"[autograd] dtype={dtype} B={B} H={H} N={N} d={d} causal={causal} mask={masked}")
    x = W.make_inputs(B, H, N, d, dtype, seed=31, with_do=True)
    m = W.random_blockmask((N + 127) // 128, 7, p=0.6, keep_diag=True) if masked else None
    dm = None if m is None else torch.from_numpy(np.ascontiguousarray(m)).to("cuda:0")
    q, k, v, do = (to_device(x[n], dtype) for n in ("q", "k", "v", "do"))
    ql, kl, vl = _leaf(q), _leaf(k), _leaf(v)
    o, lse = fa.attention(ql, kl, vl, causal=causal, blockmask=dm, return_lse=True)
    o.backward(do)
    o2, lse2 = fa.forward(q, k, v, scale, causal, dm)
    dq2, dk2, dv2 = fa.backward(q, k, v, o2, do, lse2, scale, causal, dm)
    torch.cuda.synchronize()
    for name, a, b in (("O", o.detach(), o2), ("lse", lse, lse2), ("dQ", ql.grad, dq2), ("dK", kl.grad, dk2),
                       ("dV", vl.grad, dv2)):
        assert torch.equal(a, b), f"{name} differs from the direct call"
    rq, rk, rv, ro, rl, _ = oracle.attn_bwd(x["q"].values, x["k"].values, x["v"].values, x["do"].values, scale,
                                            causal, m, return_fwd=True)
    tol = TOL_BF16 if dtype == "bf16" else TOL_F32
    if dtype == "bf16":
        check_bf16_out("O", to_host64(o), ro, tol["o"])
    else:
        check("O", to_host64(o), ro, tol["o"])
    check("lse", to_host64(lse), rl, tol["lse"])
    check("dQ", to_host64(ql.grad), rq, tol["dq"])
    check("dK", to_host64(kl.grad), rk, tol["dk"])
    check("dV", to_host64(vl.grad), rv, tol["dv"])


def test_attention_autograd_window_alibi_noncontiguous_grad():
    """fp32 kernels with a local window and ALiBi; loss = sum(O) hands the
    backward an expanded (stride-0) gradient of ones."""
    B, H, N, d = 1, 2, 150, 64
    scale = 0.125
    window = (40, 0)
    slopes = np.array([0.25, 0.0625], dtype=np.float32)
    say(f"[autograd window+alibi] B={B} H={H} N={N} d={d} window={window}")
    x = W.make_inputs(B, H, N, d, "f32", seed=33)
    q, k, v = (to_device(x[n], "f32") for n in "qkv")
    sl = torch.from_numpy(slopes).to("cuda:0")
    ql, kl, vl = _leaf(q), _leaf(k), _leaf(v)
    o = fa.attention(ql, kl, vl, scale=scale, causal=True, window=window, alibi_slopes=sl)
    o.sum().backward()
    torch.cuda.synchronize()
    ones = np.ones((B, H, N, d), dtype=np.float64)
    rq, rk, rv, ro, _, _ = oracle.attn_bwd(x["q"].values, x["k"].values, x["v"].values, ones, scale, True, None,
                                           return_fwd=True, window=window, slopes=slopes.astype(np.float64))
    check("O", to_host64(o), ro, TOL_F32["o"])
    check("dQ", to_host64(ql.grad), rq, TOL_F32["dq"])
    check("dK", to_host64(kl.grad), rk, TOL_F32["dk"])
    check("dV", to_host64(vl.grad), rv, TOL_F32["dv"])
