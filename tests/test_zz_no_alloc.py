"""fa_bwd_noalloc (the backward without a workspace argument, for callers that
cannot allocate) against fa_bwd_ex through the C ABI: identical bits on two
calls in a row, the second with a smaller input (the static scratch keeps
the first call's contents, which the second must not depend on), and the
oracle's bar on the first."""
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

CASES = [
    # B, H, N, d, causal, window, alibi, seed: the second call is smaller
    (2, 4, 1000, 128, True, None, False, 301),
    (1, 2, 300, 64, False, (60, 20), True, 302),
]


def _run(B, H, N, d, causal, window, alibi, seed):
    scale = float(np.float32(1 / math.sqrt(d)))
    x = W.make_inputs(B, H, N, d, "bf16", seed=seed, with_do=True)
    q, k, v, do = (to_device(x[n], "bf16") for n in ("q", "k", "v", "do"))
    sl = None
    if alibi:
        sl = torch.from_numpy(np.array([2.0 ** (-8.0 * (h + 1) / H) for h in range(H)], dtype=np.float32)).to(q.device)
    kw = dict(window=window, alibi_slopes=sl)
    o, lse = fa.forward(q, k, v, scale, causal, **kw)
    want = fa.backward(q, k, v, o, do, lse, scale, causal, **kw)
    got = tuple(torch.full_like(q, float("nan")) for _ in range(3))
    fa.fa_bwd_noalloc(q, k, v, o, do, lse, *got, scale, causal, None, window=window, alibi_slopes=sl)
    torch.cuda.synchronize()
    return x, scale, want, got, sl


def test_noalloc_matches_fa_bwd_twice():
    first = None
    for i, case in enumerate(CASES):
        B, H, N, d, causal, window, alibi, seed = case
        say(f"[noalloc call {i + 1}] B={B} H={H} N={N} d={d} causal={causal} window={window} alibi={alibi}")
        x, scale, want, got, sl = _run(*case)
        for name, a, b in zip(("dQ", "dK", "dV"), got, want):
            assert torch.equal(a, b), f"call {i + 1}: {name} of fa_bwd_noalloc differs from fa_bwd_ex"
        if first is None:
            first = (x, scale, got, causal, window)
    x, scale, got, causal, window = first
    rq, rk, rv = oracle.attn_bwd(x["q"].values, x["k"].values, x["v"].values, x["do"].values, scale, causal, None,
                                 window=window)
    check("dQ", to_host64(got[0]), rq, TOL_BF16["dq"])
    check("dK", to_host64(got[1]), rk, TOL_BF16["dk"])
    check("dV", to_host64(got[2]), rv, TOL_BF16["dv"])


def test_noalloc_rejects_oversize_before_launch():
    q = torch.zeros((1, 1, fa.NOALLOC_MAX_ROWS + 128, 64), dtype=torch.bfloat16, device="cuda:0")
    lse = torch.zeros((1, 1, q.shape[2]), dtype=torch.float32, device="cuda:0")
    with pytest.raises(fa.FAError) as e:
        fa.fa_bwd_noalloc(q, q, q, q, q, lse, torch.empty_like(q), torch.empty_like(q), torch.empty_like(q), 0.125)
    assert e.value.status == 5
