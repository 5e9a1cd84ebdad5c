"""Parity of decode over a paged KV cache (fa_decode_paged) with the fp64 oracle.

Every output element is compared: grouped heads (1, 4, 8 and 40 query heads
per KV head, the last needing two 32-row query groups), one and several new
queries with causal alignment to the end of the sequence, lengths that end
inside a page, a length shorter than the query count and an empty sequence,
several page sizes and head dimensions, pages in shuffled order with cache
rows past every length holding data that must be ignored, key ranges split
over many waves (merged exactly) and a single range written directly,
negative and zero scales, and the full-size decode workload of the benchmark.
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


def _ids(c):
    B, H, Hkv, Nq, d, ps, mp, lens, causal, sc = c
    return f"B{B}H{H}kv{Hkv}q{Nq}d{d}p{ps}x{mp}{'c' if causal else ''}" + ("" if sc is None else f"-s{sc}")


CASES = [
    # B, H, Hkv, Nq, d, page_size, max_pages, lengths, causal, scale (None = 1/sqrt(d))
    (3, 8, 2, 1, 128, 64, 40, [1, 700, 2049], True, None),
    (2, 16, 4, 4, 64, 32, 20, [640, 77], True, None),
    (3, 4, 4, 3, 128, 32, 8, [2, 0, 256], True, None),
    (1, 40, 1, 1, 64, 64, 16, [1000], True, None),
    (2, 8, 1, 2, 128, 128, 12, [1536, 999], False, None),
    (64, 64, 64, 1, 64, 32, 4, list(range(1, 128, 2)), True, None),
    (2, 4, 2, 5, 128, 64, 10, [600, 333], True, -0.07),
    (1, 2, 2, 1, 64, 32, 4, [100], True, 0.0),
]


def _run(B, H, Hkv, Nq, d, ps, mp, lens, causal, scale, seed):
    x = W.make_paged(B, H, Hkv, Nq, d, ps, mp, lens, seed)
    q, kc, vc = (to_device(x[n], "bf16") for n in ("q", "k_cache", "v_cache"))
    bt = torch.from_numpy(x["block_table"]).to("cuda:0")
    sl = torch.from_numpy(x["seqlens"]).to("cuda:0")
    o, lse = fa.decode_paged(q, kc, vc, bt, sl, scale, causal)
    torch.cuda.synchronize()
    o_ref, l_ref = oracle.attn_paged_fwd(x["q"].values, x["k_cache"].values, x["v_cache"].values,
                                         x["block_table"], x["seqlens"], scale, causal)
    return o, lse, o_ref, l_ref


@pytest.mark.parametrize("case", CASES, ids=_ids)
def test_decode_paged(case):
    B, H, Hkv, Nq, d, ps, mp, lens, causal, sc = case
    scale = float(np.float32(1 / math.sqrt(d) if sc is None else sc))
    ws = fa.fa_decode_workspace_size(B, H, Hkv, Nq, d, ps, mp)
    say(f"[decode] B={B} H={H} Hkv={Hkv} Nq={Nq} d={d} page={ps} max_pages={mp} lens={lens[:6]} "
        f"causal={causal} scale={scale} workspace={ws}")
    o, lse, o_ref, l_ref = _run(B, H, Hkv, Nq, d, ps, mp, lens, causal, scale, seed=81)
    check("O", to_host64(o), o_ref, TOL_BF16["o"])
    check("lse", to_host64(lse), l_ref, TOL_BF16["lse"])


def test_decode_empty_rows_exact():
    """A query with no key gets O = 0 exactly and lse = -inf."""
    o, lse, o_ref, l_ref = _run(3, 4, 2, 3, 64, 32, 4, [0, 1, 2], True, 0.125, seed=82)
    on, ln = to_host64(o), to_host64(lse)
    empty = ~np.isfinite(l_ref)
    assert empty.sum() == 3 * 4 + 2 * 4 + 1 * 4  # per head: sequence 0 all three, 1 two, 2 one
    assert np.all(on[empty] == 0.0) and np.all(np.isneginf(ln[empty]))


def test_decode_deterministic():
    args = (2, 16, 4, 2, 128, 64, 24, [1500, 700], True, 0.09)
    o1, l1, _, _ = _run(*args, seed=83)
    o2, l2, _, _ = _run(*args, seed=83)
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_decode_bad_page_index_reads_zeros():
    """A page-table entry outside the cache reads as zeros: no fault, the other
    sequences are unaffected and every output is finite."""
    B, H, Hkv, Nq, d, ps, mp = 2, 4, 2, 1, 64, 32, 6
    x = W.make_paged(B, H, Hkv, Nq, d, ps, mp, [150, 120], 84)
    bad = x["block_table"].copy()
    bad[1, 2] = 10 ** 6
    bad[1, 3] = -5
    q, kc, vc = (to_device(x[n], "bf16") for n in ("q", "k_cache", "v_cache"))
    o, lse = fa.decode_paged(q, kc, vc, torch.from_numpy(bad).to("cuda:0"),
                             torch.from_numpy(x["seqlens"]).to("cuda:0"), 0.125, True)
    torch.cuda.synchronize()
    assert torch.isfinite(o).all() and torch.isfinite(lse).all()
    o_ref, l_ref = oracle.attn_paged_fwd(x["q"].values, x["k_cache"].values, x["v_cache"].values,
                                         x["block_table"], x["seqlens"], 0.125, True)
    check("O (intact sequence)", to_host64(o[:1]), o_ref[:1], TOL_BF16["o"])


def test_full_size_decode_workload():
    w = W.WORKLOADS["bf16_paged_decode_b16h32kv8d128_len1k_8k"]
    say(f"[full decode] {w.name}")
    x = W.decode_inputs(w, seed=0)
    q, kc, vc = (to_device(x[n], "bf16") for n in ("q", "k_cache", "v_cache"))
    bt = torch.from_numpy(x["block_table"]).to("cuda:0")
    sl = torch.from_numpy(x["seqlens"]).to("cuda:0")
    o, lse = fa.decode_paged(q, kc, vc, bt, sl, w.scale, w.causal)
    torch.cuda.synchronize()
    o_ref, l_ref = oracle.attn_paged_fwd(x["q"].values, x["k_cache"].values, x["v_cache"].values,
                                         x["block_table"], x["seqlens"], w.scale, w.causal)
    check("O", to_host64(o), o_ref, TOL_BF16["o"])
    check("lse", to_host64(lse), l_ref, TOL_BF16["lse"])
