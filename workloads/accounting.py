"""Work and traffic accounting for exact attention (FLOPs and algorithmic bytes).

FLOP convention (FlashAttention-2's, restated on "FlashAttention 深度解析"
section 四): the forward does two matrix products of 2*N*N*d each per head,
so 4*B*H*N^2*d; a causal mask halves it; a block mask scales it by the
fraction of blocks kept; a local window counts its admitted (query, key)
pairs exactly, 4*d FLOPs each.  The ALiBi bias and the masking are
elementwise work and are not counted.  The backward does five such products
(S recompute, dV, dP, dK, dQ), i.e. 2.5x the forward.

Algorithmic bytes are the O(N*d) floor: every tensor crosses HBM exactly once.
The N*N score/probability traffic of unfused attention ("FlashAttention原理概览"
section 3.4) is what the method removes and is reported separately by
``naive_score_bytes``.
"""
from __future__ import annotations

from typing import Optional

import numpy as np

from . import Workload, MASK_BLOCK

BF16_BYTES = 2
F32_BYTES = 4


def elem_bytes(dtype: str) -> int:
    return {"bf16": BF16_BYTES, "f32": F32_BYTES}[dtype]


def fwd_flops(B: int, H: int, N: int, d: int, causal: bool = False,
              mask: Optional[np.ndarray] = None) -> float:
    """4*B*H*N^2*d, halved if causal, scaled by the kept-block fraction if masked."""
    dense = 4.0 * B * H * N * N * d
    if mask is None:
        return dense * (0.5 if causal else 1.0)
    return float(dense * _mask_factor(mask, causal))


def _mask_factor(mask: np.ndarray, causal: bool) -> float:
    """Block density; with causal, blocks on the diagonal count half."""
    m = mask.astype(np.float64)
    nb = m.shape[0]
    if not causal:
        return m.sum() / (nb * nb)
    lower = np.tril(m, -1).sum()
    diag = np.trace(m)
    return (lower + 0.5 * diag) / (nb * nb)


def bwd_flops(B: int, H: int, N: int, d: int, causal: bool = False,
              mask: Optional[np.ndarray] = None) -> float:
    return 2.5 * fwd_flops(B, H, N, d, causal, mask)


def window_pairs(N: int, causal: bool, window) -> int:
    """Number of (query, key) pairs a local window admits over an N x N head.

    Query i sees keys max(0, i - wl) .. min(N - 1, i + wr), with i as the
    upper end when causal and a negative bound meaning unbounded.
    """
    wl, wr = window
    i = np.arange(N, dtype=np.int64)
    lo = np.zeros(N, dtype=np.int64) if wl < 0 else np.maximum(0, i - wl)
    hi = np.full(N, N - 1, dtype=np.int64) if wr < 0 else np.minimum(N - 1, i + wr)
    if causal:
        hi = np.minimum(hi, i)
    return int(np.maximum(hi - lo + 1, 0).sum())


def fwd_flops_window(B: int, H: int, N: int, d: int, causal: bool, window) -> float:
    """4*d FLOPs (QK^T and PV) per admitted pair, counted exactly."""
    return 4.0 * B * H * d * window_pairs(N, causal, window)


def allowed_pairs(N: int, causal: bool, mask: Optional[np.ndarray] = None, window=None) -> int:
    """Number of (query, key) pairs of one N x N head that the mask admits,
    counted exactly (diagonal blocks of a causal block mask count their lower
    triangle, ragged tail blocks their true size)."""
    if window is not None:
        return window_pairs(N, causal, window)
    if mask is None:
        return N * (N + 1) // 2 if causal else N * N
    nb = mask.shape[0]
    size = np.full(nb, MASK_BLOCK, dtype=np.int64)
    size[-1] = N - MASK_BLOCK * (nb - 1)
    full = np.outer(size, size)
    if causal:
        tri = size * (size + 1) // 2
        full = np.tril(full, -1) + np.diag(tri)
    return int((full * (mask != 0)).sum())


def oracle_flops(heads: int, N: int, d: int, pairs: int, backward: bool) -> float:
    """Floating-point work the fp64 oracle performs for `heads` heads with
    `pairs` admitted pairs each: it materializes the dense N x N scores
    (2 N^2 d) in the forward and again in the backward, the dense
    dP = dO V^T (2 N^2 d), and skips zero probabilities in P V, dS K, P^T dO
    and dS^T Q (2 d per admitted pair each).  Elementwise work is not counted."""
    f = 2.0 * N * N * d + 2.0 * pairs * d
    if backward:
        f += 4.0 * N * N * d + 6.0 * pairs * d
    return heads * f


def fwd_bytes(B: int, H: int, N: int, d: int, dtype: str, nb_mask: int = 0) -> int:
    """Read q, k, v; write o (each B*H*N*d) and lse (fp32 per row); read the mask."""
    e = elem_bytes(dtype)
    return 4 * B * H * N * d * e + F32_BYTES * B * H * N + nb_mask * nb_mask


def bwd_bytes(B: int, H: int, N: int, d: int, dtype: str, nb_mask: int = 0) -> int:
    """The backward's floor: read q, k, v, o, do and lse; write dq, dk and dv."""
    e = elem_bytes(dtype)
    return 8 * B * H * N * d * e + F32_BYTES * B * H * N + nb_mask * nb_mask


def bwd_workspace_bytes(B: int, H: int, N: int, d: int) -> int:
    """Extra traffic of this implementation's backward beyond the floor: two
    fp32 row vectors (D = rowsum(dO*O) and lse in log2 units), each written once
    by the dQ kernel, which runs first, and read once by the key-outer kernel.
    dQ is accumulated in registers by the query-outer kernel, so there is no
    O(N d) fp32 accumulator and no atomic traffic."""
    return 2 * F32_BYTES * B * H * N * 2


def naive_score_bytes(B: int, H: int, N: int, dtype_bytes: int) -> int:
    """Size of one materialized N x N score matrix over all heads."""
    return B * H * N * N * dtype_bytes


def qkv_bytes_one_head(N: int, d: int, dtype_bytes: int) -> int:
    """Q, K and V of a single head."""
    return 3 * N * d * dtype_bytes


def tile_sram_bytes(Br: int, Bc: int, d: int, dtype_bytes: int) -> int:
    """SRAM for a Q tile, one K/V tile and the S tile: (Br*d + Bc*d + Br*Bc) elements."""
    return (Br * d + Bc * d + Br * Bc) * dtype_bytes


def workload_flops(w: Workload, mask: Optional[np.ndarray] = None) -> dict:
    if w.window is not None:
        if mask is not None:
            raise ValueError("a workload combines a window with no block mask")
        f = fwd_flops_window(w.B, w.H, w.N, w.d, w.causal, w.window)
    else:
        f = fwd_flops(w.B, w.H, w.N, w.d, w.causal, mask)
    out = {"fwd": f}
    if w.backward:
        out["bwd"] = 2.5 * f
    return out


def workload_bytes(w: Workload, mask: Optional[np.ndarray] = None) -> dict:
    nbm = mask.shape[0] if mask is not None else 0
    out = {"fwd": fwd_bytes(w.B, w.H, w.N, w.d, w.dtype, nbm)}
    if w.backward:
        out["bwd"] = bwd_bytes(w.B, w.H, w.N, w.d, w.dtype, nbm)
    return out


def launch_bytes(w: Workload, mask: Optional[np.ndarray] = None) -> dict:
    """Algorithmic bytes of one launch of each entry point of the step.

    fa_fwd reads q, k, v and writes o and lse; fa_bwd_prep reads o, do and lse
    and writes D = rowsum(dO*O) and the scaled lse; fa_bwd_main reads q, k, v,
    do, lse and D and writes dk and dv; fa_bwd_dq reads the same and writes dq;
    fa_bwd_dq_first reads q, k, v, o, do and lse and writes dq, D and the
    scaled lse.  The block mask, when there is one, is read by every launch
    that uses it.
    """
    e = elem_bytes(w.dtype)
    t = w.B * w.H * w.N * w.d * e
    r = w.B * w.H * w.N * F32_BYTES
    m = 0 if mask is None else int(mask.size)
    if getattr(w, "precision", "bf16") == "fp8":
        # fa_fwd_fp8 reads one-byte codes of q, k, v and their block exponents, writes bf16 o and lse
        codes = w.B * w.H * w.N * w.d
        exps = w.B * w.H * (-(-w.N // 64))
        return {"fa_fwd_fp8": 3 * codes + 3 * exps + t + r,
                "fa_fp8_quantize": 3 * (t + codes + exps)}
    out = {"fa_fwd": 4 * t + r + m}
    if w.backward:
        out.update({"fa_bwd_prep": 2 * t + 3 * r,
                    "fa_bwd_main": 6 * t + 2 * r + m,
                    "fa_bwd_dq": 5 * t + 2 * r + m,
                    "fa_bwd_dq_first": 6 * t + 3 * r + m})
    return out


def decode_pairs(Nq: int, lens, causal: bool) -> int:
    """(query, key) pairs of one query head over all sequences."""
    n = 0
    for L in np.asarray(lens, dtype=np.int64):
        for i in range(Nq):
            last = (L - Nq + i) if causal else (L - 1)
            n += int(max(0, min(last, L - 1) + 1))
    return n


def decode_flops(w, lens) -> float:
    """4*d FLOPs per (query, key) pair (QK^T and PV), every query head."""
    return 4.0 * w.d * w.H * decode_pairs(w.Nq, lens, w.causal)


def decode_bytes(w, lens) -> int:
    """Each used K and V row read once, q read, o and lse written, the page
    table and lengths read, for the sequences whose lengths are given."""
    e = elem_bytes(w.dtype)
    lens = np.asarray(lens, dtype=np.int64)
    B = int(lens.size)
    kv = 2 * int(lens.sum()) * w.Hkv * w.d * e
    qo = 2 * B * w.H * w.Nq * w.d * e
    return kv + qo + F32_BYTES * B * w.H * w.Nq + 4 * B * (w.max_pages + 1)
