"""Seeded synthetic workloads for exact attention.

This module only *generates inputs*: shapes, iid N(0,1) draws, the bf16
encoding of those draws, the 128x128 block mask and the sampled-row list.
It holds none of the attention arithmetic, so both the oracle side and the
HIP side can consume the very same bytes without sharing any computation.

The workloads follow the shapes the pages discuss (FlashAttention v1/v2 for
exact tiled attention): the case study of "FlashAttention原理概览" section 3.4
(one layer, 8 heads, sequence 8192, head dim 128), the 64K long-sequence
block-sparse setting of "FlashAttention: ... IO-Awareness" section 4, and a
plain training-sized forward.  Every draw is seeded; the generator is numpy's
PCG64 ``default_rng``.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field, asdict
from typing import Dict, Optional, Tuple

import numpy as np

MASK_BLOCK = 128  # block-mask granularity (rows and columns), see Workload.mask


@dataclass(frozen=True)
class Workload:
    name: str
    B: int
    H: int
    N: int
    d: int
    dtype: str              # "bf16" or "f32": element type of q, k, v, do, o
    causal: bool = False
    mask: Optional[str] = None   # None (dense) or "band2_random" (block-sparse)
    density: float = 1.0         # target block density when mask is set
    backward: bool = False       # the workload also runs the recompute backward
    window: Optional[Tuple[int, int]] = None  # local window (left, right); negative = unbounded
    alibi: bool = False          # add the per-head ALiBi bias with alibi_slopes(H)
    precision: str = "bf16"      # "fp8": the inputs are block-quantized to E4M3 for the FP8 forward
    description: str = ""

    @property
    def scale(self) -> float:
        """Softmax scale 1/sqrt(d), rounded to fp32 as both sides see it."""
        return float(np.float32(1.0 / math.sqrt(self.d)))

    @property
    def nb(self) -> int:
        return (self.N + MASK_BLOCK - 1) // MASK_BLOCK

    @property
    def variant(self) -> bool:
        return self.window is not None or self.alibi

    def to_dict(self) -> dict:
        return asdict(self)


WORKLOADS: Dict[str, Workload] = {
    w.name: w
    for w in [
        Workload("tiny_f32_fwd", 1, 1, 128, 64, "f32",
                 description="tiny exact attention forward, fp32"),
        Workload("bf16_fwd_b4h16n2048d64", 4, 16, 2048, 64, "bf16",
                 description="bf16 forward, non-causal"),
        Workload("bf16_causal_fwd_b1h8n8192d128", 1, 8, 8192, 128, "bf16", causal=True,
                 description="bf16 causal forward at long context (case-study shape)"),
        Workload("bf16_causal_fwdbwd_b2h16n4096d128", 2, 16, 4096, 128, "bf16", causal=True,
                 backward=True,
                 description="bf16 causal forward + recompute backward"),
        Workload("bf16_blocksparse_fwd_b1h8n65536d64", 1, 8, 65536, 64, "bf16",
                 mask="band2_random", density=1.0 / 8,
                 description="bf16 block-sparse forward at 64K, 128x128 blocks, density 1/8"),
        Workload("fp8_causal_fwd_b2h16n4096d128", 2, 16, 4096, 128, "bf16", causal=True, precision="fp8",
                 description="FP8 causal forward (E4M3, 64-row block scales, incoherent map on Q and K) "
                             "of the benchmarked step's shape"),
        Workload("bf16_window_alibi_fwdbwd_b2h16n4096d128", 2, 16, 4096, 128, "bf16", causal=True,
                 backward=True, window=(1023, -1), alibi=True,
                 description="bf16 causal sliding window of 1024 keys with ALiBi, forward + backward"),
        Workload("bf16_causal_fwd_b1h8n8192d256", 1, 8, 8192, 256, "bf16", causal=True,
                 description="bf16 causal forward at the largest head size the pages name (256), "
                             "case-study sequence length"),
        Workload("bf16_causal_fwdbwd_b2h16n4096d96", 2, 16, 4096, 96, "bf16", causal=True, backward=True,
                 description="bf16 causal forward + backward at a head size that is a multiple of 16 "
                             "but not of the tile width (rows padded to 128 in the tiles)"),
    ]
}

# Seed offsets per tensor (base seed s): q=s, k=s+1, v=s+2, do=s+3, mask=s+4, rows=s+5,
# page table=s+6, sequence lengths=s+7, incoherent-map signs=s+8.
SEED_Q, SEED_K, SEED_V, SEED_DO, SEED_MASK, SEED_ROWS, SEED_PAGES, SEED_LENS, SEED_SIGNS = range(9)


def fp8_signs(d: int, seed: int = 0) -> np.ndarray:
    """The random sign vector of the incoherent map (float32 +-1, length d)."""
    return np.random.default_rng(seed + SEED_SIGNS).choice([-1.0, 1.0], size=d).astype(np.float32)


@dataclass(frozen=True)
class DecodeWorkload:
    """Decode over a paged KV cache: Nq new queries per sequence, B sequences
    whose lengths are drawn uniformly from [min_len, max_len], H query heads
    grouped onto Hkv KV heads, pages of page_size positions."""
    name: str
    B: int
    H: int
    Hkv: int
    Nq: int
    d: int
    page_size: int
    min_len: int
    max_len: int
    causal: bool = True
    dtype: str = "bf16"
    description: str = ""
    kind: str = "decode"

    @property
    def scale(self) -> float:
        return float(np.float32(1.0 / math.sqrt(self.d)))

    @property
    def max_pages(self) -> int:
        return -(-self.max_len // self.page_size)

    @property
    def num_pages(self) -> int:
        return self.B * self.max_pages

    def to_dict(self) -> dict:
        return asdict(self)


WORKLOADS["bf16_paged_decode_b16h32kv8d128_len1k_8k"] = DecodeWorkload(
    "bf16_paged_decode_b16h32kv8d128_len1k_8k", B=16, H=32, Hkv=8, Nq=1, d=128, page_size=256,
    min_len=1024, max_len=8192,
    description="bf16 decode, one new token per sequence, 16 sequences of 1K-8K cached tokens in 256-token pages, "
                "32 query heads on 8 KV heads")


# ----------------------------------------------------------------------------
# Encodings
# ----------------------------------------------------------------------------

def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (round to nearest, ties to even).

    Returns the 16-bit patterns as uint16.  Inputs here are finite normal
    draws; NaN/Inf are not produced by the generators and are not handled.
    """
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    r = (u + np.uint32(0x7FFF) + lsb) >> np.uint32(16)
    return r.astype(np.uint16)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """Exact widening of bfloat16 bit patterns to float32."""
    return (np.ascontiguousarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


# ----------------------------------------------------------------------------
# Tensors
# ----------------------------------------------------------------------------

def normal(shape, seed: int) -> np.ndarray:
    """iid N(0,1) float32 draws from numpy's PCG64 generator."""
    return np.random.default_rng(seed).standard_normal(shape, dtype=np.float32)


@dataclass
class Tensor:
    """One input tensor: exact values as float32 plus the stored bits.

    ``values`` holds exactly the numbers the kernels read (bf16-representable
    for bf16 workloads), ``bits`` the storage (uint16 for bf16, float32 for
    f32).  The oracle widens ``values`` to float64.
    """
    values: np.ndarray
    bits: np.ndarray
    dtype: str


def make_tensor(shape, seed: int, dtype: str) -> Tensor:
    x = normal(shape, seed)
    if dtype == "bf16":
        bits = f32_to_bf16_bits(x)
        return Tensor(bf16_bits_to_f32(bits), bits, dtype)
    if dtype == "f32":
        return Tensor(x, x, dtype)
    raise ValueError(f"unknown dtype {dtype}")


def make_inputs(B: int, H: int, N: int, d: int, dtype: str, seed: int = 0,
                with_do: bool = False) -> Dict[str, Tensor]:
    """q, k, v (and do) of shape [B, H, N, d], iid N(0,1), encoded as dtype."""
    shape = (B, H, N, d)
    out = {
        "q": make_tensor(shape, seed + SEED_Q, dtype),
        "k": make_tensor(shape, seed + SEED_K, dtype),
        "v": make_tensor(shape, seed + SEED_V, dtype),
    }
    if with_do:
        out["do"] = make_tensor(shape, seed + SEED_DO, dtype)
    return out


def workload_inputs(w: Workload, seed: int = 0) -> Dict[str, Tensor]:
    return make_inputs(w.B, w.H, w.N, w.d, w.dtype, seed, with_do=w.backward)


# ----------------------------------------------------------------------------
# ALiBi slopes
# ----------------------------------------------------------------------------

def alibi_slopes(H: int) -> np.ndarray:
    """The geometric ALiBi slopes 2^(-8 (h+1) / H), h = 0..H-1, as float32.

    They are inputs of the variant (one per head), passed unchanged to both
    sides; for H a power of two this is the usual per-head sequence.
    """
    return np.array([2.0 ** (-8.0 * (h + 1) / H) for h in range(H)], dtype=np.float32)


def workload_variant(w: Workload):
    """(window, slopes) of a workload: None for each part it does not use."""
    return w.window, (alibi_slopes(w.H) if w.alibi else None)


# ----------------------------------------------------------------------------
# Block mask
# ----------------------------------------------------------------------------

def make_blockmask(nb: int, seed: int, band: int = 2, density: float = 1.0 / 8) -> np.ndarray:
    """Block mask of shape [nb, nb] (uint8, 1 = block attended).

    Each block row keeps the band |row - col| <= ``band`` (the diagonal and
    its neighbours, clipped at the edges) and then gains distinct off-band
    columns drawn uniformly without replacement until it holds
    ``max(band blocks, round(nb * density))`` blocks.  One mask is shared by
    every batch entry and head.
    """
    rng = np.random.default_rng(seed)
    target = int(round(nb * density))
    m = np.zeros((nb, nb), dtype=np.uint8)
    cols = np.arange(nb)
    for r in range(nb):
        in_band = np.abs(cols - r) <= band
        m[r, in_band] = 1
        need = target - int(in_band.sum())
        if need > 0:
            off = cols[~in_band]
            pick = rng.choice(off, size=min(need, off.size), replace=False)
            m[r, pick] = 1
    return m


def workload_mask(w: Workload, seed: int = 0) -> Optional[np.ndarray]:
    if w.mask is None:
        return None
    if w.mask == "band2_random":
        return make_blockmask(w.nb, seed + SEED_MASK, band=2, density=w.density)
    raise ValueError(f"unknown mask kind {w.mask}")


def random_blockmask(nb: int, seed: int, p: float = 0.5, keep_diag: bool = False) -> np.ndarray:
    """Bernoulli(p) block mask (for edge-case tests: may leave rows empty)."""
    m = (np.random.default_rng(seed).random((nb, nb)) < p).astype(np.uint8)
    if keep_diag:
        np.fill_diagonal(m, 1)
    return m


# ----------------------------------------------------------------------------
# Sampled rows (for full-size parity where the oracle runs row by row)
# ----------------------------------------------------------------------------

def sample_rows(BH: int, N: int, nrows: int, seed: int) -> np.ndarray:
    """``nrows`` distinct (bh, i) pairs, shape [nrows, 2] (int64).

    Rows 0, 127, 128, N/2-1, N/2 and N-1 of head 0 (tile and block
    boundaries) are always included; the rest are drawn uniformly without
    replacement over all BH*N rows.
    """
    forced = []
    for i in (0, MASK_BLOCK - 1, MASK_BLOCK, N // 2 - 1, N // 2, N - 1):
        if 0 <= i < N and (0, i) not in forced:
            forced.append((0, i))
    forced = forced[:nrows]
    total = BH * N
    nrand = min(nrows, total) - len(forced)
    rng = np.random.default_rng(seed)
    forced_flat = {bh * N + i for bh, i in forced}
    picked = []
    while len(picked) < nrand:
        cand = rng.choice(total, size=nrand - len(picked), replace=False)
        for c in cand:
            c = int(c)
            if c not in forced_flat and c not in picked:
                picked.append(c)
                if len(picked) == nrand:
                    break
    flat = [bh * N + i for bh, i in forced] + picked
    flat = np.array(sorted(flat), dtype=np.int64)
    return np.stack([flat // N, flat % N], axis=1)


# ----------------------------------------------------------------------------
# Paged KV cache (decode)
# ----------------------------------------------------------------------------

def make_paged(B: int, H: int, Hkv: int, Nq: int, d: int, page_size: int, max_pages: int, lens, seed: int,
               dtype: str = "bf16", num_pages: Optional[int] = None) -> Dict[str, object]:
    """q [B,H,Nq,d], k_cache / v_cache [num_pages, page_size, Hkv, d] (iid N(0,1)
    encoded as dtype), block_table [B, max_pages] int32 and seqlens [B] int32.

    Every sequence owns max_pages distinct physical pages in a seeded random
    order (a shuffled allocator); cache rows past a sequence's length hold
    draws too, which the computation must ignore.
    """
    num_pages = B * max_pages if num_pages is None else num_pages
    if num_pages < B * max_pages:
        raise ValueError("num_pages must cover every sequence's pages")
    perm = np.random.default_rng(seed + SEED_PAGES).permutation(num_pages)[:B * max_pages]
    return {
        "q": make_tensor((B, H, Nq, d), seed + SEED_Q, dtype),
        "k_cache": make_tensor((num_pages, page_size, Hkv, d), seed + SEED_K, dtype),
        "v_cache": make_tensor((num_pages, page_size, Hkv, d), seed + SEED_V, dtype),
        "block_table": perm.reshape(B, max_pages).astype(np.int32),
        "seqlens": np.asarray(lens, dtype=np.int32),
    }


def decode_inputs(w: DecodeWorkload, seed: int = 0) -> Dict[str, object]:
    lens = np.random.default_rng(seed + SEED_LENS).integers(w.min_len, w.max_len + 1, size=w.B)
    return make_paged(w.B, w.H, w.Hkv, w.Nq, w.d, w.page_size, w.max_pages, lens, seed, w.dtype)
