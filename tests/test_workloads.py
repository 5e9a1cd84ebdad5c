"""Seeded input generators and work/byte accounting (CPU only)."""
import json
import os

import numpy as np

import workloads as W
from workloads import accounting as A

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "pages_byte_counts.json")


def test_pages_byte_counts():
    g = json.load(open(GOLDEN))
    a = g["naive_score_matrix_bytes"]["args"]
    assert A.naive_score_bytes(a["B"], a["H"], a["N"], a["dtype_bytes"]) == g["naive_score_matrix_bytes"]["value"]
    a = g["qkv_one_head_bytes"]["args"]
    assert A.qkv_bytes_one_head(a["N"], a["d"], a["dtype_bytes"]) == g["qkv_one_head_bytes"]["value"]
    a = g["o_one_head_bytes"]["args"]
    # one head's O is a third of its Q/K/V reads
    assert A.qkv_bytes_one_head(a["N"], a["d"], a["dtype_bytes"]) // 3 == g["o_one_head_bytes"]["value"]
    a = g["tile_sram_bytes"]["args"]
    assert A.tile_sram_bytes(a["Br"], a["Bc"], a["d"], a["dtype_bytes"]) == g["tile_sram_bytes"]["value"]
    a = g["naive_passes_over_S_bytes"]["args"]
    assert a["passes"] * A.naive_score_bytes(a["B"], a["H"], a["N"], a["dtype_bytes"]) == \
        g["naive_passes_over_S_bytes"]["value"]


def test_flop_convention():
    # 4*B*H*N^2*d; causal halves; block mask scales by kept fraction
    assert A.fwd_flops(1, 8, 8192, 128, causal=True) == 137438953472.0
    assert A.fwd_flops(4, 16, 2048, 64) == 68719476736.0
    assert A.bwd_flops(2, 16, 4096, 128, causal=True) == 2.5 * A.fwd_flops(2, 16, 4096, 128, True)
    m = np.zeros((4, 4), np.uint8)
    m[0, 0] = m[1, 1] = 1
    assert A.fwd_flops(1, 1, 512, 64, mask=m) == 4.0 * 512 * 512 * 64 * 2 / 16
    # with causal, diagonal blocks count half; strictly-upper blocks not at all
    m[0, 3] = 1
    assert A.fwd_flops(1, 1, 512, 64, causal=True, mask=m) == 4.0 * 512 * 512 * 64 * 1 / 16


def test_bf16_rounding_rne():
    x = np.array([1.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, 1.0 + 2 ** -9, -2.5, 3.140625,
                  1.0 + 2 ** -8 + 2 ** -20], dtype=np.float32)
    b = W.bf16_bits_to_f32(W.f32_to_bf16_bits(x))
    # ties to even: 1+2^-8 is halfway between 1 and 1+2^-7 -> 1; 1+3*2^-8 -> 1+2^-6
    assert b.tolist() == [1.0, 1.0, 1.0 + 2 ** -6, 1.0, -2.5, 3.140625, 1.0 + 2 ** -7]


def test_inputs_seeded_and_exact():
    a = W.make_inputs(1, 2, 64, 16, "bf16", seed=3, with_do=True)
    b = W.make_inputs(1, 2, 64, 16, "bf16", seed=3, with_do=True)
    for key in "q", "k", "v", "do":
        assert np.array_equal(a[key].bits, b[key].bits)
        # values are exactly the bf16 numbers the bits encode
        assert np.array_equal(W.f32_to_bf16_bits(a[key].values), a[key].bits)
    assert not np.array_equal(a["q"].bits, a["k"].bits)
    f = W.make_inputs(1, 1, 8, 4, "f32", seed=1)
    assert f["q"].values.dtype == np.float32


def test_blockmask_recipe():
    nb = 512
    m = W.make_blockmask(nb, seed=4, band=2, density=1 / 8)
    assert m.shape == (nb, nb) and m.dtype == np.uint8
    rows = m.sum(axis=1)
    assert np.all(rows == nb // 8)
    assert m.sum() * 8 == nb * nb
    for r in range(nb):
        for c in range(max(0, r - 2), min(nb, r + 3)):
            assert m[r, c] == 1
    assert np.array_equal(m, W.make_blockmask(nb, seed=4))
    assert not np.array_equal(m, W.make_blockmask(nb, seed=5))


def test_sample_rows():
    r = W.sample_rows(8, 65536, 512, seed=5)
    assert r.shape == (512, 2)
    flat = r[:, 0] * 65536 + r[:, 1]
    assert len(set(flat.tolist())) == 512
    for i in (0, 127, 128, 32767, 32768, 65535):
        assert (0 * 65536 + i) in set(flat.tolist())
    assert np.array_equal(r, W.sample_rows(8, 65536, 512, seed=5))


def test_workload_table():
    w = W.WORKLOADS["bf16_causal_fwd_b1h8n8192d128"]
    assert (w.B, w.H, w.N, w.d, w.causal) == (1, 8, 8192, 128, True)
    assert w.scale == float(np.float32(1 / np.sqrt(128)))
    assert A.workload_bytes(w)["fwd"] == 67371008
    w = W.WORKLOADS["bf16_blocksparse_fwd_b1h8n65536d64"]
    m = W.workload_mask(w)
    assert A.workload_flops(w, m)["fwd"] == 4.0 * 8 * 65536 ** 2 * 64 / 8


def test_window_pairs_brute_force():
    # count admitted pairs one by one against the closed-form per-row count
    rng = np.random.default_rng(7)
    for _ in range(40):
        N = int(rng.integers(1, 70))
        wl, wr = (int(rng.integers(-1, N + 2)) for _ in range(2))
        causal = bool(rng.integers(0, 2))
        n = 0
        for i in range(N):
            for j in range(N):
                ok = (wl < 0 or j >= i - wl) and (wr < 0 or j <= i + wr) and (not causal or j <= i)
                n += ok
        assert A.window_pairs(N, causal, (wl, wr)) == n, (N, wl, wr, causal)
    # an unbounded window is the dense or causal count
    assert A.window_pairs(100, False, (-1, -1)) == 100 * 100
    assert A.window_pairs(100, True, (-1, -1)) == 100 * 101 // 2
    # a 1024-key causal window at N=4096: rows 0..1023 see i + 1 keys, the rest 1024
    assert A.window_pairs(4096, True, (1023, -1)) == 1024 * 1025 // 2 + (4096 - 1024) * 1024


def test_window_workload():
    w = W.WORKLOADS["bf16_window_alibi_fwdbwd_b2h16n4096d128"]
    assert w.variant and w.causal and w.backward and w.window == (1023, -1)
    win, sl = W.workload_variant(w)
    assert win == (1023, -1)
    # slopes: 2^(-8(h+1)/H), a geometric sequence ending at 2^-8
    assert sl.dtype == np.float32 and sl.shape == (16,)
    assert sl[1] == np.float32(0.5) and sl[-1] == np.float32(2.0 ** -8)
    assert np.allclose(sl[1:] / sl[:-1], 2.0 ** -0.5, rtol=1e-6)
    f = A.workload_flops(w)
    assert f["fwd"] == 4.0 * 2 * 16 * 128 * A.window_pairs(4096, True, (1023, -1))
    assert f["bwd"] == 2.5 * f["fwd"]
    assert W.workload_variant(W.WORKLOADS["bf16_causal_fwd_b1h8n8192d128"]) == (None, None)


def test_decode_workload_and_accounting():
    w = W.WORKLOADS["bf16_paged_decode_b16h32kv8d128_len1k_8k"]
    x = W.decode_inputs(w)
    lens = x["seqlens"]
    assert lens.dtype == np.int32 and lens.shape == (16,) and lens.min() >= 1024 and lens.max() <= 8192
    bt = x["block_table"]
    assert bt.shape == (16, 32) and len(set(bt.ravel().tolist())) == bt.size  # distinct physical pages
    assert x["k_cache"].bits.shape == (16 * 32, 256, 8, 128)
    # pairs: one query at the end of each sequence sees every key
    assert A.decode_pairs(1, lens, True) == int(lens.sum())
    assert A.decode_pairs(3, [5], True) == 3 + 4 + 5 and A.decode_pairs(3, [1], True) == 1
    assert A.decode_flops(w, lens) == 4.0 * 128 * 32 * int(lens.sum())
    assert A.decode_bytes(w, lens) == (2 * int(lens.sum()) * 8 * 128 * 2 + 2 * 16 * 32 * 128 * 2 + 4 * 16 * 32
                                       + 4 * 16 * 33)
