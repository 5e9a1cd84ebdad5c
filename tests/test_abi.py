"""The C ABI library loads, exports what include/fa.h declares, and validates
arguments before touching the GPU (CPU only: no compute call is made)."""
import ctypes
import os
import re

import pytest

import exact_io_aware_59_amd as fa

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fa.h")

# fake, never dereferenced device addresses (validation returns before any HIP call)
P1, P2, P3, P4, P5, P6, P7, P8, P9 = (0x10000 * (i + 1) for i in range(9))
BIG = 1 << 40  # spacing so that fake tensors do not overlap


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"^\s*(?:const\s+)?[A-Za-z_][A-Za-z0-9_]*\s*\**\s*(fa_[a-z0-9_]+)\s*\(", text, flags=re.M)
    return sorted(set(names))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(fa.library_path()):
        from exact_io_aware_59_amd import build
        build.build()
    return fa.load()


def test_exports_every_declared_symbol(lib):
    names = declared_functions()
    assert set(names) >= {"fa_fwd", "fa_fwd_f32", "fa_bwd", "fa_bwd_f32", "fa_bwd_workspace_size",
                          "fa_status_string", "fa_version", "fa_decode_paged", "fa_decode_workspace_size",
                          "fa_fp8_quantize", "fa_fwd_fp8"}
    for n in names:
        assert hasattr(lib, n), n


def test_version_and_status(lib):
    assert fa.fa_version() == fa.ABI_VERSION == 7
    for s in range(6):
        assert fa.fa_status_string(s)
    assert fa.fa_status_string(99) == "unknown status"


def test_workspace_size(lib):
    ws = fa.fa_bwd_workspace_size(2, 16, 4096, 128)
    rows = 2 * 16 * 4096
    assert ws == 2 * rows * 4  # both row vectors already 256-byte multiples
    assert fa.fa_bwd_workspace_size(1, 1, 3, 64) == 2 * 256
    assert fa.fa_bwd_workspace_size(0, 1, 1, 64) == 0


def _fwd(lib, q=P1, k=P1 + BIG, v=P1 + 2 * BIG, o=P1 + 3 * BIG, lse=P1 + 4 * BIG, B=1, H=1, N=128, d=64,
         scale=0.125, causal=0, mask=None, f32=False):
    fn = lib.fa_fwd_f32 if f32 else lib.fa_fwd
    return fn(q, k, v, o, lse, B, H, N, d, ctypes.c_float(scale), causal, mask, None)


def test_fwd_validation(lib):
    nan = float("nan")
    for f32 in (False, True):
        assert _fwd(lib, q=None, f32=f32) == 1
        assert _fwd(lib, lse=None, f32=f32) == 1
        assert _fwd(lib, B=0, f32=f32) == 1
        assert _fwd(lib, N=-5, f32=f32) == 1
        assert _fwd(lib, scale=nan, f32=f32) == 1
        assert _fwd(lib, scale=float("inf"), f32=f32) == 1
        assert _fwd(lib, causal=2, f32=f32) == 1
        assert _fwd(lib, d=72, f32=f32) == 2   # not a multiple of 16
        assert _fwd(lib, d=272, f32=f32) == 2  # above 256
        if f32:
            assert _fwd(lib, d=144, f32=f32) == 2  # the fp32 path stops at 128
        assert _fwd(lib, B=1 << 20, H=1 << 10, N=4096, f32=f32) == 1  # more than 2^31 elements
        assert _fwd(lib, o=P1, f32=f32) == 1  # output aliases q
        assert _fwd(lib, lse=P1 + 3 * BIG + 100, f32=f32) == 1  # lse inside o
        assert _fwd(lib, N=4194305, mask=P9, f32=f32) == 2
        # a head whose byte offsets (plus tail slack) would not fit 32 bits
        assert _fwd(lib, N=(1 << 25) - 1, d=64, f32=f32) == 2


def _bwd(lib, ws=P9, ws_bytes=None, B=1, H=1, N=128, d=64, dq=P1 + 6 * BIG, dk=P1 + 7 * BIG, dv=P1 + 8 * BIG,
         scale=0.125, f32=False):
    fn = lib.fa_bwd_f32 if f32 else lib.fa_bwd
    if ws_bytes is None:
        ws_bytes = lib.fa_bwd_workspace_size(B, H, N, d)
    ws = ws + 16 * BIG if ws else ws
    return fn(P1, P1 + BIG, P1 + 2 * BIG, P1 + 3 * BIG, P1 + 4 * BIG, P1 + 5 * BIG, dq, dk, dv, B, H, N, d,
              ctypes.c_float(scale), 0, None, ws, ws_bytes, None)


def test_bwd_validation(lib):
    for f32 in (False, True):
        assert _bwd(lib, ws=None, f32=f32) == 3
        assert _bwd(lib, ws_bytes=100, f32=f32) == 3
        assert _bwd(lib, ws=P9 + 8, f32=f32) == 3  # misaligned
        assert _bwd(lib, dq=None, f32=f32) == 1
        assert _bwd(lib, dk=P1 + 6 * BIG, f32=f32) == 1  # dk aliases dq
        assert _bwd(lib, dv=P1, f32=f32) == 1  # dv aliases q
        assert _bwd(lib, d=40, f32=f32) == 2   # not a multiple of 16
        assert _bwd(lib, d=144, f32=f32) == 2  # the backward stops at 128
        assert _bwd(lib, scale=float("nan"), f32=f32) == 1


def test_binding_raises_without_library(monkeypatch, tmp_path):
    monkeypatch.setattr(fa, "_lib", None)
    monkeypatch.setattr(fa, "library_path", lambda: str(tmp_path / "missing.so"))
    with pytest.raises(ImportError):
        fa.load()


def test_alignment_validation(lib):
    assert _fwd(lib, q=P1 + 2) == 1
    assert _fwd(lib, lse=P1 + 4 * BIG + 2) == 1
    assert _bwd(lib, dq=P1 + 6 * BIG + 8) == 1


def test_stage_validation(lib):
    ws = P9 + 16 * BIG
    nbytes = lib.fa_bwd_workspace_size(1, 1, 128, 64)
    assert lib.fa_bwd_prep(None, P2, P3, 1, 1, 128, 64, ws, nbytes, None) == 1
    assert lib.fa_bwd_prep(P1, P1 + BIG, None, 1, 1, 128, 64, ws, nbytes, None) == 1
    assert lib.fa_bwd_prep(P1, P1 + BIG, P1 + 2 * BIG, 1, 1, 128, 64, ws, nbytes - 1, None) == 3
    assert lib.fa_bwd_prep(P1, P1 + BIG, P1 + 2 * BIG, 1, 1, 128, 144, ws, nbytes, None) == 2
    assert lib.fa_bwd_dq(P1, P1 + BIG, P1 + 2 * BIG, P1 + 3 * BIG, None, 1, 1, 128, 64, ctypes.c_float(0.1), 0,
                         None, ws, nbytes, None) == 1
    assert lib.fa_bwd_dq(P1, P1 + BIG, P1 + 2 * BIG, P1 + 3 * BIG, P1 + 4 * BIG, 1, 1, 128, 64,
                         ctypes.c_float(0.1), 0, None, None, nbytes, None) == 3
    assert lib.fa_bwd_dq(P1, P1 + BIG, P1 + 2 * BIG, P1 + 3 * BIG, P1, 1, 1, 128, 64,
                         ctypes.c_float(0.1), 0, None, ws, nbytes, None) == 1  # dq aliases q
    assert lib.fa_bwd_main(P1, P1 + BIG, None, P1 + 3 * BIG, P1 + 4 * BIG, P1 + 5 * BIG,
                           1, 1, 128, 64, ctypes.c_float(0.1), 0, None, ws, nbytes, None) == 1
    assert lib.fa_bwd_main(P1, P1 + BIG, P1 + 2 * BIG, P1 + 3 * BIG, P1 + 4 * BIG, P1 + 4 * BIG,
                           1, 1, 128, 64, ctypes.c_float(0.1), 0, None, ws, nbytes, None) == 1  # dk aliases dv
    s = ctypes.c_float(0.1)
    # fa_bwd_dq_first(q, k, v, o, dO, lse, dq, ...): o and lse are required, dq must not alias an input
    assert lib.fa_bwd_dq_first(P1, P1 + BIG, P1 + 2 * BIG, None, P1 + 4 * BIG, P1 + 5 * BIG, P1 + 6 * BIG,
                               1, 1, 128, 64, s, 0, None, ws, nbytes, None) == 1
    assert lib.fa_bwd_dq_first(P1, P1 + BIG, P1 + 2 * BIG, P1 + 3 * BIG, P1 + 4 * BIG, None, P1 + 6 * BIG,
                               1, 1, 128, 64, s, 0, None, ws, nbytes, None) == 1
    assert lib.fa_bwd_dq_first(P1, P1 + BIG, P1 + 2 * BIG, P1 + 3 * BIG, P1 + 4 * BIG, P1 + 5 * BIG,
                               P1 + 3 * BIG, 1, 1, 128, 64, s, 0, None, ws, nbytes, None) == 1  # dq aliases o
    assert lib.fa_bwd_dq_first(P1, P1 + BIG, P1 + 2 * BIG, P1 + 3 * BIG, P1 + 4 * BIG, P1 + 5 * BIG,
                               P1 + 6 * BIG, 1, 1, 128, 64, s, 0, None, ws, nbytes - 1, None) == 3
    assert lib.fa_bwd_dq_first(P1, P1 + BIG, P1 + 2 * BIG, P1 + 3 * BIG, P1 + 4 * BIG, P1 + 5 * BIG,
                               P1 + 6 * BIG, 1, 1, 128, 144, s, 0, None, ws, nbytes, None) == 2


def test_variant_validation(lib):
    """The _ex entry points take a host fa_variant; a misaligned ALiBi slopes pointer is rejected."""
    bad = ctypes.pointer(fa.Variant(16, 0, P1 + 2))
    ok = ctypes.pointer(fa.Variant(-1, -1, None))
    s = ctypes.c_float(0.125)
    ws = P9 + 16 * BIG
    nbytes = lib.fa_bwd_workspace_size(1, 1, 128, 64)
    for fn in (lib.fa_fwd_ex, lib.fa_fwd_f32_ex):
        assert fn(P1, P1 + BIG, P1 + 2 * BIG, P1 + 3 * BIG, P1 + 4 * BIG, 1, 1, 128, 64, s, 0, None, bad,
                  None) == 1
        # other errors are still reported with a valid variant
        assert fn(P1, P1 + BIG, P1 + 2 * BIG, P1 + 3 * BIG, P1 + 4 * BIG, 1, 1, 128, 72, s, 0, None, ok,
                  None) == 2
    for fn in (lib.fa_bwd_ex, lib.fa_bwd_f32_ex):
        assert fn(P1, P1 + BIG, P1 + 2 * BIG, P1 + 3 * BIG, P1 + 4 * BIG, P1 + 5 * BIG, P1 + 6 * BIG,
                  P1 + 7 * BIG, P1 + 8 * BIG, 1, 1, 128, 64, s, 0, None, bad, ws, nbytes, None) == 1
    assert lib.fa_bwd_main_ex(P1, P1 + BIG, P1 + 2 * BIG, P1 + 3 * BIG, P1 + 4 * BIG, P1 + 5 * BIG,
                              1, 1, 128, 64, s, 0, None, bad, ws, nbytes, None) == 1
    assert lib.fa_bwd_dq_ex(P1, P1 + BIG, P1 + 2 * BIG, P1 + 3 * BIG, P1 + 4 * BIG, 1, 1, 128, 64, s, 0, None,
                            bad, ws, nbytes, None) == 1
    assert lib.fa_bwd_dq_first_ex(P1, P1 + BIG, P1 + 2 * BIG, P1 + 3 * BIG, P1 + 4 * BIG, P1 + 5 * BIG,
                                  P1 + 6 * BIG, 1, 1, 128, 64, s, 0, None, bad, ws, nbytes, None) == 1


def _dec(lib, q=P1, kc=P1 + BIG, vc=P1 + 2 * BIG, bt=P1 + 3 * BIG, sl=P1 + 4 * BIG, o=P1 + 5 * BIG,
         lse=P1 + 6 * BIG, B=2, H=8, Hkv=2, Nq=1, d=128, num_pages=16, page_size=64, max_pages=8, scale=0.1,
         causal=1, ws=P1 + 7 * BIG, ws_bytes=1 << 30):
    return lib.fa_decode_paged(q, kc, vc, bt, sl, o, lse, B, H, Hkv, Nq, d, num_pages, page_size, max_pages,
                               ctypes.c_float(scale), causal, ws, ws_bytes, None)


def test_decode_workspace_plan(lib):
    # 2 sequences x 2 KV heads: the keys split into ranges of >= 256 keys
    ws = fa.fa_decode_workspace_size(2, 8, 2, 1, 128, 64, 8)
    rows = 2 * 8 * 1
    parts = 2  # capacity 512 keys, at least 256 per range
    assert ws == (rows * parts * 128 * 4 + 255) // 256 * 256 + (rows * parts * 2 * 4 + 255) // 256 * 256
    # enough (sequence, KV head) pairs to fill the chip: one range, no workspace
    assert fa.fa_decode_workspace_size(64, 64, 64, 1, 64, 32, 4) == 0
    assert fa.fa_decode_workspace_size(2, 8, 3, 1, 128, 64, 8) == 0  # H % H_kv != 0: invalid


def test_decode_validation(lib):
    ok = fa.fa_decode_workspace_size(2, 8, 2, 1, 128, 64, 8)
    assert ok > 0
    E, U, W = 1, 2, 3
    assert _dec(lib, q=0) == E
    assert _dec(lib, bt=0) == E
    assert _dec(lib, sl=0) == E
    assert _dec(lib, Hkv=3) == E                 # H % H_kv
    assert _dec(lib, d=96) == U
    assert _dec(lib, page_size=48) == U          # not a multiple of 32
    assert _dec(lib, scale=float("nan")) == E
    assert _dec(lib, causal=2) == E
    assert _dec(lib, num_pages=0) == E
    assert _dec(lib, Nq=0) == E
    assert _dec(lib, q=P1 + 8) == E              # misaligned
    assert _dec(lib, sl=P1 + 4 * BIG + 2) == E   # misaligned int32
    assert _dec(lib, ws=0) == W
    assert _dec(lib, ws_bytes=ok - 1) == W
    assert _dec(lib, ws=P1 + 7 * BIG + 64) == W  # not 256-byte aligned
    assert _dec(lib, o=P1) == E                  # o aliases q
    assert _dec(lib, ws=P1 + BIG) == E           # workspace inside the K cache
    assert _dec(lib, max_pages=1 << 26, page_size=64) == E  # capacity >= 2^31


def test_fp8_validation(lib):
    E, U = 1, 2
    q8, k8, v8 = P1, P1 + BIG, P1 + 2 * BIG
    qe, ke, ve = P1 + 3 * BIG, P1 + 4 * BIG, P1 + 5 * BIG
    o, lse = P1 + 6 * BIG, P1 + 7 * BIG

    def fwd(**kw):
        a = dict(q=q8, qe=qe, k=k8, ke=ke, v=v8, ve=ve, o=o, lse=lse, B=1, H=2, N=300, d=128, scale=0.1, causal=1)
        a.update(kw)
        return lib.fa_fwd_fp8(a["q"], a["qe"], a["k"], a["ke"], a["v"], a["ve"], a["o"], a["lse"], a["B"], a["H"],
                              a["N"], a["d"], ctypes.c_float(a["scale"]), a["causal"], None)
    assert fwd(q=0) == E and fwd(ve=0) == E and fwd(lse=0) == E
    assert fwd(d=96) == U and fwd(N=0) == E and fwd(causal=3) == E
    assert fwd(scale=float("inf")) == E
    assert fwd(q=P1 + 4) == E               # codes must be 16-byte aligned
    assert fwd(o=P1 + 8) == E               # o misaligned
    assert fwd(o=q8) == E                   # o aliases the Q codes
    assert fwd(lse=ke) == E                 # lse aliases K's exponents

    def quant(**kw):
        a = dict(x=P1, codes=P1 + BIG, exps=P1 + 2 * BIG, B=1, H=1, N=100, d=64, signs=None, k_side=0)
        a.update(kw)
        return lib.fa_fp8_quantize(a["x"], a["codes"], a["exps"], a["B"], a["H"], a["N"], a["d"], a["signs"],
                                   a["k_side"], None)
    assert quant(x=0) == E and quant(codes=0) == E and quant(exps=0) == E
    assert quant(d=32) == U and quant(k_side=2) == E
    assert quant(codes=P1 + 100) == E       # codes overlap x
    assert quant(signs=P1 + 2 * BIG + 1) == E  # signs misaligned


def test_noalloc_validation(lib):
    """fa_bwd_noalloc rejects B*H*N beyond its static scratch before touching the GPU."""
    def call(B, H, N, d=64):
        return lib.fa_bwd_noalloc(P1, P1 + BIG, P1 + 2 * BIG, P1 + 3 * BIG, P1 + 4 * BIG, P1 + 5 * BIG,
                                  P1 + 6 * BIG, P1 + 7 * BIG, P1 + 8 * BIG, B, H, N, d, ctypes.c_float(0.125), 1,
                                  None, None, None)
    assert fa.NOALLOC_MAX_ROWS == 2097152
    assert call(1, 1, fa.NOALLOC_MAX_ROWS + 1) == 5
    assert call(2, 16, 65537) == 5
    assert call(1 << 20, 1 << 10, 4096) == 5
    assert "scratch" in fa.fa_status_string(5)
