"""fp64 CPU oracle for exact softmax attention.

TEST INFRASTRUCTURE ONLY: imported by ``tests/``, by the ``smoke()`` check and
by the CPU-baseline leg of ``bench.py``.  The product path (the HIP library
and its binding) never imports, links or calls anything here, and this module
imports nothing from it.

The arithmetic lives in ``ref_attn.c`` (plain C, OpenMP over rows, no BLAS);
this file only compiles it with gcc and marshals numpy arrays.  All functions
take and return float64 arrays of shape [B, H, N, d] (lse: [B, H, N]), an
optional uint8 block mask [nb, nb], nb = ceil(N / 128), and optionally a local
window ``window=(wl, wr)`` (key j allowed for query i iff i - wl <= j <= i + wr,
a negative bound = unbounded) and ALiBi slopes ``slopes`` [H] (the score gets
-slope_h * |i - j|).  ``attn_paged_fwd`` is decode over a paged KV cache.

Every function is pinned by tests/test_oracle.py against facts that do not
come from this code: a brute-force evaluation with a different softmax
formula, closed forms, invariances and central finite differences.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional, Tuple

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "ref_attn.c")
_LIB = os.path.join(_HERE, "libref_attn.so")
_lib = None

_dp = ctypes.POINTER(ctypes.c_double)
_u8p = ctypes.POINTER(ctypes.c_uint8)
_i64p = ctypes.POINTER(ctypes.c_int64)


def build(force: bool = False) -> str:
    """Compile ref_attn.c into libref_attn.so with gcc (fp64, no fast-math)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp%d" % os.getpid()
        cmd = ["gcc", "-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared", "-ffp-contract=off",
               _SRC, "-o", tmp, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB)
    return _LIB


class _Lib:
    """ctypes view of one compiled copy of ref_attn.c."""

    def __init__(self, path: str):
        lib = ctypes.CDLL(path)
        c_int, c_double = ctypes.c_int, ctypes.c_double
        lib.ref_num_threads.restype = c_int
        lib.ref_attn_probs.argtypes = [_dp, _dp, c_int, c_int, c_double, c_int, _u8p, _dp, _dp]
        lib.ref_attn_fwd.argtypes = [_dp, _dp, _dp, c_int, c_int, c_int, c_int, c_double, c_int,
                                     _u8p, _dp, _dp]
        lib.ref_attn_fwd_rows.argtypes = [_dp, _dp, _dp, c_int, c_int, c_int, c_int, c_double,
                                          c_int, _u8p, _i64p, c_int, _dp, _dp]
        lib.ref_attn_fwd_online.argtypes = [_dp, _dp, _dp, c_int, c_int, c_int, c_int, c_double,
                                            c_int, _u8p, c_int, _dp, _dp]
        lib.ref_attn_bwd.argtypes = [_dp, _dp, _dp, _dp, c_int, c_int, c_int, c_int, c_double,
                                     c_int, _u8p, _dp, _dp, _dp, _dp, _dp, _dp]
        lib.ref_attn_fwd_ex.argtypes = [_dp, _dp, _dp, c_int, c_int, c_int, c_int, c_double, c_int,
                                        _u8p, c_int, c_int, _dp, _dp, _dp]
        lib.ref_attn_fwd_rows_ex.argtypes = [_dp, _dp, _dp, c_int, c_int, c_int, c_int, c_double,
                                             c_int, _u8p, c_int, c_int, _dp, _i64p, c_int, _dp, _dp]
        lib.ref_attn_fwd_online_ex.argtypes = [_dp, _dp, _dp, c_int, c_int, c_int, c_int, c_double,
                                               c_int, _u8p, c_int, c_int, _dp, c_int, _dp, _dp]
        lib.ref_attn_bwd_ex.argtypes = [_dp, _dp, _dp, _dp, c_int, c_int, c_int, c_int, c_double,
                                        c_int, _u8p, c_int, c_int, _dp, _dp, _dp, _dp, _dp, _dp, _dp]
        _i32p = ctypes.POINTER(ctypes.c_int32)
        lib.ref_attn_paged_fwd.argtypes = [_dp, _dp, _dp, _i32p, _i32p, c_int, c_int, c_int, c_int, c_int,
                                           c_int, c_int, c_int, c_double, c_int, _dp, _dp]
        _u8 = ctypes.POINTER(ctypes.c_uint8)
        _i8 = ctypes.POINTER(ctypes.c_int8)
        lib.ref_e4m3_encode.argtypes = [_dp, ctypes.c_long, _u8]
        lib.ref_e4m3_decode.argtypes = [_u8, ctypes.c_long, _dp]
        lib.ref_fp8_quantize.argtypes = [_dp, c_int, c_int, c_int, c_int, c_int, _dp, c_int, _u8, _i8]
        lib.ref_hadamard.argtypes = [_dp, ctypes.c_long, c_int, _dp, c_int, _dp]
        for f in ("ref_attn_probs", "ref_attn_fwd", "ref_attn_fwd_rows", "ref_attn_fwd_online",
                  "ref_attn_bwd", "ref_attn_fwd_ex", "ref_attn_fwd_rows_ex", "ref_attn_fwd_online_ex",
                  "ref_attn_bwd_ex", "ref_attn_paged_fwd", "ref_e4m3_encode", "ref_e4m3_decode",
                  "ref_fp8_quantize", "ref_hadamard"):
            getattr(lib, f).restype = c_int
        self.lib = lib


def _load():
    global _lib
    if _lib is None:
        build()
        _lib = _Lib(_LIB).lib
    return _lib


def num_threads() -> int:
    """OpenMP threads the oracle uses (OMP_NUM_THREADS, else all cores)."""
    return int(_load().ref_num_threads())


def _f64(a) -> np.ndarray:
    return np.ascontiguousarray(a, dtype=np.float64)


def _ptr(a: Optional[np.ndarray], t=_dp):
    if a is None:
        return ctypes.cast(None, t)
    return a.ctypes.data_as(t)


def _mask(mask, N: int):
    if mask is None:
        return None
    m = np.ascontiguousarray(mask, dtype=np.uint8)
    nb = (N + 127) // 128
    if m.shape != (nb, nb):
        raise ValueError(f"mask must be [{nb}, {nb}], got {m.shape}")
    return m


def _shape(q):
    if q.ndim != 4:
        raise ValueError("expected [B, H, N, d]")
    return q.shape


def _window(window):
    """(wl, wr) with -1 for an unbounded side."""
    if window is None:
        return -1, -1
    wl, wr = window
    wl = -1 if wl is None or wl < 0 else int(wl)
    wr = -1 if wr is None or wr < 0 else int(wr)
    return wl, wr


def _slopes(slopes, H: int):
    if slopes is None:
        return None
    a = np.ascontiguousarray(slopes, dtype=np.float64).reshape(-1)
    if a.shape != (H,):
        raise ValueError(f"slopes must have H={H} entries, got {a.shape}")
    return a


def _check(rc: int, what: str):
    if rc != 0:
        raise MemoryError(f"oracle {what} failed (allocation)")


def attn_fwd(q, k, v, scale: float, causal: bool = False, mask=None, window=None,
             slopes=None) -> Tuple[np.ndarray, np.ndarray]:
    """Exact attention forward: (O [B,H,N,d], lse [B,H,N]) from the definition."""
    q, k, v = _f64(q), _f64(k), _f64(v)
    B, H, N, d = _shape(q)
    m = _mask(mask, N)
    wl, wr = _window(window)
    sl = _slopes(slopes, H)
    o = np.empty_like(q)
    lse = np.empty((B, H, N), dtype=np.float64)
    rc = _load().ref_attn_fwd_ex(_ptr(q), _ptr(k), _ptr(v), B, H, N, d, float(scale), int(causal),
                                 _ptr(m, _u8p), wl, wr, _ptr(sl), _ptr(o), _ptr(lse))
    _check(rc, "fwd")
    return o, lse


def attn_paged_fwd(q, k_cache, v_cache, block_table, seqlens, scale: float,
                   causal: bool = False) -> Tuple[np.ndarray, np.ndarray]:
    """Decode over a paged KV cache: (O [B,H,Nq,d], lse [B,H,Nq]).

    q: [B, H, Nq, d]; k_cache, v_cache: [num_pages, page_size, Hkv, d];
    block_table: [B, max_pages] int32 (logical page -> physical page);
    seqlens: [B] int32.  Query head h reads KV head h // (H // Hkv); the Nq
    queries are the last Nq positions of their sequence (causal: query i sees
    positions <= L - Nq + i).
    """
    q, kc, vc = _f64(q), _f64(k_cache), _f64(v_cache)
    B, H, Nq, d = _shape(q)
    if kc.ndim != 4 or kc.shape != vc.shape or kc.shape[3] != d:
        raise ValueError("k_cache and v_cache must be [num_pages, page_size, Hkv, d]")
    num_pages, page_size, Hkv, _ = kc.shape
    bt = np.ascontiguousarray(block_table, dtype=np.int32)
    sl = np.ascontiguousarray(seqlens, dtype=np.int32).reshape(-1)
    if bt.ndim != 2 or bt.shape[0] != B or sl.shape != (B,):
        raise ValueError("block_table must be [B, max_pages] and seqlens [B]")
    o = np.empty_like(q)
    lse = np.empty((B, H, Nq), dtype=np.float64)
    i32p = ctypes.POINTER(ctypes.c_int32)
    rc = _load().ref_attn_paged_fwd(_ptr(q), _ptr(kc), _ptr(vc), _ptr(bt, i32p), _ptr(sl, i32p), B, H, Hkv, Nq,
                                    d, num_pages, page_size, bt.shape[1], float(scale), int(causal),
                                    _ptr(o), _ptr(lse))
    if rc != 0:
        raise ValueError(f"oracle paged_fwd rejected its arguments (code {rc})")
    return o, lse


def e4m3_encode(x) -> np.ndarray:
    """Nearest FP8 E4M3 (OCP E4M3FN) codes of x, ties to even, saturating at +-448."""
    a = _f64(x)
    out = np.empty(a.shape, dtype=np.uint8)
    _load().ref_e4m3_encode(_ptr(a), a.size, _ptr(out, ctypes.POINTER(ctypes.c_uint8)))
    return out


def e4m3_decode(codes) -> np.ndarray:
    c = np.ascontiguousarray(codes, dtype=np.uint8)
    out = np.empty(c.shape, dtype=np.float64)
    _load().ref_e4m3_decode(_ptr(c, ctypes.POINTER(ctypes.c_uint8)), c.size, _ptr(out))
    return out


def hadamard(x, sigma, inverse_side: bool = False) -> np.ndarray:
    """Rows of x [..., d] -> H (sigma o x) (times 1/d when inverse_side), H Sylvester of order d."""
    a = _f64(x)
    d = a.shape[-1]
    sg = _f64(sigma).reshape(-1)
    out = np.empty_like(a)
    rc = _load().ref_hadamard(_ptr(a), a.size // d, d, _ptr(sg), int(inverse_side), _ptr(out))
    if rc != 0:
        raise ValueError("hadamard needs d a power of two")
    return out


def fp8_quantize(x, block: int, sigma=None, inverse_side: bool = False):
    """Block quantization of [B, H, N, d] (after the optional incoherent map):
    (codes uint8 [B,H,N,d], exponents int8 [B,H,ceil(N/block)])."""
    a = _f64(x)
    B, H, N, d = _shape(a)
    sg = None if sigma is None else _f64(sigma).reshape(-1)
    codes = np.empty(a.shape, dtype=np.uint8)
    exps = np.empty((B, H, -(-N // block)), dtype=np.int8)
    rc = _load().ref_fp8_quantize(_ptr(a), B, H, N, d, int(block), _ptr(sg), int(inverse_side),
                                  _ptr(codes, ctypes.POINTER(ctypes.c_uint8)), _ptr(exps, ctypes.POINTER(ctypes.c_int8)))
    if rc != 0:
        raise ValueError("fp8_quantize: bad block or d")
    return codes, exps


def fp8_dequantize(codes, exps, block: int) -> np.ndarray:
    v = e4m3_decode(codes)
    N = v.shape[2]
    e = np.repeat(np.asarray(exps, dtype=np.float64), block, axis=2)[:, :, :N]
    return v * np.exp2(e)[..., None]


def attn_fp8_fwd(q, k, v, scale: float, causal: bool = False, block: int = 64, sigma=None):
    """FP8 forward reference: Q and K through the incoherent map (if sigma), Q, K
    and V block-quantized to E4M3, exact attention of the dequantized values.
    Returns (O, lse, quantized) with quantized = {name: (codes, exps)}."""
    qc = fp8_quantize(q, block, sigma, False)
    kc = fp8_quantize(k, block, sigma, True)
    vc = fp8_quantize(v, block, None, False)
    o, lse = attn_fwd(fp8_dequantize(*qc, block), fp8_dequantize(*kc, block), fp8_dequantize(*vc, block),
                      scale, causal)
    return o, lse, {"q": qc, "k": kc, "v": vc}


def attn_fwd_rows(q, k, v, scale: float, rows, causal: bool = False, mask=None, window=None, slopes=None):
    """Output rows only: rows is [R, 2] of (b*H + h, i).  Returns (O [R, d], lse [R])."""
    q, k, v = _f64(q), _f64(k), _f64(v)
    B, H, N, d = _shape(q)
    m = _mask(mask, N)
    r = np.ascontiguousarray(rows, dtype=np.int64)
    if r.ndim != 2 or r.shape[1] != 2:
        raise ValueError("rows must be [R, 2]")
    if r.size and (r[:, 0].min() < 0 or r[:, 0].max() >= B * H or r[:, 1].min() < 0 or r[:, 1].max() >= N):
        raise ValueError("row index out of range")
    wl, wr = _window(window)
    sl = _slopes(slopes, H)
    o = np.empty((r.shape[0], d), dtype=np.float64)
    lse = np.empty((r.shape[0],), dtype=np.float64)
    rc = _load().ref_attn_fwd_rows_ex(_ptr(q), _ptr(k), _ptr(v), B, H, N, d, float(scale), int(causal),
                                      _ptr(m, _u8p), wl, wr, _ptr(sl), _ptr(r, _i64p), r.shape[0],
                                      _ptr(o), _ptr(lse))
    _check(rc, "fwd_rows")
    return o, lse


def attn_fwd_online(q, k, v, scale: float, chunk: int, causal: bool = False, mask=None, window=None,
                    slopes=None):
    """Online-softmax forward scanning keys in chunks of ``chunk`` (same outputs as attn_fwd)."""
    q, k, v = _f64(q), _f64(k), _f64(v)
    B, H, N, d = _shape(q)
    m = _mask(mask, N)
    wl, wr = _window(window)
    sl = _slopes(slopes, H)
    o = np.empty_like(q)
    lse = np.empty((B, H, N), dtype=np.float64)
    rc = _load().ref_attn_fwd_online_ex(_ptr(q), _ptr(k), _ptr(v), B, H, N, d, float(scale),
                                        int(causal), _ptr(m, _u8p), wl, wr, _ptr(sl), int(chunk), _ptr(o),
                                        _ptr(lse))
    _check(rc, "fwd_online")
    return o, lse


def attn_probs(q_head, k_head, scale: float, causal: bool = False, mask=None):
    """P [N, N] and lse [N] of one head (q_head, k_head: [N, d])."""
    q, k = _f64(q_head), _f64(k_head)
    N, d = q.shape
    m = _mask(mask, N)
    P = np.empty((N, N), dtype=np.float64)
    lse = np.empty((N,), dtype=np.float64)
    rc = _load().ref_attn_probs(_ptr(q), _ptr(k), N, d, float(scale), int(causal), _ptr(m, _u8p),
                                _ptr(P), _ptr(lse))
    _check(rc, "probs")
    return P, lse


def attn_bwd(q, k, v, do, scale: float, causal: bool = False, mask=None, return_fwd: bool = False,
             window=None, slopes=None):
    """Gradients (dQ, dK, dV) of sum(dO * O) with O the exact attention output.

    With ``return_fwd`` also returns (O, lse, D) where D_i = sum_j P_ij dP_ij.
    """
    q, k, v, do = _f64(q), _f64(k), _f64(v), _f64(do)
    B, H, N, d = _shape(q)
    m = _mask(mask, N)
    wl, wr = _window(window)
    sl = _slopes(slopes, H)
    dq, dk, dv = np.empty_like(q), np.empty_like(q), np.empty_like(q)
    o = np.empty_like(q) if return_fwd else None
    lse = np.empty((B, H, N)) if return_fwd else None
    D = np.empty((B, H, N)) if return_fwd else None
    rc = _load().ref_attn_bwd_ex(_ptr(q), _ptr(k), _ptr(v), _ptr(do), B, H, N, d, float(scale),
                                 int(causal), _ptr(m, _u8p), wl, wr, _ptr(sl), _ptr(dq), _ptr(dk),
                                 _ptr(dv), _ptr(o), _ptr(lse), _ptr(D))
    _check(rc, "bwd")
    if return_fwd:
        return dq, dk, dv, o, lse, D
    return dq, dk, dv


class Oracle:
    """The functions above bound to a given compiled copy of the oracle.

    ``Oracle()`` is the oracle itself.  ``Oracle(path)`` loads another build of
    a (possibly modified) ref_attn.c; tests use it to plant mistakes in the
    oracle and show that the pins catch them.
    """

    def __init__(self, path: Optional[str] = None):
        self._path = path

    def _swap(self, fn, *a, **kw):
        global _lib
        if self._path is None:
            return fn(*a, **kw)
        saved = _lib
        _lib = _Lib(self._path).lib
        try:
            return fn(*a, **kw)
        finally:
            _lib = saved

    def attn_fwd(self, *a, **kw):
        return self._swap(attn_fwd, *a, **kw)

    def attn_fwd_rows(self, *a, **kw):
        return self._swap(attn_fwd_rows, *a, **kw)

    def attn_fwd_online(self, *a, **kw):
        return self._swap(attn_fwd_online, *a, **kw)

    def attn_probs(self, *a, **kw):
        return self._swap(attn_probs, *a, **kw)

    def attn_bwd(self, *a, **kw):
        return self._swap(attn_bwd, *a, **kw)

    def attn_paged_fwd(self, *a, **kw):
        return self._swap(attn_paged_fwd, *a, **kw)

    def e4m3_encode(self, *a, **kw):
        return self._swap(e4m3_encode, *a, **kw)

    def e4m3_decode(self, *a, **kw):
        return self._swap(e4m3_decode, *a, **kw)

    def hadamard(self, *a, **kw):
        return self._swap(hadamard, *a, **kw)

    def fp8_quantize(self, *a, **kw):
        return self._swap(fp8_quantize, *a, **kw)

    def fp8_dequantize(self, *a, **kw):
        return self._swap(fp8_dequantize, *a, **kw)

    def attn_fp8_fwd(self, *a, **kw):
        return self._swap(attn_fp8_fwd, *a, **kw)


def build_variant(src_text: str, out_path: str) -> str:
    """Compile a modified copy of ref_attn.c (given as text) to ``out_path``."""
    src = out_path + ".c"
    with open(src, "w") as f:
        f.write(src_text)
    subprocess.run(["gcc", "-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared", "-ffp-contract=off",
                    src, "-o", out_path, "-lm"], check=True)
    return out_path


def source_text() -> str:
    with open(_SRC) as f:
        return f.read()
