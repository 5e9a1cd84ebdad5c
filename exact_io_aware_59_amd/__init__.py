"""Exact IO-aware attention on AMD MI355X (gfx950): Python binding of libfa.so.

Argument marshalling only: every step of the computation runs in the HIP
kernels of ``libfa.so`` (built in-tree by ``exact_io_aware_59_amd.build``).
The functions named like the C ABI (``fa_fwd``, ``fa_bwd``, ...) take torch
tensors that already live on the GPU, pass their device pointers and the
current HIP stream, and raise ``FAError`` on a non-zero status.  ``forward``
and ``backward`` additionally allocate the outputs (and the backward's
workspace) with torch.  There is no fallback: without the built library every
call raises.

Tensors are [B, H, N, d], contiguous; bf16 for fa_fwd/fa_bwd, float32 for the
_f32 entry points; lse is float32 [B, H, N]; the optional block mask is a
uint8 tensor [ceil(N/128), ceil(N/128)] on the same device.  The _ex entry
points (and ``forward`` / ``backward`` given ``window`` or ``alibi_slopes``)
take the local window (left, right) -- None or a negative bound is
unbounded -- and ALiBi slopes as a float32 tensor [H] on the device.
"""
from __future__ import annotations

import ctypes
import math
import os
from typing import Optional, Tuple

__all__ = [
    "FAError", "library_path", "load", "fa_fwd", "fa_fwd_f32", "fa_bwd", "fa_bwd_f32",
    "fa_bwd_workspace_size", "fa_bwd_prep", "fa_bwd_main", "fa_bwd_dq", "fa_bwd_dq_first", "fa_status_string",
    "fa_version", "fa_bwd_dq_first_ex",
    "fa_fwd_ex", "fa_fwd_f32_ex", "fa_bwd_ex", "fa_bwd_f32_ex", "fa_bwd_main_ex", "fa_bwd_dq_ex", "Variant",
    "forward", "backward", "workspace", "fa_decode_workspace_size", "fa_decode_paged", "decode_workspace",
    "decode_paged", "fa_fp8_quantize", "fa_fwd_fp8", "quantize_fp8", "forward_fp8", "FP8_BLOCK",
    "MASK_BLOCK", "ABI_VERSION", "fa_bwd_noalloc", "NOALLOC_MAX_ROWS", "load_debug", "debug_library_path",
    "fa_debug_flags", "DEBUG_ROW_SUM", "DEBUG_NON_FINITE", "attention",
]

MASK_BLOCK = 128
ABI_VERSION = 7  # FA_VERSION of the fa.h these argument lists follow
NOALLOC_MAX_ROWS = 2097152  # FA_NOALLOC_MAX_ROWS
_PKG = os.path.dirname(os.path.abspath(__file__))
_lib = None


class Variant(ctypes.Structure):
    """fa_variant: local window (negative = unbounded) and a device pointer to ALiBi slopes (or 0)."""
    _fields_ = [("window_left", ctypes.c_int), ("window_right", ctypes.c_int),
                ("alibi_slopes", ctypes.c_void_p)]


class FAError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {fa_status_string(status)} (status {status})")


def library_path() -> str:
    return os.path.join(_PKG, "libfa.so")


def debug_library_path() -> str:
    """The same library built with the kernels' debug self-check (FA_DEBUG_CHECK)."""
    return os.path.join(_PKG, "libfa_debug.so")


def load():
    """Load libfa.so (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    _lib = _open(library_path())
    return _lib


def load_debug():
    """A separate handle on libfa_debug.so, with the same argument lists as
    load(); the module's wrappers keep using libfa.so."""
    return _open(debug_library_path())


def _open(path: str):
    if not os.path.exists(path):
        raise ImportError(f"{path} is missing: build it with `python -m exact_io_aware_59_amd.build`")
    lib = ctypes.CDLL(path)
    vp, i, f, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t
    lib.fa_fwd.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, f, i, vp, vp]
    lib.fa_fwd_f32.argtypes = lib.fa_fwd.argtypes
    lib.fa_bwd.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, i, i, i, i, f, i, vp, vp, sz, vp]
    lib.fa_bwd_f32.argtypes = lib.fa_bwd.argtypes
    lib.fa_bwd_prep.argtypes = [vp, vp, vp, i, i, i, i, vp, sz, vp]
    lib.fa_bwd_main.argtypes = [vp, vp, vp, vp, vp, vp, i, i, i, i, f, i, vp, vp, sz, vp]
    lib.fa_bwd_dq.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, f, i, vp, vp, sz, vp]
    vr = ctypes.POINTER(Variant)
    lib.fa_fwd_ex.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, f, i, vp, vr, vp]
    lib.fa_fwd_f32_ex.argtypes = lib.fa_fwd_ex.argtypes
    lib.fa_bwd_ex.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, i, i, i, i, f, i, vp, vr, vp, sz, vp]
    lib.fa_bwd_f32_ex.argtypes = lib.fa_bwd_ex.argtypes
    lib.fa_bwd_noalloc.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, i, i, i, i, f, i, vp, vr, vp]
    lib.fa_bwd_main_ex.argtypes = [vp, vp, vp, vp, vp, vp, i, i, i, i, f, i, vp, vr, vp, sz, vp]
    lib.fa_bwd_dq_ex.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, f, i, vp, vr, vp, sz, vp]
    lib.fa_bwd_dq_first.argtypes = [vp, vp, vp, vp, vp, vp, vp, i, i, i, i, f, i, vp, vp, sz, vp]
    lib.fa_bwd_dq_first_ex.argtypes = [vp, vp, vp, vp, vp, vp, vp, i, i, i, i, f, i, vp, vr, vp, sz, vp]
    for name in ("fa_fwd", "fa_fwd_f32", "fa_bwd", "fa_bwd_f32", "fa_bwd_prep", "fa_bwd_main", "fa_bwd_dq",
                 "fa_version", "fa_fwd_ex", "fa_fwd_f32_ex", "fa_bwd_ex", "fa_bwd_f32_ex", "fa_bwd_main_ex",
                 "fa_bwd_dq_ex", "fa_bwd_dq_first", "fa_bwd_dq_first_ex", "fa_decode_paged", "fa_fp8_quantize",
                 "fa_fwd_fp8", "fa_bwd_noalloc"):
        getattr(lib, name).restype = i
    lib.fa_decode_workspace_size.argtypes = [i, i, i, i, i, i, i]
    lib.fa_decode_workspace_size.restype = sz
    lib.fa_decode_paged.argtypes = [vp, vp, vp, vp, vp, vp, vp, i, i, i, i, i, i, i, i, f, i, vp, sz, vp]
    lib.fa_decode_paged.restype = i
    lib.fa_fp8_quantize.argtypes = [vp, vp, vp, i, i, i, i, vp, i, vp]
    lib.fa_fp8_quantize.restype = i
    lib.fa_fwd_fp8.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, i, i, i, i, f, i, vp]
    lib.fa_fwd_fp8.restype = i
    lib.fa_bwd_workspace_size.argtypes = [i, i, i, i]
    lib.fa_bwd_workspace_size.restype = sz
    lib.fa_status_string.argtypes = [i]
    lib.fa_status_string.restype = ctypes.c_char_p
    lib.fa_version.argtypes = []
    lib.fa_debug_flags.argtypes = [i]
    lib.fa_debug_flags.restype = i
    if lib.fa_version() != ABI_VERSION:
        raise ImportError(f"{path} reports ABI version {lib.fa_version()}, the binding expects {ABI_VERSION}: "
                          "rebuild it with `python -m exact_io_aware_59_amd.build`")
    return lib


def fa_status_string(status: int) -> str:
    return load().fa_status_string(int(status)).decode()


def fa_version() -> int:
    return int(load().fa_version())


DEBUG_ROW_SUM = 1      # FA_DEBUG_ROW_SUM
DEBUG_NON_FINITE = 2   # FA_DEBUG_NON_FINITE


def fa_debug_flags(clear: bool = False, lib=None) -> int:
    """Self-check flags of a FA_DEBUG_CHECK build (load_debug()); 0 for libfa.so."""
    return int((lib or load()).fa_debug_flags(1 if clear else 0))


def fa_bwd_workspace_size(B: int, H: int, N: int, d: int) -> int:
    return int(load().fa_bwd_workspace_size(B, H, N, d))


# ----------------------------------------------------------------------------
# marshalling helpers
# ----------------------------------------------------------------------------

def _ptr(t) -> Optional[int]:
    if t is None:
        return None
    if not t.is_contiguous():
        raise ValueError("tensors must be contiguous")
    return t.data_ptr()


def _stream(stream) -> Optional[int]:
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _dims(q) -> Tuple[int, int, int, int]:
    import torch
    if not isinstance(q, torch.Tensor) or q.dim() != 4:
        raise ValueError("expected a [B, H, N, d] torch tensor")
    B, H, N, d = q.shape
    return int(B), int(H), int(N), int(d)


def _variant(window=None, alibi_slopes=None):
    """ctypes fa_variant pointer (or None for the plain computation)."""
    if window is None and alibi_slopes is None:
        return None
    wl, wr = window if window is not None else (None, None)
    v = Variant(-1 if wl is None or wl < 0 else int(wl), -1 if wr is None or wr < 0 else int(wr),
                _ptr(alibi_slopes) if alibi_slopes is not None else None)
    return ctypes.pointer(v)


def _check(status: int, where: str):
    if status != 0:
        raise FAError(status, where)


# ----------------------------------------------------------------------------
# argument validation (the C ABI sees plain pointers and cannot check what a
# buffer holds: a wrong dtype, shape or device would make a kernel read or
# write past an allocation, so every mirror checks its tensors first and
# raises ValueError before anything is enqueued)
# ----------------------------------------------------------------------------

def _dtype(name: str):
    import torch
    return {"bf16": torch.bfloat16, "f32": torch.float32, "u8": torch.uint8, "i8": torch.int8,
            "i32": torch.int32, "bool": torch.bool}[name]


def _tensors(where: str, specs, device=None):
    """specs: (name, tensor or None, dtype name(s), shape or None, optional).  Checks dtype, then
    shape, then that every tensor is a contiguous CUDA tensor on one device; returns that device."""
    import torch
    for name, t, dts, shape, optional in specs:
        if t is None:
            if optional:
                continue
            raise ValueError(f"{where}: {name} is required")
        if not isinstance(t, torch.Tensor):
            raise ValueError(f"{where}: {name} must be a torch tensor")
        allowed = [_dtype(x) for x in (dts if isinstance(dts, tuple) else (dts,))]
        if t.dtype not in allowed:
            raise ValueError(f"{where}: {name} has dtype {t.dtype}, expected "
                             + " or ".join(str(a) for a in allowed))
        if shape is not None and tuple(t.shape) != tuple(shape):
            raise ValueError(f"{where}: {name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    for name, t, _, _, _ in specs:
        if t is None:
            continue
        if t.device.type != "cuda":
            raise ValueError(f"{where}: {name} is on {t.device}, expected a CUDA (HIP) device")
        if device is None:
            device = t.device
        elif t.device != device:
            raise ValueError(f"{where}: {name} is on {t.device}, the other tensors on {device}")
        if not t.is_contiguous():
            raise ValueError(f"{where}: {name} must be contiguous")
    return device


def _attn_specs(dt: str, q, B, H, N, d, **named):
    """Specs for tensors of the attention entry points: bf16/f32 [B,H,N,d] ones
    (q, k, v, o, do, dq, dk, dv), lse float32 [B,H,N]."""
    specs = [("q", q, dt, (B, H, N, d), False)] if q is not None else []
    for name, t in named.items():
        if name == "lse":
            specs.append(("lse", t, "f32", (B, H, N), False))
        else:
            specs.append((name, t, dt, (B, H, N, d), False))
    return specs


def _mask_spec(blockmask, N):
    """uint8 or bool [ceil(N/128)]^2 (both one byte per entry, nonzero = kept)."""
    nb = (N + MASK_BLOCK - 1) // MASK_BLOCK
    return ("blockmask", blockmask, ("u8", "bool"), (nb, nb), True)


def _variant_specs(H, window, alibi_slopes):
    if window is not None:
        if len(window) != 2 or any(w is not None and not isinstance(w, int) for w in window):
            raise ValueError("window must be (left, right) with int or None bounds")
    return [("alibi_slopes", alibi_slopes, "f32", (H,), True)]


def _ws_spec(workspace):
    return ("workspace", workspace, "u8", None, True)


# ----------------------------------------------------------------------------
# C ABI mirrors
# ----------------------------------------------------------------------------

def fa_fwd(q, k, v, o, lse, scale: float, causal: bool = False, blockmask=None, stream=None):
    B, H, N, d = _dims(q)
    _tensors("fa_fwd", _attn_specs("bf16", q, B, H, N, d, k=k, v=v, o=o, lse=lse) + [_mask_spec(blockmask, N)])
    _check(load().fa_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), B, H, N, d, float(scale),
                         int(bool(causal)), _ptr(blockmask), _stream(stream)), "fa_fwd")


def fa_fwd_f32(q, k, v, o, lse, scale: float, causal: bool = False, blockmask=None, stream=None):
    B, H, N, d = _dims(q)
    _tensors("fa_fwd_f32", _attn_specs("f32", q, B, H, N, d, k=k, v=v, o=o, lse=lse) + [_mask_spec(blockmask, N)])
    _check(load().fa_fwd_f32(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), B, H, N, d, float(scale),
                             int(bool(causal)), _ptr(blockmask), _stream(stream)), "fa_fwd_f32")


def fa_bwd(q, k, v, o, do, lse, dq, dk, dv, scale: float, causal: bool = False, blockmask=None,
           workspace=None, stream=None):
    B, H, N, d = _dims(q)
    _tensors("fa_bwd", _attn_specs("bf16", q, B, H, N, d, k=k, v=v, o=o, do=do, lse=lse, dq=dq, dk=dk, dv=dv)
             + [_mask_spec(blockmask, N), _ws_spec(workspace)])
    nbytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _check(load().fa_bwd(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(do), _ptr(lse), _ptr(dq), _ptr(dk),
                         _ptr(dv), B, H, N, d, float(scale), int(bool(causal)), _ptr(blockmask),
                         _ptr(workspace), nbytes, _stream(stream)), "fa_bwd")


def fa_bwd_f32(q, k, v, o, do, lse, dq, dk, dv, scale: float, causal: bool = False, blockmask=None,
               workspace=None, stream=None):
    B, H, N, d = _dims(q)
    _tensors("fa_bwd_f32", _attn_specs("f32", q, B, H, N, d, k=k, v=v, o=o, do=do, lse=lse, dq=dq, dk=dk, dv=dv)
             + [_mask_spec(blockmask, N), _ws_spec(workspace)])
    nbytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _check(load().fa_bwd_f32(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(do), _ptr(lse), _ptr(dq),
                             _ptr(dk), _ptr(dv), B, H, N, d, float(scale), int(bool(causal)),
                             _ptr(blockmask), _ptr(workspace), nbytes, _stream(stream)), "fa_bwd_f32")


def _nbytes(t) -> int:
    return t.numel() * t.element_size() if t is not None else 0


def fa_bwd_prep(o, do, lse, workspace, stream=None):
    B, H, N, d = _dims(o)
    _tensors("fa_bwd_prep", _attn_specs("bf16", None, B, H, N, d, o=o, do=do, lse=lse) + [_ws_spec(workspace)])
    _check(load().fa_bwd_prep(_ptr(o), _ptr(do), _ptr(lse), B, H, N, d, _ptr(workspace), _nbytes(workspace),
                              _stream(stream)), "fa_bwd_prep")


def fa_bwd_main(q, k, v, do, dk, dv, scale: float, causal: bool = False, blockmask=None, workspace=None,
                stream=None):
    B, H, N, d = _dims(q)
    _tensors("fa_bwd_main", _attn_specs("bf16", q, B, H, N, d, k=k, v=v, do=do, dk=dk, dv=dv)
             + [_mask_spec(blockmask, N), _ws_spec(workspace)])
    _check(load().fa_bwd_main(_ptr(q), _ptr(k), _ptr(v), _ptr(do), _ptr(dk), _ptr(dv), B, H, N, d,
                              float(scale), int(bool(causal)), _ptr(blockmask), _ptr(workspace),
                              _nbytes(workspace), _stream(stream)), "fa_bwd_main")


def fa_bwd_dq(q, k, v, do, dq, scale: float, causal: bool = False, blockmask=None, workspace=None, stream=None):
    B, H, N, d = _dims(q)
    _tensors("fa_bwd_dq", _attn_specs("bf16", q, B, H, N, d, k=k, v=v, do=do, dq=dq)
             + [_mask_spec(blockmask, N), _ws_spec(workspace)])
    _check(load().fa_bwd_dq(_ptr(q), _ptr(k), _ptr(v), _ptr(do), _ptr(dq), B, H, N, d, float(scale),
                            int(bool(causal)), _ptr(blockmask), _ptr(workspace), _nbytes(workspace),
                            _stream(stream)), "fa_bwd_dq")


def fa_bwd_dq_first(q, k, v, o, do, lse, dq, scale: float, causal: bool = False, blockmask=None, workspace=None,
                    stream=None):
    B, H, N, d = _dims(q)
    _tensors("fa_bwd_dq_first", _attn_specs("bf16", q, B, H, N, d, k=k, v=v, o=o, do=do, lse=lse, dq=dq)
             + [_mask_spec(blockmask, N), _ws_spec(workspace)])
    _check(load().fa_bwd_dq_first(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(do), _ptr(lse), _ptr(dq), B, H, N, d,
                                  float(scale), int(bool(causal)), _ptr(blockmask), _ptr(workspace),
                                  _nbytes(workspace), _stream(stream)), "fa_bwd_dq_first")


def fa_fwd_ex(q, k, v, o, lse, scale: float, causal: bool = False, blockmask=None, window=None,
              alibi_slopes=None, stream=None):
    B, H, N, d = _dims(q)
    _tensors("fa_fwd_ex", _attn_specs("bf16", q, B, H, N, d, k=k, v=v, o=o, lse=lse) + [_mask_spec(blockmask, N)]
             + _variant_specs(H, window, alibi_slopes))
    _check(load().fa_fwd_ex(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), B, H, N, d, float(scale),
                            int(bool(causal)), _ptr(blockmask), _variant(window, alibi_slopes), _stream(stream)),
           "fa_fwd_ex")


def fa_fwd_f32_ex(q, k, v, o, lse, scale: float, causal: bool = False, blockmask=None, window=None,
                  alibi_slopes=None, stream=None):
    B, H, N, d = _dims(q)
    _tensors("fa_fwd_f32_ex", _attn_specs("f32", q, B, H, N, d, k=k, v=v, o=o, lse=lse)
             + [_mask_spec(blockmask, N)] + _variant_specs(H, window, alibi_slopes))
    _check(load().fa_fwd_f32_ex(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), B, H, N, d, float(scale),
                                int(bool(causal)), _ptr(blockmask), _variant(window, alibi_slopes),
                                _stream(stream)), "fa_fwd_f32_ex")


def fa_bwd_ex(q, k, v, o, do, lse, dq, dk, dv, scale: float, causal: bool = False, blockmask=None, window=None,
              alibi_slopes=None, workspace=None, stream=None):
    B, H, N, d = _dims(q)
    _tensors("fa_bwd_ex", _attn_specs("bf16", q, B, H, N, d, k=k, v=v, o=o, do=do, lse=lse, dq=dq, dk=dk, dv=dv)
             + [_mask_spec(blockmask, N), _ws_spec(workspace)] + _variant_specs(H, window, alibi_slopes))
    _check(load().fa_bwd_ex(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(do), _ptr(lse), _ptr(dq), _ptr(dk),
                            _ptr(dv), B, H, N, d, float(scale), int(bool(causal)), _ptr(blockmask),
                            _variant(window, alibi_slopes), _ptr(workspace), _nbytes(workspace),
                            _stream(stream)), "fa_bwd_ex")


def fa_bwd_noalloc(q, k, v, o, do, lse, dq, dk, dv, scale: float, causal: bool = False, blockmask=None,
                   window=None, alibi_slopes=None, stream=None):
    """fa_bwd_ex without a workspace: the library's static device scratch holds
    the backward's row vectors (B*H*N <= NOALLOC_MAX_ROWS; calls that overlap
    in time on one GPU race)."""
    B, H, N, d = _dims(q)
    _tensors("fa_bwd_noalloc", _attn_specs("bf16", q, B, H, N, d, k=k, v=v, o=o, do=do, lse=lse, dq=dq, dk=dk, dv=dv)
             + [_mask_spec(blockmask, N)] + _variant_specs(H, window, alibi_slopes))
    _check(load().fa_bwd_noalloc(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(do), _ptr(lse), _ptr(dq), _ptr(dk),
                                 _ptr(dv), B, H, N, d, float(scale), int(bool(causal)), _ptr(blockmask),
                                 _variant(window, alibi_slopes), _stream(stream)), "fa_bwd_noalloc")


def fa_bwd_f32_ex(q, k, v, o, do, lse, dq, dk, dv, scale: float, causal: bool = False, blockmask=None,
                  window=None, alibi_slopes=None, workspace=None, stream=None):
    B, H, N, d = _dims(q)
    _tensors("fa_bwd_f32_ex", _attn_specs("f32", q, B, H, N, d, k=k, v=v, o=o, do=do, lse=lse, dq=dq, dk=dk, dv=dv)
             + [_mask_spec(blockmask, N), _ws_spec(workspace)] + _variant_specs(H, window, alibi_slopes))
    _check(load().fa_bwd_f32_ex(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(do), _ptr(lse), _ptr(dq), _ptr(dk),
                                _ptr(dv), B, H, N, d, float(scale), int(bool(causal)), _ptr(blockmask),
                                _variant(window, alibi_slopes), _ptr(workspace), _nbytes(workspace),
                                _stream(stream)), "fa_bwd_f32_ex")


def fa_bwd_main_ex(q, k, v, do, dk, dv, scale: float, causal: bool = False, blockmask=None, window=None,
                   alibi_slopes=None, workspace=None, stream=None):
    B, H, N, d = _dims(q)
    _tensors("fa_bwd_main_ex", _attn_specs("bf16", q, B, H, N, d, k=k, v=v, do=do, dk=dk, dv=dv)
             + [_mask_spec(blockmask, N), _ws_spec(workspace)] + _variant_specs(H, window, alibi_slopes))
    _check(load().fa_bwd_main_ex(_ptr(q), _ptr(k), _ptr(v), _ptr(do), _ptr(dk), _ptr(dv), B, H, N, d,
                                 float(scale), int(bool(causal)), _ptr(blockmask), _variant(window, alibi_slopes),
                                 _ptr(workspace), _nbytes(workspace), _stream(stream)), "fa_bwd_main_ex")


def fa_bwd_dq_ex(q, k, v, do, dq, scale: float, causal: bool = False, blockmask=None, window=None,
                 alibi_slopes=None, workspace=None, stream=None):
    B, H, N, d = _dims(q)
    _tensors("fa_bwd_dq_ex", _attn_specs("bf16", q, B, H, N, d, k=k, v=v, do=do, dq=dq)
             + [_mask_spec(blockmask, N), _ws_spec(workspace)] + _variant_specs(H, window, alibi_slopes))
    _check(load().fa_bwd_dq_ex(_ptr(q), _ptr(k), _ptr(v), _ptr(do), _ptr(dq), B, H, N, d, float(scale),
                               int(bool(causal)), _ptr(blockmask), _variant(window, alibi_slopes), _ptr(workspace),
                               _nbytes(workspace), _stream(stream)), "fa_bwd_dq_ex")


def fa_bwd_dq_first_ex(q, k, v, o, do, lse, dq, scale: float, causal: bool = False, blockmask=None, window=None,
                       alibi_slopes=None, workspace=None, stream=None):
    B, H, N, d = _dims(q)
    _tensors("fa_bwd_dq_first_ex", _attn_specs("bf16", q, B, H, N, d, k=k, v=v, o=o, do=do, lse=lse, dq=dq)
             + [_mask_spec(blockmask, N), _ws_spec(workspace)] + _variant_specs(H, window, alibi_slopes))
    _check(load().fa_bwd_dq_first_ex(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(do), _ptr(lse), _ptr(dq), B, H, N,
                                     d, float(scale), int(bool(causal)), _ptr(blockmask),
                                     _variant(window, alibi_slopes), _ptr(workspace), _nbytes(workspace),
                                     _stream(stream)), "fa_bwd_dq_first_ex")


# ----------------------------------------------------------------------------
# allocating wrappers
# ----------------------------------------------------------------------------

def fa_decode_workspace_size(B: int, H: int, H_kv: int, Nq: int, d: int, page_size: int, max_pages: int) -> int:
    return int(load().fa_decode_workspace_size(B, H, H_kv, Nq, d, page_size, max_pages))


def fa_decode_paged(q, k_cache, v_cache, block_table, seqlens, o, lse, scale: float, causal: bool = True,
                    workspace=None, stream=None):
    """Decode over a paged KV cache (bf16): q [B,H,Nq,d]; caches [num_pages,page_size,H_kv,d];
    block_table int32 [B,max_pages]; seqlens int32 [B]; writes o [B,H,Nq,d] and lse [B,H,Nq]."""
    B, H, Nq, d = _dims(q)
    import torch
    if not isinstance(k_cache, torch.Tensor) or k_cache.dim() != 4 or int(k_cache.shape[3]) != d:
        raise ValueError("fa_decode_paged: k_cache must be [num_pages, page_size, H_kv, d]")
    num_pages, page_size, H_kv, _ = (int(x) for x in k_cache.shape)
    if not isinstance(block_table, torch.Tensor) or block_table.dim() != 2 or int(block_table.shape[0]) != B:
        raise ValueError("fa_decode_paged: block_table must be int32 [B, max_pages]")
    max_pages = int(block_table.shape[1])
    _tensors("fa_decode_paged", [
        ("q", q, "bf16", (B, H, Nq, d), False),
        ("k_cache", k_cache, "bf16", (num_pages, page_size, H_kv, d), False),
        ("v_cache", v_cache, "bf16", (num_pages, page_size, H_kv, d), False),
        ("block_table", block_table, "i32", (B, max_pages), False),
        ("seqlens", seqlens, "i32", (B,), False),
        ("o", o, "bf16", (B, H, Nq, d), False),
        ("lse", lse, "f32", (B, H, Nq), False),
        _ws_spec(workspace)])
    _check(load().fa_decode_paged(_ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(block_table), _ptr(seqlens),
                                  _ptr(o), _ptr(lse), B, H, H_kv, Nq, d, num_pages, page_size, max_pages,
                                  float(scale), int(bool(causal)), _ptr(workspace), _nbytes(workspace),
                                  _stream(stream)), "fa_decode_paged")


def decode_workspace(q, k_cache, block_table):
    """A workspace tensor for decode_paged / fa_decode_paged, or None when none is needed."""
    import torch
    B, H, Nq, d = _dims(q)
    _, page_size, H_kv, _ = (int(x) for x in k_cache.shape)
    n = fa_decode_workspace_size(B, H, H_kv, Nq, d, page_size, int(block_table.shape[1]))
    return torch.empty(n, dtype=torch.uint8, device=q.device) if n > 0 else None


def decode_paged(q, k_cache, v_cache, block_table, seqlens, scale: Optional[float] = None, causal: bool = True,
                 ws=None, stream=None):
    """Allocate o and lse (and a workspace) on q's device and run fa_decode_paged."""
    import torch
    B, H, Nq, d = _dims(q)
    scale = _default_scale(d) if scale is None else scale
    o = torch.empty_like(q)
    lse = torch.empty((B, H, Nq), dtype=torch.float32, device=q.device)
    if ws is None:
        ws = decode_workspace(q, k_cache, block_table)
    fa_decode_paged(q, k_cache, v_cache, block_table, seqlens, o, lse, scale, causal, ws, stream)
    return o, lse


FP8_BLOCK = 64


def fa_fp8_quantize(x, codes, exps, signs=None, k_side: bool = False, stream=None):
    """Block-quantize bf16 x [B,H,N,d] to E4M3 codes (uint8, same shape) and int8
    block exponents [B,H,ceil(N/64)]; signs (float [d] of +-1) applies the incoherent map."""
    B, H, N, d = _dims(x)
    _tensors("fa_fp8_quantize", [
        ("x", x, "bf16", (B, H, N, d), False),
        ("codes", codes, "u8", (B, H, N, d), False),
        ("exps", exps, "i8", (B, H, (N + FP8_BLOCK - 1) // FP8_BLOCK), False),
        ("signs", signs, "f32", (d,), True)])
    _check(load().fa_fp8_quantize(_ptr(x), _ptr(codes), _ptr(exps), B, H, N, d, _ptr(signs), int(bool(k_side)),
                                  _stream(stream)), "fa_fp8_quantize")


def fa_fwd_fp8(q8, qe, k8, ke, v8, ve, o, lse, scale: float, causal: bool = False, stream=None):
    B, H, N, d = _dims(q8)
    ne = (B, H, (N + FP8_BLOCK - 1) // FP8_BLOCK)
    _tensors("fa_fwd_fp8", [
        ("q8", q8, "u8", (B, H, N, d), False), ("qe", qe, "i8", ne, False),
        ("k8", k8, "u8", (B, H, N, d), False), ("ke", ke, "i8", ne, False),
        ("v8", v8, "u8", (B, H, N, d), False), ("ve", ve, "i8", ne, False),
        ("o", o, "bf16", (B, H, N, d), False), ("lse", lse, "f32", (B, H, N), False)])
    _check(load().fa_fwd_fp8(_ptr(q8), _ptr(qe), _ptr(k8), _ptr(ke), _ptr(v8), _ptr(ve), _ptr(o), _ptr(lse), B, H,
                             N, d, float(scale), int(bool(causal)), _stream(stream)), "fa_fwd_fp8")


def quantize_fp8(x, signs=None, k_side: bool = False, stream=None):
    """Allocate and fill (codes, exps) for a bf16 tensor on its device."""
    import torch
    B, H, N, d = _dims(x)
    codes = torch.empty((B, H, N, d), dtype=torch.uint8, device=x.device)
    exps = torch.empty((B, H, (N + FP8_BLOCK - 1) // FP8_BLOCK), dtype=torch.int8, device=x.device)
    fa_fp8_quantize(x, codes, exps, signs, k_side, stream)
    return codes, exps


def forward_fp8(q, k, v, scale: Optional[float] = None, causal: bool = False, signs=None, stream=None):
    """Quantize bf16 q, k, v (q and k through the incoherent map when signs is given)
    and run the FP8 forward; returns (o bf16, lse)."""
    import torch
    B, H, N, d = _dims(q)
    scale = _default_scale(d) if scale is None else scale
    q8, qe = quantize_fp8(q, signs, False, stream)
    k8, ke = quantize_fp8(k, signs, True, stream)
    v8, ve = quantize_fp8(v, None, False, stream)
    o = torch.empty_like(q)
    lse = torch.empty((B, H, N), dtype=torch.float32, device=q.device)
    fa_fwd_fp8(q8, qe, k8, ke, v8, ve, o, lse, scale, causal, stream)
    return o, lse


def _compute_dtype(q, where: str):
    """forward / backward run bf16 tensors on the bf16 kernels and float32 ones
    on the fp32 kernels; any other dtype is rejected (the entry points then
    check every other tensor against q)."""
    import torch
    if q.dtype not in (torch.bfloat16, torch.float32):
        raise ValueError(f"{where}: q has dtype {q.dtype}; bfloat16 and float32 are supported")


def _default_scale(d: int) -> float:
    return 1.0 / math.sqrt(d)


def forward(q, k, v, scale: Optional[float] = None, causal: bool = False, blockmask=None, stream=None,
            window=None, alibi_slopes=None):
    """Returns (o, lse).  bf16 inputs use fa_fwd(_ex), float32 inputs fa_fwd_f32(_ex)."""
    import torch
    B, H, N, d = _dims(q)
    _compute_dtype(q, "forward")
    scale = _default_scale(d) if scale is None else scale
    o = torch.empty_like(q)
    lse = torch.empty((B, H, N), dtype=torch.float32, device=q.device)
    if window is None and alibi_slopes is None:
        fn = fa_fwd if q.dtype == torch.bfloat16 else fa_fwd_f32
        fn(q, k, v, o, lse, scale, causal, blockmask, stream)
    else:
        fn = fa_fwd_ex if q.dtype == torch.bfloat16 else fa_fwd_f32_ex
        fn(q, k, v, o, lse, scale, causal, blockmask, window, alibi_slopes, stream)
    return o, lse


def workspace(B: int, H: int, N: int, d: int, device):
    """A backward workspace of the size fa_bwd needs (256-byte aligned by torch's allocator)."""
    import torch
    return torch.empty(fa_bwd_workspace_size(B, H, N, d), dtype=torch.uint8, device=device)


def backward(q, k, v, o, do, lse, scale: Optional[float] = None, causal: bool = False, blockmask=None,
             ws=None, stream=None, window=None, alibi_slopes=None):
    """Returns (dq, dk, dv).  bf16 inputs use fa_bwd(_ex), float32 inputs fa_bwd_f32(_ex)."""
    import torch
    B, H, N, d = _dims(q)
    _compute_dtype(q, "backward")
    scale = _default_scale(d) if scale is None else scale
    dq, dk, dv = torch.empty_like(q), torch.empty_like(q), torch.empty_like(q)
    if ws is None:
        ws = workspace(B, H, N, d, q.device)
    if window is None and alibi_slopes is None:
        fn = fa_bwd if q.dtype == torch.bfloat16 else fa_bwd_f32
        fn(q, k, v, o, do, lse, dq, dk, dv, scale, causal, blockmask, ws, stream)
    else:
        fn = fa_bwd_ex if q.dtype == torch.bfloat16 else fa_bwd_f32_ex
        fn(q, k, v, o, do, lse, dq, dk, dv, scale, causal, blockmask, window, alibi_slopes, ws, stream)
    return dq, dk, dv


_attention_fn = None


def _attention_function():
    """The autograd Function behind ``attention`` (built on first use, so that
    importing the binding does not import torch)."""
    global _attention_fn
    if _attention_fn is None:
        import torch

        class _Attention(torch.autograd.Function):
            @staticmethod
            def forward(ctx, q, k, v, scale, causal, blockmask, window, alibi_slopes):
                o, lse = forward(q, k, v, scale, causal, blockmask, window=window, alibi_slopes=alibi_slopes)
                ctx.save_for_backward(q, k, v, o, lse)
                ctx.args = (scale, causal, blockmask, window, alibi_slopes)
                ctx.mark_non_differentiable(lse)
                return o, lse

            @staticmethod
            def backward(ctx, do, _dlse):
                q, k, v, o, lse = ctx.saved_tensors
                scale, causal, blockmask, window, alibi_slopes = ctx.args
                dq, dk, dv = backward(q, k, v, o, do.contiguous(), lse, scale, causal, blockmask,
                                      window=window, alibi_slopes=alibi_slopes)
                return dq, dk, dv, None, None, None, None, None

        _attention_fn = _Attention
    return _attention_fn


def attention(q, k, v, scale: Optional[float] = None, causal: bool = False, blockmask=None, window=None,
              alibi_slopes=None, return_lse: bool = False):
    """Exact attention softmax(scale Q K^T [+ mask / window / ALiBi]) V with autograd.

    q, k, v: contiguous [B, H, N, d] bf16 (bf16 kernels) or float32 (fp32
    kernels) tensors on the GPU; scale defaults to 1/sqrt(d).  The forward
    runs ``forward`` and saves (q, k, v, O, lse); the backward runs
    ``backward`` on the incoming dO (made contiguous), so the gradients are
    those of fa_bwd(_ex) / fa_bwd_f32(_ex).  lse (float32 [B, H, N], natural
    log) is returned too with ``return_lse`` and carries no gradient."""
    d = q.shape[-1]
    scale = _default_scale(d) if scale is None else scale
    o, lse = _attention_function().apply(q, k, v, scale, causal, blockmask, window, alibi_slopes)
    return (o, lse) if return_lse else o
