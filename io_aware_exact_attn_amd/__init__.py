"""Python binding of the gfx950 exact-attention library (``libattn.so``).

Argument marshalling only: every step of the computation runs in the HIP
kernels behind the C ABI declared in ``include/attn.h``.  The functions keep
the C names and argument order; tensors may be passed where the C side takes
a pointer (their ``data_ptr()`` is used, and they must be CUDA/HIP tensors),
and a ``torch.cuda.Stream`` (or ``None`` for the current stream) where it
takes a stream.

If the library has not been built, importing this package raises
``ImportError``: there is no fallback implementation.
"""
from __future__ import annotations

import ctypes
import os

__all__ = [
    "ATTN_OK", "ATTN_ERR_NULL", "ATTN_ERR_SHAPE", "ATTN_ERR_UNSUPPORTED", "ATTN_ERR_SCALE",
    "ATTN_ERR_ALIGN", "ATTN_ERR_HIP", "ATTN_ERR_SCRATCH", "ATTN_BF16", "ATTN_BF16_OUT_F32", "ATTN_FP8_E4M3",
    "AttnError", "attn_fwd", "attn_fwd_fp8", "attn_bwd", "attn_bwd_noalloc", "attn_quantize_fp8", "attn_status_str", "attn_kernel_name",
    "library_path", "lib",
]

ATTN_OK, ATTN_ERR_NULL, ATTN_ERR_SHAPE, ATTN_ERR_UNSUPPORTED = 0, 1, 2, 3
ATTN_ERR_SCALE, ATTN_ERR_ALIGN, ATTN_ERR_HIP, ATTN_ERR_SCRATCH = 4, 5, 6, 7
ATTN_BF16, ATTN_BF16_OUT_F32, ATTN_FP8_E4M3 = 0, 1, 2

_HERE = os.path.dirname(os.path.abspath(__file__))
library_path = os.path.join(_HERE, "libattn.so")

if not os.path.exists(library_path):
    raise ImportError(
        f"{library_path} is missing: build it with `python io_aware_exact_attn_amd/build.py` "
        "(there is no non-HIP implementation)")

# PyTorch owns the device memory and the streams handed to the library, and it
# ships its own HIP runtime, loaded under the unversioned name libamdhip64.so.
# Importing torch first lets the dynamic loader resolve the library's
# libamdhip64.so.7 to that same runtime (same SONAME).  Loading the library
# first would map a second HIP runtime into the process, in which torch's
# pointers and stream handles are invalid.
import torch  # noqa: E402,F401

lib = ctypes.CDLL(library_path)

_vp, _i, _f = ctypes.c_void_p, ctypes.c_int, ctypes.c_float
lib.attn_fwd.argtypes = [_vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _f, _i, _vp, _i, _vp]
lib.attn_fwd.restype = _i
lib.attn_fwd_fp8.argtypes = [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _f, _i, _vp, _vp]
lib.attn_fwd_fp8.restype = _i
lib.attn_bwd.argtypes = [_vp] * 10 + [_i, _i, _i, _i, _f, _i, _vp, _vp]
lib.attn_bwd.restype = _i
lib.attn_bwd_noalloc.argtypes = [_vp] * 9 + [_i, _i, _i, _i, _f, _i, _vp, _vp]
lib.attn_bwd_noalloc.restype = _i
lib.attn_quantize_fp8.argtypes = [_vp, _vp, _vp, _i, _i, _i, _i, _vp, _vp]
lib.attn_quantize_fp8.restype = _i
lib.attn_quantize_fp8_rotated.argtypes = [_vp, _vp, _vp, _vp, _i, _i, _i, _i, _vp, _vp]
lib.attn_quantize_fp8_rotated.restype = _i
lib.attn_quantize_mxfp8.argtypes = [_vp, _vp, _vp, _i, _i, _i, _i, _vp, _i, _vp]
lib.attn_quantize_mxfp8.restype = _i
lib.attn_fwd_mxfp8.argtypes = [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _f, _i, _vp, _vp]
lib.attn_fwd_mxfp8.restype = _i
lib.attn_status_str.argtypes = [_i]
lib.attn_status_str.restype = ctypes.c_char_p
lib.attn_kernel_name.argtypes = [_i, _i, _i, _i, _i]
lib.attn_kernel_name.restype = ctypes.c_char_p


class AttnError(RuntimeError):
    def __init__(self, status: int, fn: str):
        super().__init__(f"{fn}: {attn_status_str(status)} (status {status})")
        self.status = status


def _ptr(x):
    """A device pointer from a tensor, an int address, or None (NULL)."""
    if x is None:
        return None
    if isinstance(x, int):
        return x
    if hasattr(x, "data_ptr"):
        if not x.is_cuda:
            raise ValueError("tensor arguments must live in GPU memory")
        return x.data_ptr()
    raise TypeError(f"cannot pass {type(x).__name__} as a pointer")


def _stream(s):
    if s is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(s, int):
        return s
    return s.cuda_stream


def attn_status_str(status: int) -> str:
    return lib.attn_status_str(status).decode()


def attn_kernel_name(d: int, causal: int, packed: int, dtype: int, fp8: int = 0) -> str:
    return lib.attn_kernel_name(d, causal, packed, dtype, fp8).decode()


def attn_fwd(q, k, v, o, lse, B, H, N, d, scale, causal, cu_seqlens, dtype, stream=None,
             check: bool = True) -> int:
    """Enqueue the bf16 attention forward (see ``attn_fwd`` in include/attn.h).

    Returns the status; with ``check`` a nonzero status raises AttnError.
    """
    st = lib.attn_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), int(B), int(H), int(N),
                      int(d), float(scale), int(causal), _ptr(cu_seqlens), int(dtype),
                      _stream(stream))
    if check and st != ATTN_OK:
        raise AttnError(st, "attn_fwd")
    return st


def attn_fwd_fp8(q, k, v, q_scale, k_scale, v_scale, o, lse, B, H, N, d, scale, causal,
                 cu_seqlens=None, stream=None, check: bool = True) -> int:
    """Enqueue the block-scaled e4m3 attention forward (see ``attn_fwd_fp8``)."""
    st = lib.attn_fwd_fp8(_ptr(q), _ptr(k), _ptr(v), _ptr(q_scale), _ptr(k_scale), _ptr(v_scale),
                          _ptr(o), _ptr(lse), int(B), int(H), int(N), int(d), float(scale),
                          int(causal), _ptr(cu_seqlens), _stream(stream))
    if check and st != ATTN_OK:
        raise AttnError(st, "attn_fwd_fp8")
    return st


def attn_fwd_mxfp8(q, k, v, q_scale, k_scale, v_scale, o, lse, B, H, N, d, scale, causal,
                   cu_seqlens=None, stream=None, check: bool = True) -> int:
    """Enqueue the MXFP8 attention forward (see ``attn_fwd_mxfp8``)."""
    st = lib.attn_fwd_mxfp8(_ptr(q), _ptr(k), _ptr(v), _ptr(q_scale), _ptr(k_scale), _ptr(v_scale),
                            _ptr(o), _ptr(lse), int(B), int(H), int(N), int(d), float(scale),
                            int(causal), _ptr(cu_seqlens), _stream(stream))
    if check and st != ATTN_OK:
        raise AttnError(st, "attn_fwd_mxfp8")
    return st


def attn_quantize_fp8(x, y, scales, B, H, N, d, cu_seqlens=None, stream=None, check: bool = True) -> int:
    """Enqueue the bf16 -> e4m3 block quantisation (see ``attn_quantize_fp8``)."""
    st = lib.attn_quantize_fp8(_ptr(x), _ptr(y), _ptr(scales), int(B), int(H), int(N), int(d),
                               _ptr(cu_seqlens), _stream(stream))
    if check and st != ATTN_OK:
        raise AttnError(st, "attn_quantize_fp8")
    return st


def attn_quantize_fp8_rotated(x, y, scales, signs, B, H, N, d, cu_seqlens=None, stream=None,
                              check: bool = True) -> int:
    """Enqueue the random-sign Hadamard rotation plus e4m3 block quantisation
    (see ``attn_quantize_fp8_rotated``); ``signs`` is a device int8 tensor of d."""
    st = lib.attn_quantize_fp8_rotated(_ptr(x), _ptr(y), _ptr(scales), _ptr(signs), int(B), int(H), int(N),
                                       int(d), _ptr(cu_seqlens), _stream(stream))
    if check and st != ATTN_OK:
        raise AttnError(st, "attn_quantize_fp8_rotated")
    return st


def attn_quantize_mxfp8(x, y, scales, B, H, N, d, cu_seqlens=None, along_tokens=0, stream=None,
                        check: bool = True) -> int:
    """Enqueue the bf16 -> MXFP8 quantisation (see ``attn_quantize_mxfp8``):
    blocks of 32 along d (Q, K) or, with ``along_tokens``, along tokens (V)."""
    st = lib.attn_quantize_mxfp8(_ptr(x), _ptr(y), _ptr(scales), int(B), int(H), int(N), int(d), _ptr(cu_seqlens),
                                 int(along_tokens), _stream(stream))
    if check and st != ATTN_OK:
        raise AttnError(st, "attn_quantize_mxfp8")
    return st


def attn_bwd(q, k, v, o, dout, lse, delta, dq, dk, dv, B, H, N, d, scale, causal, cu_seqlens=None,
             stream=None, check: bool = True) -> int:
    """Enqueue the bf16 attention backward (see ``attn_bwd`` in include/attn.h)."""
    st = lib.attn_bwd(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(dout), _ptr(lse), _ptr(delta), _ptr(dq),
                      _ptr(dk), _ptr(dv), int(B), int(H), int(N), int(d), float(scale), int(causal),
                      _ptr(cu_seqlens), _stream(stream))
    if check and st != ATTN_OK:
        raise AttnError(st, "attn_bwd")
    return st


def attn_bwd_noalloc(q, k, v, o, dout, lse, dq, dk, dv, B, H, N, d, scale, causal, cu_seqlens=None,
                     stream=None, check: bool = True) -> int:
    """Enqueue the bf16 attention backward without a caller workspace (see
    ``attn_bwd_noalloc`` in include/attn.h): D goes to the library's fixed
    per-GPU scratch."""
    st = lib.attn_bwd_noalloc(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(dout), _ptr(lse), _ptr(dq), _ptr(dk),
                              _ptr(dv), int(B), int(H), int(N), int(d), float(scale), int(causal),
                              _ptr(cu_seqlens), _stream(stream))
    if check and st != ATTN_OK:
        raise AttnError(st, "attn_bwd_noalloc")
    return st
