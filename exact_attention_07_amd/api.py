"""ctypes binding of libfa.so (entry points declared in include/fa.h).

Argument marshalling only: every step of the attention runs in the HIP
kernels of libfa.so.  Tensors are torch tensors on the GPU (torch provides
device memory and the current stream); the library is loaded on first use and
its absence is an error.
"""
from __future__ import annotations

import ctypes
import math
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libfa.so")

FA_STATUS = {0: "FA_OK", 1: "FA_ERR_NULL", 2: "FA_ERR_SHAPE", 3: "FA_ERR_HEAD_DIM", 4: "FA_ERR_GQA_RATIO",
             5: "FA_ERR_ALIGN", 6: "FA_ERR_SCALE", 7: "FA_ERR_HIP", 8: "FA_ERR_FLAG"}

_lib = None


class FaError(RuntimeError):
    def __init__(self, status: int, what: str):
        super().__init__(f"{what}: {FA_STATUS.get(status, status)} ({_lib.fa_status_string(status).decode()})")
        self.status = status


def lib() -> ctypes.CDLL:
    """Load libfa.so (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build it with `python -m exact_attention_07_amd.build`")
    L = ctypes.CDLL(LIB_PATH)
    vp, i, f = ctypes.c_void_p, ctypes.c_int, ctypes.c_float
    fwd_args = [vp, vp, vp, vp, vp, i, i, i, i, i, i, f, i, vp]
    for name in ("fa_fwd", "fa_fwd_f32"):
        fn = getattr(L, name)
        fn.argtypes = fwd_args
        fn.restype = ctypes.c_int
    L.fa_status_string.argtypes = [ctypes.c_int]
    L.fa_status_string.restype = ctypes.c_char_p
    L.fa_abi_version.argtypes = []
    L.fa_abi_version.restype = ctypes.c_int
    _lib = L
    return L


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    import torch
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _shapes(q, k, v, o, lse):
    if q.dim() != 4 or k.dim() != 4 or v.dim() != 4:
        raise ValueError("q, k, v must be [B, H, N, d]")
    B, Hq, Nq, d = q.shape
    Bk, Hkv, Nk, dk = k.shape
    if tuple(v.shape) != tuple(k.shape) or Bk != B or dk != d:
        raise ValueError(f"shape mismatch q{tuple(q.shape)} k{tuple(k.shape)} v{tuple(v.shape)}")
    if tuple(o.shape) != tuple(q.shape):
        raise ValueError("o must have q's shape")
    if lse is not None and tuple(lse.shape) != (B, Hq, Nq):
        raise ValueError("lse must be [B, Hq, Nq]")
    for t in (q, k, v, o) + ((lse,) if lse is not None else ()):
        if not t.is_cuda or not t.is_contiguous():
            raise ValueError("tensors must be contiguous GPU tensors")
    return B, Hq, Hkv, Nq, Nk, d


def _check(st, what):
    if st != 0:
        raise FaError(st, what)


def fa_fwd(q, k, v, o, lse, scale: float, causal: bool, stream=None) -> None:
    """bf16 forward pass into caller-allocated o (bf16) and lse (fp32 or None)."""
    import torch
    for t in (q, k, v, o):
        if t.dtype != torch.bfloat16:
            raise TypeError("fa_fwd takes bfloat16 q, k, v, o")
    B, Hq, Hkv, Nq, Nk, d = _shapes(q, k, v, o, lse)
    _check(lib().fa_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), B, Hq, Hkv, Nq, Nk, d,
                        float(scale), int(bool(causal)), _stream(stream)), "fa_fwd")


def fa_fwd_f32(q, k, v, o, lse, scale: float, causal: bool, stream=None) -> None:
    """fp32 forward pass into caller-allocated o (fp32) and lse (fp32 or None)."""
    import torch
    for t in (q, k, v, o):
        if t.dtype != torch.float32:
            raise TypeError("fa_fwd_f32 takes float32 q, k, v, o")
    B, Hq, Hkv, Nq, Nk, d = _shapes(q, k, v, o, lse)
    _check(lib().fa_fwd_f32(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), B, Hq, Hkv, Nq, Nk, d,
                            float(scale), int(bool(causal)), _stream(stream)), "fa_fwd_f32")


def attention(q, k, v, causal: bool = False, scale: float | None = None, stream=None):
    """Allocate o and lse and run the forward pass matching q's dtype; returns (o, lse)."""
    import torch
    if scale is None:
        scale = 1.0 / math.sqrt(q.shape[-1])
    o = torch.empty_like(q)
    lse = torch.empty(q.shape[:3], dtype=torch.float32, device=q.device)
    if q.dtype == torch.bfloat16:
        fa_fwd(q, k, v, o, lse, scale, causal, stream)
    elif q.dtype == torch.float32:
        fa_fwd_f32(q, k, v, o, lse, scale, causal, stream)
    else:
        raise TypeError(f"unsupported dtype {q.dtype}")
    return o, lse
