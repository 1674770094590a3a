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
             5: "FA_ERR_ALIGN", 6: "FA_ERR_SCALE", 7: "FA_ERR_HIP", 8: "FA_ERR_FLAG", 9: "FA_ERR_WORKSPACE",
             10: "FA_ERR_SCRATCH_LIMIT"}

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
    L.fa_fwd_exp2_emulated.argtypes = fwd_args[:-1] + [i, vp]
    L.fa_fwd_exp2_emulated.restype = ctypes.c_int
    L.fa_fp8_prepare.argtypes = [vp] * 9 + [f] + [i] * 6 + [vp]
    L.fa_fp8_prepare.restype = ctypes.c_int
    L.fa_fwd_fp8.argtypes = [vp] * 6 + [i] * 6 + [i, vp]
    L.fa_fwd_fp8.restype = ctypes.c_int
    L.fa_fwd_splitkv.argtypes = [vp] * 5 + [i] * 6 + [f, i, i, vp, ctypes.c_size_t, vp]
    L.fa_fwd_splitkv.restype = ctypes.c_int
    L.fa_fwd_splitkv_noalloc.argtypes = [vp] * 5 + [i] * 6 + [f, i, i, vp]
    L.fa_fwd_splitkv_noalloc.restype = ctypes.c_int
    L.fa_fwd_splitkv_workspace_size.argtypes = [i] * 8
    L.fa_fwd_splitkv_workspace_size.restype = ctypes.c_size_t
    L.fa_bwd.argtypes = [vp] * 9 + [i] * 6 + [f, i, vp, ctypes.c_size_t, vp]
    L.fa_bwd.restype = ctypes.c_int
    L.fa_bwd_dq.argtypes = [vp] * 7 + [i] * 6 + [f, i, vp, ctypes.c_size_t, vp]
    L.fa_bwd_dq.restype = ctypes.c_int
    L.fa_bwd_dkdv.argtypes = [vp] * 6 + [i] * 6 + [f, i, vp, ctypes.c_size_t, vp]
    L.fa_bwd_dkdv.restype = ctypes.c_int
    L.fa_bwd_workspace_size.argtypes = [i] * 7
    L.fa_bwd_workspace_size.restype = ctypes.c_size_t
    L.fa_mfma_ceiling_out_bytes.argtypes = []
    L.fa_mfma_ceiling_out_bytes.restype = ctypes.c_size_t
    L.fa_mfma_ceiling_flops.argtypes = [i, i]
    L.fa_mfma_ceiling_flops.restype = ctypes.c_double
    L.fa_mfma_ceiling.argtypes = [vp, ctypes.c_size_t, i, i, i, vp]
    L.fa_mfma_ceiling.restype = ctypes.c_int
    L.fa_issue_cost_cases.argtypes = []
    L.fa_issue_cost_cases.restype = ctypes.c_int
    ip = ctypes.POINTER(ctypes.c_int)
    L.fa_issue_cost_case.argtypes = [i, ip, ip, ip, ip]
    L.fa_issue_cost_case.restype = ctypes.c_int
    L.fa_issue_cost_case_mfma.argtypes = [i, ip]
    L.fa_issue_cost_case_mfma.restype = ctypes.c_int
    L.fa_issue_cost.argtypes = [vp, ctypes.c_size_t, i, i, vp]
    L.fa_issue_cost.restype = ctypes.c_int
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


def fa_fwd_exp2_emulated(q, k, v, o, lse, scale: float, causal: bool, quarters: int, stream=None) -> None:
    """fa_fwd with `quarters` (1 or 2) of every four exponentials computed on the FMA pipe (d = 64, 128)."""
    import torch
    for t in (q, k, v, o):
        if t.dtype != torch.bfloat16:
            raise TypeError("fa_fwd_exp2_emulated takes bfloat16 q, k, v, o")
    B, Hq, Hkv, Nq, Nk, d = _shapes(q, k, v, o, lse)
    _check(lib().fa_fwd_exp2_emulated(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), B, Hq, Hkv, Nq, Nk, d,
                                      float(scale), int(bool(causal)), int(quarters), _stream(stream)),
           "fa_fwd_exp2_emulated")


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


def padded_keys(nk: int) -> int:
    """Key count of the transposed fp8 V (a multiple of 64)."""
    return (nk + 63) // 64 * 64


def fa_fp8_prepare(q, k, v, q8, k8, v8t, descale, amax_ws, signs=None, scale: float | None = None,
                   stream=None) -> None:
    """Rotate (if signs is given) and quantise bf16 q, k, v into e4m3 codes (uint8 tensors) for the
    softmax scale `scale` (default 1/sqrt(d)), which the Q codes carry."""
    import torch
    B, Hq, Nq, d = q.shape
    _, Hkv, Nk, _ = k.shape
    if q.dtype != torch.bfloat16 or k.dtype != torch.bfloat16 or v.dtype != torch.bfloat16:
        raise TypeError("fa_fp8_prepare takes bfloat16 q, k, v")
    if tuple(q8.shape) != tuple(q.shape) or tuple(k8.shape) != tuple(k.shape) or \
            tuple(v8t.shape) != (B, Hkv, d, padded_keys(Nk)) or tuple(v.shape) != tuple(k.shape):
        raise ValueError("code tensor shapes: q8 like q, k8 like k, v8t [B, Hkv, d, Nk rounded up to 64]")
    for t in (q8, k8, v8t):
        if t.dtype != torch.uint8:
            raise TypeError("code tensors are uint8")
    if descale.numel() < 3 or descale.dtype != torch.float32 or amax_ws.numel() < 3 or amax_ws.dtype != torch.int32:
        raise ValueError("descale: 3 float32, amax_ws: 3 int32")
    for t in (q, k, v, q8, k8, v8t, descale, amax_ws) + ((signs,) if signs is not None else ()):
        if not t.is_cuda or not t.is_contiguous():
            raise ValueError("tensors must be contiguous GPU tensors")
    if signs is not None and (signs.numel() != d or signs.dtype != torch.float32):
        raise ValueError("signs: d float32 values")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    _check(lib().fa_fp8_prepare(_ptr(q), _ptr(k), _ptr(v), _ptr(q8), _ptr(k8), _ptr(v8t), _ptr(descale),
                                _ptr(amax_ws), _ptr(signs), float(scale), B, Hq, Hkv, Nq, Nk, d, _stream(stream)),
           "fa_fp8_prepare")


def fa_fwd_fp8(q8, k8, v8t, descale, o, lse, causal: bool, stream=None) -> None:
    """fp8 forward pass on codes from fa_fp8_prepare (which fixed the softmax scale) into o (bf16) and lse
    (fp32 or None)."""
    import torch
    B, Hq, Nq, d = q8.shape
    _, Hkv, Nk, _ = k8.shape
    if tuple(v8t.shape) != (B, Hkv, d, padded_keys(Nk)) or tuple(o.shape) != tuple(q8.shape):
        raise ValueError("shape mismatch")
    if o.dtype != torch.bfloat16:
        raise TypeError("o is bfloat16")
    if lse is not None and tuple(lse.shape) != (B, Hq, Nq):
        raise ValueError("lse must be [B, Hq, Nq]")
    for t in (q8, k8, v8t, descale, o) + ((lse,) if lse is not None else ()):
        if not t.is_cuda or not t.is_contiguous():
            raise ValueError("tensors must be contiguous GPU tensors")
    _check(lib().fa_fwd_fp8(_ptr(q8), _ptr(k8), _ptr(v8t), _ptr(descale), _ptr(o), _ptr(lse), B, Hq, Hkv, Nq, Nk,
                            d, int(bool(causal)), _stream(stream)), "fa_fwd_fp8")


def attention_fp8(q, k, v, causal: bool = False, scale: float | None = None, signs=None, stream=None):
    """Quantise bf16 q, k, v (optionally rotating q and k) and run the fp8 forward pass.

    Returns (o, lse, prep) with prep = dict(q8, k8, v8t, descale).
    """
    import torch
    B, Hq, Nq, d = q.shape
    _, Hkv, Nk, _ = k.shape
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    dev = q.device
    q8 = torch.empty(q.shape, dtype=torch.uint8, device=dev)
    k8 = torch.empty(k.shape, dtype=torch.uint8, device=dev)
    v8t = torch.empty((B, Hkv, d, padded_keys(Nk)), dtype=torch.uint8, device=dev)
    descale = torch.empty(3, dtype=torch.float32, device=dev)
    amax_ws = torch.empty(3, dtype=torch.int32, device=dev)
    fa_fp8_prepare(q, k, v, q8, k8, v8t, descale, amax_ws, signs, scale, stream)
    o = torch.empty(q.shape, dtype=torch.bfloat16, device=dev)
    lse = torch.empty((B, Hq, Nq), dtype=torch.float32, device=dev)
    fa_fwd_fp8(q8, k8, v8t, descale, o, lse, causal, stream)
    return o, lse, {"q8": q8, "k8": k8, "v8t": v8t, "descale": descale}


def splitkv_workspace_size(B, Hq, Hkv, Nq, Nk, d, causal: bool, nsplit: int = 0) -> int:
    """Bytes of workspace fa_fwd_splitkv needs for these arguments (0: none)."""
    return int(lib().fa_fwd_splitkv_workspace_size(B, Hq, Hkv, Nq, Nk, d, int(bool(causal)), nsplit))


def fa_fwd_splitkv(q, k, v, o, lse, scale: float, causal: bool, nsplit: int = 0, workspace=None, stream=None) -> None:
    """bf16 forward pass with the keys split into ranges (partials merged on the GPU)."""
    import torch
    B, Hq, Hkv, Nq, Nk, d = _shapes(q, k, v, o, lse)
    for t in (q, k, v, o):
        if t.dtype != torch.bfloat16:
            raise TypeError("fa_fwd_splitkv takes bfloat16 q, k, v, o")
    if lse is not None and lse.dtype != torch.float32:
        raise TypeError("lse must be float32")
    if workspace is not None and (not workspace.is_cuda or not workspace.is_contiguous()):
        raise ValueError("workspace must be a contiguous GPU tensor")
    nbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib().fa_fwd_splitkv(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), B, Hq, Hkv, Nq, Nk, d, float(scale),
                                int(bool(causal)), int(nsplit), _ptr(workspace), nbytes, _stream(stream)),
           "fa_fwd_splitkv")


def attention_splitkv(q, k, v, causal: bool = False, scale: float | None = None, nsplit: int = 0, stream=None):
    """Allocate o, lse and the workspace, run fa_fwd_splitkv, return (o, lse)."""
    import torch
    B, Hq, Nq, d = q.shape
    _, Hkv, Nk, _ = k.shape
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    o = torch.empty_like(q)
    lse = torch.empty((B, Hq, Nq), dtype=torch.float32, device=q.device)
    nbytes = splitkv_workspace_size(B, Hq, Hkv, Nq, Nk, d, causal, nsplit)
    ws = torch.empty((nbytes + 15) // 16 * 4, dtype=torch.float32, device=q.device) if nbytes else None
    fa_fwd_splitkv(q, k, v, o, lse, scale, causal, nsplit, ws, stream)
    return o, lse


def bwd_workspace_size(B, Hq, Hkv, Nq, Nk, d, causal: bool) -> int:
    """Bytes of workspace fa_bwd needs (0 for arguments it would reject)."""
    return int(lib().fa_bwd_workspace_size(B, Hq, Hkv, Nq, Nk, d, int(bool(causal))))


def _bwd_args(q, k, v, o, lse, do, dq, dk, dv, workspace):
    import torch
    B, Hq, Hkv, Nq, Nk, d = _shapes(q, k, v, o, lse)
    for t in (q, k, v, o, do, dq, dk, dv):
        if t.dtype != torch.bfloat16:
            raise TypeError("fa_bwd takes bfloat16 q, k, v, o, do, dq, dk, dv")
    if lse is None or lse.dtype != torch.float32:
        raise TypeError("lse must be a float32 tensor")
    if tuple(do.shape) != tuple(q.shape) or tuple(dq.shape) != tuple(q.shape):
        raise ValueError("do and dq must have q's shape")
    if tuple(dk.shape) != tuple(k.shape) or tuple(dv.shape) != tuple(k.shape):
        raise ValueError("dk and dv must have k's shape")
    for t in (do, dq, dk, dv):
        if not t.is_cuda or not t.is_contiguous():
            raise ValueError("tensors must be contiguous GPU tensors")
    if workspace is not None and (not workspace.is_cuda or not workspace.is_contiguous()):
        raise ValueError("workspace must be a contiguous GPU tensor")
    nbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    return (B, Hq, Hkv, Nq, Nk, d), nbytes


def fa_bwd(q, k, v, o, lse, do, dq, dk, dv, scale: float, causal: bool, workspace, stream=None) -> None:
    """bf16 backward pass: gradients into caller-allocated dq (q's shape), dk, dv (k's shape)."""
    dims, nbytes = _bwd_args(q, k, v, o, lse, do, dq, dk, dv, workspace)
    _check(lib().fa_bwd(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(do), _ptr(lse), _ptr(dq), _ptr(dk), _ptr(dv),
                        *dims, float(scale), int(bool(causal)), _ptr(workspace), nbytes, _stream(stream)), "fa_bwd")


def fa_bwd_dq(q, k, v, o, lse, do, dq, scale: float, causal: bool, workspace, stream=None) -> None:
    """First stage of fa_bwd: dq, and the per-row (LSE log2 e, D) pairs into the workspace."""
    dims, nbytes = _bwd_args(q, k, v, o, lse, do, dq, k, v, workspace)
    _check(lib().fa_bwd_dq(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(do), _ptr(lse), _ptr(dq), *dims, float(scale),
                           int(bool(causal)), _ptr(workspace), nbytes, _stream(stream)), "fa_bwd_dq")


def fa_bwd_dkdv(q, k, v, o, lse, do, dk, dv, scale: float, causal: bool, workspace, stream=None) -> None:
    """Second stage of fa_bwd: dk and dv from the pairs fa_bwd_dq left in the workspace, which also takes
    the partial sums when the heads of a group are split (o, lse: shape checks only)."""
    dims, nbytes = _bwd_args(q, k, v, o, lse, do, q, dk, dv, workspace)
    _check(lib().fa_bwd_dkdv(_ptr(q), _ptr(k), _ptr(v), _ptr(do), _ptr(dk), _ptr(dv), *dims, float(scale),
                             int(bool(causal)), _ptr(workspace), nbytes, _stream(stream)), "fa_bwd_dkdv")


def attention_backward(q, k, v, o, lse, do, causal: bool = False, scale: float | None = None, stream=None):
    """Allocate the gradients and the workspace, run fa_bwd, return (dq, dk, dv).

    o and lse are fa_fwd's outputs for the same q, k, v, causal and scale."""
    import torch
    B, Hq, Nq, d = q.shape
    _, Hkv, Nk, _ = k.shape
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    nbytes = bwd_workspace_size(B, Hq, Hkv, Nq, Nk, d, causal)
    ws = torch.empty((nbytes + 15) // 16 * 4, dtype=torch.float32, device=q.device)
    fa_bwd(q, k, v, o, lse, do, dq, dk, dv, scale, causal, ws, stream)
    return dq, dk, dv


def mfma_ceiling_out_bytes() -> int:
    """Bytes of device memory fa_mfma_ceiling's `out` must hold."""
    return int(lib().fa_mfma_ceiling_out_bytes())


def mfma_ceiling_flops(fp8: bool, iters: int) -> float:
    """Matrix flops of one fa_mfma_ceiling launch."""
    return float(lib().fa_mfma_ceiling_flops(int(bool(fp8)), int(iters)))


def mfma_ceiling(out, fp8: bool, iters: int, random: bool = True, stream=None) -> None:
    """Enqueue the MFMA-only loop (the measured ceiling) into `out` (a float32 GPU tensor)."""
    import torch
    if out.dtype != torch.float32 or not out.is_cuda or not out.is_contiguous():
        raise ValueError("out must be a contiguous float32 GPU tensor")
    _check(lib().fa_mfma_ceiling(_ptr(out), out.numel() * 4, int(bool(fp8)), int(iters), int(bool(random)),
                                 _stream(stream)), "fa_mfma_ceiling")


# matrix instruction of an issue-cost case, by the kind number fa.h gives
ISSUE_MFMA = ("bf16", "fp8", "fp8_scaled", "fp8_alternating")


def issue_cost_cases() -> list:
    """The issue-cost loop's cases: one dict of per-round counts (and the MFMA kind) per case."""
    L = lib()
    out = []
    for i in range(int(L.fa_issue_cost_cases())):
        c = [ctypes.c_int() for _ in range(4)]
        _check(L.fa_issue_cost_case(i, *[ctypes.byref(x) for x in c]), "fa_issue_cost_case")
        kind = ctypes.c_int()
        _check(L.fa_issue_cost_case_mfma(i, ctypes.byref(kind)), "fa_issue_cost_case_mfma")
        out.append(dict(zip(("mfmas", "exps", "cvts", "fmas"), (x.value for x in c)), mfma=ISSUE_MFMA[kind.value]))
    return out


def issue_cost(out, case: int, iters: int, stream=None) -> None:
    """Enqueue case `case` of the issue-cost loop into `out` (a float32 GPU tensor)."""
    import torch
    if out.dtype != torch.float32 or not out.is_cuda or not out.is_contiguous():
        raise ValueError("out must be a contiguous float32 GPU tensor")
    _check(lib().fa_issue_cost(_ptr(out), out.numel() * 4, int(case), int(iters), _stream(stream)), "fa_issue_cost")


def fa_fwd_splitkv_noalloc(q, k, v, o, lse, scale: float, causal: bool, nsplit: int = 0, stream=None) -> None:
    """fa_fwd_splitkv with the parts in the library's fixed per-GPU scratch (no workspace argument)."""
    import torch
    B, Hq, Hkv, Nq, Nk, d = _shapes(q, k, v, o, lse)
    for t in (q, k, v, o):
        if t.dtype != torch.bfloat16:
            raise TypeError("fa_fwd_splitkv_noalloc takes bfloat16 q, k, v, o")
    if lse is not None and lse.dtype != torch.float32:
        raise TypeError("lse must be float32")
    _check(lib().fa_fwd_splitkv_noalloc(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), B, Hq, Hkv, Nq, Nk, d,
                                        float(scale), int(bool(causal)), int(nsplit), _stream(stream)),
           "fa_fwd_splitkv_noalloc")
