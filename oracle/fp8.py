"""FP8 "incoherent processing" step in fp64 (test infrastructure only).

Restates "FlashAttention-3 — 闪电注意力-3", section on low precision (FP8) and
quantisation error: before quantisation Q and K are multiplied by a random
orthogonal matrix, for example a Hadamard matrix; the rotation spreads
outliers over all channels, and because the matrix is orthogonal the product
Q K^T is unchanged.

Readings where the page is silent:
  * matrix: M = diag(signs) * H_d / sqrt(d) with H_d the Sylvester Hadamard
    matrix (H_1 = [1], H_2n = [[H, H], [H, -H]]) and signs in {+1, -1}^d drawn
    by the caller; applied on the right, x -> x M, to Q and K only (V is not
    rotated); signs = None means no rotation.
  * the softmax scale is folded into the query codes: the quantised query
    is x = c0 * (rotated Q) with c0 = softmax scale * log2(e), so that the
    products of the codes are scores in base-2 units (the attention
    computes exp(scale * s) as 2^(c0 * s)).
  * scales: one per tensor.  For Q and K the smallest power of two s with
    amax(|x|) / s <= 448 over the whole (rotated) tensor; for V
    s = amax(|x|) / 448.  s = 1 if the tensor is all zero;
    codes = e4m3_rne(x / s).  In a floating-point format a scale chosen
    anywhere within a factor of two gives every code the same relative
    precision; a power of two lets the product of two scales be applied
    exactly.
  * V is stored transposed, [B][Hkv][d][Nk].
"""
from __future__ import annotations

import math

import numpy as np

from .formats import E4M3_MAX, e4m3_decode, e4m3_encode_rne


def sylvester_hadamard(n: int) -> np.ndarray:
    """Integer Sylvester Hadamard matrix of order n (a power of two)."""
    if n < 1 or n & (n - 1):
        raise ValueError("order must be a power of two")
    h = np.ones((1, 1), dtype=np.int64)
    while h.shape[0] < n:
        h = np.block([[h, h], [h, -h]])
    return h


def rotation(signs) -> np.ndarray:
    """The orthogonal matrix diag(signs) * H_d / sqrt(d), fp64."""
    s = np.asarray(signs, dtype=np.float64)
    d = s.size
    return (s[:, None] * sylvester_hadamard(d)) / np.sqrt(d)


def quantise(x, pow2: bool = False) -> tuple[np.ndarray, float]:
    """Per-tensor e4m3 quantisation: returns (codes, scale) with x ~ scale * decode(codes).

    scale = amax|x| / 448, or with pow2 the smallest power of two that is
    not below it; 1 for an all-zero tensor."""
    x = np.asarray(x, dtype=np.float64)
    amax = float(np.max(np.abs(x))) if x.size else 0.0
    if not amax > 0:
        s = 1.0
    elif pow2:
        m, e = math.frexp(amax / E4M3_MAX)       # amax / 448 = m * 2^e, 0.5 <= m < 1
        s = math.ldexp(1.0, e - 1 if m == 0.5 else e)
    else:
        s = amax / E4M3_MAX
    return e4m3_encode_rne(x / s), s


def prepare(q, k, v, signs=None, scale: float | None = None) -> dict:
    """Rotate Q and K (if signs is given), fold c0 = scale * log2(e) into Q,
    quantise Q, K, V per tensor, transpose V.

    q [B,Hq,Nq,d], k and v [B,Hkv,Nk,d] (fp64 values); scale defaults to
    1/sqrt(d).  Returns a dict with q8, k8 (uint8 codes, same layouts), v8t
    (uint8 codes [B,Hkv,d,Nk]), scales (s_q, s_k, s_v), c0 and the rotated
    fp64 tensors qr, kr (qr without c0).
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    if signs is not None:
        m = rotation(signs)
        qr, kr = q @ m, k @ m
    else:
        qr, kr = q, k
    if scale is None:
        scale = 1.0 / math.sqrt(q.shape[-1])
    c0 = scale * math.log2(math.e)
    q8, sq = quantise(c0 * qr, pow2=True)
    k8, sk = quantise(kr, pow2=True)
    v8, sv = quantise(v)
    return {
        "q8": q8, "k8": k8, "v8t": np.ascontiguousarray(np.swapaxes(v8, 2, 3)),
        "scales": (sq, sk, sv), "c0": c0, "qr": qr, "kr": kr,
    }


def dequantised(prep: dict):
    """fp64 tensors (q, k, v) the quantised codes stand for (q without c0), V back in [B,Hkv,Nk,d]."""
    sq, sk, sv = prep["scales"]
    q = e4m3_decode(prep["q8"]) * sq / prep["c0"]
    k = e4m3_decode(prep["k8"]) * sk
    v = np.swapaxes(e4m3_decode(prep["v8t"]) * sv, 2, 3)
    return q, k, v
