"""Seeded synthetic inputs for the attention forward pass.

This module only draws random numbers and encodes them (fp32 -> bf16 bit
patterns); it holds none of the attention arithmetic.  Both the HIP path and
the fp64 oracle consume what it returns.

Every tensor comes from its own numpy Generator seeded with
SeedSequence([config_or_seed, tensor_id]); tensor ids: Q=0, K=1, V=2,
outlier channels=3, Q outliers=4, K outliers=5, Hadamard signs=6, the
upstream gradient dO of the backward pass=7.  Values are
standard normal fp32, rounded to bf16 (nearest, ties to even) unless the
tensor dtype is fp32.

The five standing workloads (shapes of the FlashAttention pages' use cases:
a tiny single head, a GPT-2-small layer at 1K tokens, a Llama-style GQA long
context, a head dimension of 256, and FP8 with outliers):
  1  B=1  H=1        N=128   d=64   fp32, scale 1/8, non-causal
  2  B=8  H=12       N=1024  d=64   bf16, causal
  3  B=2  Hq=32 Hkv=8 N=8192 d=128  bf16, causal
  4  B=4  H=16       N=4096  d=256  bf16, non-causal, 0.5% of channels of Q and K x8
  5  B=4  H=16       N=8192  d=128  bf16 source for FP8 (e4m3), non-causal,
                                     Q and K entries set to +-50 with probability 0.001
"""
from __future__ import annotations

import math
from dataclasses import dataclass

import numpy as np

TID_Q, TID_K, TID_V, TID_CHANNELS, TID_QOUT, TID_KOUT, TID_SIGNS, TID_DO = range(8)


@dataclass(frozen=True)
class Workload:
    name: str
    B: int
    Hq: int
    Hkv: int
    Nq: int
    Nk: int
    d: int
    dtype: str            # "f32", "bf16" or "fp8" (bf16 source quantised to e4m3)
    causal: bool
    outlier_channel_frac: float = 0.0   # fraction of feature channels of Q and K scaled by outlier_factor
    outlier_factor: float = 8.0
    outlier_prob: float = 0.0           # per-entry probability that a Q/K entry is set to +-outlier_value
    outlier_value: float = 50.0
    scale: float | None = None          # None -> 1/sqrt(d)

    @property
    def softmax_scale(self) -> float:
        return self.scale if self.scale is not None else 1.0 / math.sqrt(self.d)

    def flops(self) -> float:
        """4*B*Hq*Nq*Nk*d, halved when causal."""
        f = 4.0 * self.B * self.Hq * self.Nq * self.Nk * self.d
        return f / 2 if self.causal else f


CONFIGS = {
    1: Workload("tiny single head B1 H1 N128 d64 fp32", 1, 1, 1, 128, 128, 64, "f32", False, scale=1.0 / 8.0),
    2: Workload("GPT-2-small causal B8 H12 N1024 d64 bf16", 8, 12, 12, 1024, 1024, 64, "bf16", True),
    3: Workload("GQA causal B2 Hq32 Hkv8 N8192 d128 bf16", 2, 32, 8, 8192, 8192, 128, "bf16", True),
    4: Workload("outlier channels B4 H16 N4096 d256 bf16", 4, 16, 16, 4096, 4096, 256, "bf16", False,
                outlier_channel_frac=0.005),
    5: Workload("fp8 e4m3 Hadamard B4 H16 N8192 d128", 4, 16, 16, 8192, 8192, 128, "fp8", False,
                outlier_prob=0.001),
}


def _rng(seed_key, tid):
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence(list(seed_key) + [tid])))


def f32_to_bf16_bits(x) -> np.ndarray:
    """Round fp32 values to bf16 (nearest, ties to even); returns uint16 bit patterns."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    r = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return r.astype(np.uint16)


def _normal(seed_key, tid, shape):
    return _rng(seed_key, tid).standard_normal(size=shape, dtype=np.float32)


def make_inputs(w: Workload, seed_key=(0,)) -> dict:
    """Draw q, k, v for workload w.

    Returns {"q","k","v"}: uint16 bf16 bit patterns for bf16/fp8 workloads,
    float32 arrays for f32; plus "signs" (float32 +-1, length d) for fp8 and
    "outlier_channels" (int array) when channels were scaled.
    """
    qs = (w.B, w.Hq, w.Nq, w.d)
    ks = (w.B, w.Hkv, w.Nk, w.d)
    q = _normal(seed_key, TID_Q, qs)
    k = _normal(seed_key, TID_K, ks)
    v = _normal(seed_key, TID_V, ks)
    out = {}
    if w.outlier_channel_frac > 0:
        n_out = max(1, int(round(w.outlier_channel_frac * w.d)))
        ch = np.sort(_rng(seed_key, TID_CHANNELS).choice(w.d, size=n_out, replace=False))
        q[..., ch] *= np.float32(w.outlier_factor)
        k[..., ch] *= np.float32(w.outlier_factor)
        out["outlier_channels"] = ch
    if w.outlier_prob > 0:
        for t, tid in ((q, TID_QOUT), (k, TID_KOUT)):
            g = _rng(seed_key, tid)
            hit = g.random(size=t.shape, dtype=np.float32) < w.outlier_prob
            sign = g.integers(0, 2, size=int(hit.sum()), dtype=np.int8) * 2 - 1
            t[hit] = sign.astype(np.float32) * np.float32(w.outlier_value)
    if w.dtype == "fp8":
        out["signs"] = (_rng(seed_key, TID_SIGNS).integers(0, 2, size=w.d) * 2 - 1).astype(np.float32)
    if w.dtype == "f32":
        out.update(q=q, k=k, v=v)
    else:
        out.update(q=f32_to_bf16_bits(q), k=f32_to_bf16_bits(k), v=f32_to_bf16_bits(v))
    return out


def make_dout(w: Workload, seed_key=(0,)) -> np.ndarray:
    """Upstream gradient dL/dO for the backward pass: standard normal, q's
    shape, as bf16 bit patterns (uint16)."""
    return f32_to_bf16_bits(_normal(seed_key, TID_DO, (w.B, w.Hq, w.Nq, w.d)))


# A decoding step of a GQA model over a long context (one new query per
# sequence): the workload of the key-split path.  Tensor ids as above, seed
# key (6,).
DECODE = Workload("GQA decode B8 Hq32 Hkv8 Nq1 Nk32768 d128 bf16", 8, 32, 8, 1, 32768, 128, "bf16", True)


def make_config(cfg, seed: int | None = None) -> tuple[Workload, dict]:
    """Inputs of standing workload cfg (1..5, or "decode"); seed None reproduces the standing draw."""
    w = DECODE if cfg == "decode" else CONFIGS[cfg]
    cid = 6 if cfg == "decode" else cfg
    key = (cid,) if seed is None else (cid, seed)
    return w, make_inputs(w, key)


def workload(B, Hq, Hkv, Nq, Nk, d, dtype="bf16", causal=False, **kw) -> Workload:
    """An ad-hoc workload (tests of edge cases and ragged shapes)."""
    return Workload(f"B{B} Hq{Hq} Hkv{Hkv} Nq{Nq} Nk{Nk} d{d} {dtype}{' causal' if causal else ''}",
                    B, Hq, Hkv, Nq, Nk, d, dtype, causal, **kw)
