"""Whole-tensor comparison of GPU outputs with the fp64 oracle, one (b, h) head
per task over a pool of host processes.

The oracle (oracle.attention_fp64: S and P materialised, two passes) runs
unchanged on one query head at a time; each task compares every element of
that head's GPU output with it and returns sums, so that the statistics of
the whole tensor (max and mean |dO|, max |dLSE|, cosine and RMSE over all
elements) are exact aggregates, not samples.

Test infrastructure: imported by the GPU parity tests only.
"""
from __future__ import annotations

import math
import multiprocessing as mp
import os

import numpy as np


def pool_size() -> int:
    """Worker processes: the host cores this process may use, at most 16."""
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def _init_worker():
    # one BLAS thread per worker: the pool supplies the parallelism
    try:
        from threadpoolctl import threadpool_limits
        threadpool_limits(1)
    except Exception:  # noqa: BLE001
        pass


def _decode(a):
    from oracle.formats import bf16_bits_to_f64
    return bf16_bits_to_f64(a) if a.dtype in (np.uint16, np.int16) else np.asarray(a, dtype=np.float64)


def _head_task(args):
    """Oracle of one head; statistics of every given output against it."""
    from oracle import attention_fp64
    q, k, v, scale, causal, outs = args
    o_ref, lse_ref = attention_fp64(_decode(q)[None, None], _decode(k)[None, None], _decode(v)[None, None],
                                    scale, causal)
    o_ref, lse_ref = o_ref[0, 0], lse_ref[0, 0]
    res = []
    for o_gpu, lse_gpu in outs:
        o = _decode(o_gpu)
        finite = bool(np.isfinite(o).all())
        e = o - o_ref
        ae = np.abs(e)
        st = {"n": o.size, "nonfinite": int((~np.isfinite(o)).sum()), "max_abs": float(ae.max()) if finite else math.inf,
              "sum_abs": float(ae.sum()), "sum_sq": float((e * e).sum()), "dot": float((o * o_ref).sum()),
              "sum_o2": float((o * o).sum()), "sum_r2": float((o_ref * o_ref).sum())}
        if lse_gpu is not None:
            lse = np.asarray(lse_gpu, dtype=np.float64)
            inf_ref = np.isneginf(lse_ref)
            st["lse_inf_mismatch"] = int((np.isneginf(lse) != inf_ref).sum())
            live = ~inf_ref
            st["lse_max_abs"] = float(np.abs(lse[live] - lse_ref[live]).max()) if live.any() else 0.0
        res.append(st)
    return res


def compare_all_heads(q, k, v, scale: float, causal: bool, outputs, workers: int | None = None):
    """Compare GPU outputs with the oracle on every element.

    q [B, Hq, Nq, d], k and v [B, Hkv, Nk, d]: the exact inputs the GPU
    consumed (bf16 bit patterns as uint16, or fp32/fp64 values).
    outputs: {name: (o [B, Hq, Nq, d] (bf16 bits or float), lse [B, Hq, Nq] or None)}.
    Returns {name: {"max_abs", "mean_abs", "rmse", "cosine", "lse_max_abs",
    "lse_inf_mismatch", "nonfinite", "n"}} over all elements.
    """
    B, Hq = q.shape[:2]
    Hkv = k.shape[1]
    g = Hq // Hkv
    names = list(outputs)
    tasks = []
    for b in range(B):
        for h in range(Hq):
            outs = []
            for nm in names:
                o, lse = outputs[nm]
                outs.append((np.ascontiguousarray(o[b, h]), None if lse is None else np.ascontiguousarray(lse[b, h])))
            tasks.append((np.ascontiguousarray(q[b, h]), np.ascontiguousarray(k[b, h // g]),
                          np.ascontiguousarray(v[b, h // g]), scale, causal, outs))
    workers = workers or pool_size()
    if workers == 1:
        per_head = [_head_task(t) for t in tasks]
    else:
        # spawn: the workers start clean, without the parent's GPU runtime state
        with mp.get_context("spawn").Pool(workers, initializer=_init_worker) as pool:
            per_head = pool.map(_head_task, tasks, chunksize=1)
    out = {}
    for i, nm in enumerate(names):
        sts = [ph[i] for ph in per_head]
        n = sum(s["n"] for s in sts)
        dot, so2, sr2 = (sum(s[f] for s in sts) for f in ("dot", "sum_o2", "sum_r2"))
        agg = {"n": n, "nonfinite": sum(s["nonfinite"] for s in sts),
               "max_abs": max(s["max_abs"] for s in sts), "mean_abs": sum(s["sum_abs"] for s in sts) / n,
               "rmse": math.sqrt(sum(s["sum_sq"] for s in sts) / n),
               "cosine": dot / math.sqrt(so2 * sr2) if so2 > 0 and sr2 > 0 else float("nan")}
        if "lse_max_abs" in sts[0]:
            agg["lse_max_abs"] = max(s["lse_max_abs"] for s in sts)
            agg["lse_inf_mismatch"] = sum(s["lse_inf_mismatch"] for s in sts)
        out[nm] = agg
    return out


def _stats(o, r):
    e = o - r
    return np.array([(o * r).sum(), (o * o).sum(), (r * r).sum(), (e * e).sum(), np.abs(e).sum(), np.abs(e).max(),
                     float((~np.isfinite(o)).sum())])


def _fp8_head_task(args):
    """Oracle on the unquantised source and on the dequantised codes of each
    run, for one head; statistics of each run's GPU output against both, and
    of the dequantised oracle against the source oracle."""
    from oracle import attention_fp64
    from oracle.formats import e4m3_decode
    q, k, v, scale, runs = args
    o_true, _ = attention_fp64(_decode(q)[None, None], _decode(k)[None, None], _decode(v)[None, None], scale, False)
    o_true = o_true[0, 0]
    res = []
    for o_gpu, q8, k8, v8, sc in runs:
        qq, kk, vv = (e4m3_decode(c) * s for c, s in zip((q8, k8, v8), sc))
        o_deq, _ = attention_fp64(qq[None, None], kk[None, None], vv[None, None], scale, False)
        o_deq = o_deq[0, 0]
        o = _decode(o_gpu)
        res.append({"gpu_true": _stats(o, o_true), "gpu_deq": _stats(o, o_deq), "deq_true": _stats(o_deq, o_true)})
    return res


def _agg(rows, n):
    t = sum(rows)
    return {"cosine": float(t[0] / math.sqrt(t[1] * t[2])) if t[1] > 0 and t[2] > 0 else float("nan"),
            "rmse": math.sqrt(t[3] / n), "mean_abs": float(t[4] / n), "max_abs": float(max(r[5] for r in rows)),
            "nonfinite": int(t[6]), "n": n}


def compare_fp8_all_heads(q, k, v, scale: float, runs, workers: int | None = None):
    """Non-causal fp8 attention outputs against the fp64 oracle on every element.

    q, k, v: the bf16 source (uint16 bit patterns), [B, H, N, d] (MHA).
    runs: {name: (o [B, H, N, d] bf16 bits, q8, k8, v8 (e4m3 codes; v8 in
    [B, Hkv, Nk, d] key order), (s_q, s_k, s_v))}, each tensor represented
    by s * decode(code) (for Q codes that carry a factor c0, s_q / c0).
    Returns {name: {"gpu_true", "gpu_deq", "deq_true"}}, each with cosine,
    rmse, mean_abs, max_abs over all elements: the GPU output against the
    oracle on the source (the accuracy of the fp8 path), against the oracle on
    the dequantised codes (the kernel's own error), and the dequantised oracle
    against the source oracle (the error of the format alone).
    """
    B, H = q.shape[:2]
    Hkv = k.shape[1]
    g = H // Hkv
    names = list(runs)
    tasks = []
    for b in range(B):
        for h in range(H):
            hk = h // g
            rr = []
            for nm in names:
                o, q8, k8, v8, sc = runs[nm]
                rr.append((np.ascontiguousarray(o[b, h]), np.ascontiguousarray(q8[b, h]),
                           np.ascontiguousarray(k8[b, hk]), np.ascontiguousarray(v8[b, hk]), tuple(map(float, sc))))
            tasks.append((np.ascontiguousarray(q[b, h]), np.ascontiguousarray(k[b, hk]), np.ascontiguousarray(v[b, hk]),
                          scale, rr))
    workers = workers or pool_size()
    if workers == 1:
        per_head = [_fp8_head_task(t) for t in tasks]
    else:
        with mp.get_context("spawn").Pool(workers, initializer=_init_worker) as pool:
            per_head = pool.map(_fp8_head_task, tasks, chunksize=1)
    n = q[..., 0].size * runs[names[0]][0].shape[-1]
    return {nm: {key: _agg([ph[i][key] for ph in per_head], n) for key in ("gpu_true", "gpu_deq", "deq_true")}
            for i, nm in enumerate(names)}
