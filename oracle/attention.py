"""Reference attention in fp64 (test infrastructure only; see package docstring).

Sources (the pages these functions restate):
  * "FlashAttention (SV)", section "Problematik med standard-attention": the
    result is softmax(Q K^T / sqrt(d_k)) V, and a naive implementation builds
    the whole N x N score matrix S.  attention_fp64 does exactly that on purpose.
  * "FlashAttention (SV)", section "Online-beräkning av Softmax": a running
    maximum and a running sum of exponentials, updated block by block, give the
    exact softmax.  online_fp64 follows that scheme.
  * "FlashAttention-4震撼发布" (first algorithmic improvement): the output
    rescaling is skipped most of the time.  online_fp64 models this with a
    threshold tau on the growth of the running maximum (log2 units).
  * "FlashAttention (SV)", section "Sammanslagning av operationer": masking is
    part of the computation; the causal reading used here is bottom-right
    aligned, key j visible to query i iff j <= i + (Nk - Nq).
  * "FlashAttention-4震撼发布" (FlashAttention-2 list): MQA and GQA; query head h
    reads key/value head h // (Hq // Hkv).
  * "FlashAttention (SV)", section "Online-beräkning av Softmax": softmax
    statistics of separate key blocks combine exactly, given each block's
    maximum and sum of exponentials.  attention_keys_fp64 and merge_fp64 use
    this for attention split over key ranges (each part keeps its own
    normalised output and log-sum-exp).
  * The pages report training results ("FlashAttention-4震撼发布",
    FlashAttention-2 list; "FlashAttention (SV)", section "Empiriska
    resultat") without a backward algorithm: attention_backward_fp64 is the
    gradient of the definition above, written out.

Layouts: q [B, Hq, Nq, d], k and v [B, Hkv, Nk, d]; outputs o [B, Hq, Nq, d]
(v may have its own last dimension, which o then has)
and lse [B, Hq, Nq] (natural log, scale included).  A row with no visible key
gets o = 0 and lse = -inf.
"""
from __future__ import annotations

import math
import numpy as np

LOG2E = 1.0 / math.log(2.0)


def kv_head_of(h_q: int, hq: int, hkv: int) -> int:
    """Contiguous GQA grouping: hq // hkv query heads share one key/value head."""
    if hq % hkv != 0:
        raise ValueError("Hq must be a multiple of Hkv")
    return h_q // (hq // hkv)


def _visible(nq: int, nk: int, causal: bool, q_pos=None) -> np.ndarray:
    """Boolean [len(q_pos), Nk] visibility mask (bottom-right causal alignment)."""
    if q_pos is None:
        q_pos = np.arange(nq)
    q_pos = np.asarray(q_pos, dtype=np.int64)
    if not causal:
        return np.ones((q_pos.size, nk), dtype=bool)
    j = np.arange(nk)[None, :]
    return j <= (q_pos[:, None] + (nk - nq))


def _softmax_rows(s: np.ndarray, vis: np.ndarray):
    """Two-pass softmax of score rows: returns P (materialised), row max m, row sum l."""
    s = np.where(vis, s, -np.inf)
    m = s.max(axis=1)
    m_safe = np.where(np.isfinite(m), m, 0.0)
    p = np.exp(s - m_safe[:, None])          # masked entries: exp(-inf) = 0
    l = p.sum(axis=1)
    return p, m, l


def attention_fp64(q, k, v, scale: float, causal: bool, return_p: bool = False):
    """The plain definition O = softmax(scale * Q K^T) V, evaluated in fp64.

    For every (b, h_q): pass 1 builds S = scale * Q K^T (masked to -inf where
    not visible) and its row maxima; pass 2 builds P = exp(S - m), its row sums
    l, then O = (P V) / l and LSE = m + ln l.  If return_p, also returns the
    list of normalised P matrices (P / l), one per (b, h_q), in loop order.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    B, HQ, NQ, _ = q.shape
    _, HKV, NK, _ = k.shape
    o = np.zeros((B, HQ, NQ, v.shape[-1]), dtype=np.float64)
    lse = np.full((B, HQ, NQ), -np.inf, dtype=np.float64)
    ps = []
    vis = _visible(NQ, NK, causal)
    for b in range(B):
        for h in range(HQ):
            hk = kv_head_of(h, HQ, HKV)
            s = scale * (q[b, h] @ k[b, hk].T)
            p, m, l = _softmax_rows(s, vis)
            live = l > 0
            o[b, h][live] = (p[live] @ v[b, hk]) / l[live][:, None]
            lse[b, h][live] = m[live] + np.log(l[live])
            if return_p:
                pn = np.zeros_like(p)
                pn[live] = p[live] / l[live][:, None]
                ps.append(pn)
    if return_p:
        return o, lse, ps
    return o, lse


def attention_rows_fp64(q, k, v, scale: float, causal: bool, rows):
    """The same definition restricted to query rows rows = [(b, h_q, i), ...].

    q may be any array-like indexable as q[b, h, i] (so a large tensor need not
    be converted whole); returns o [len(rows), d] and lse [len(rows)].
    """
    B, HQ, NQ, _ = q.shape
    _, HKV, NK, _ = k.shape
    o = np.zeros((len(rows), v.shape[-1]), dtype=np.float64)
    lse = np.full((len(rows),), -np.inf, dtype=np.float64)
    for r, (b, h, i) in enumerate(rows):
        hk = kv_head_of(int(h), HQ, HKV)
        qi = np.asarray(q[b, h, i], dtype=np.float64)
        kk = np.asarray(k[b, hk], dtype=np.float64)
        vv = np.asarray(v[b, hk], dtype=np.float64)
        s = scale * (kk @ qi)[None, :]
        p, m, l = _softmax_rows(s, _visible(NQ, NK, causal, [i]))
        if l[0] > 0:
            o[r] = (p[0] @ vv) / l[0]
            lse[r] = m[0] + math.log(l[0])
    return o, lse


def online_fp64(q, k, v, scale: float, causal: bool, bc: int, tau: float, group: int = 1):
    """Block-by-block online softmax (running max and exponent sum) in fp64.

    Keys are visited in ascending blocks of bc.  Scores are kept in log2 units
    (t = scale * log2(e) * q.k).  Each row keeps a reference maximum m_ref that
    the exponentials are taken against, a running sum l and an unnormalised
    output acc.  After a block, the running maximum m_new of a row may exceed
    m_ref; only when some row of the same group of `group` consecutive rows
    exceeds it by more than tau are the rows of that group rescaled
    (acc and l multiplied by 2^(m_ref - m_new), m_ref <- m_new).  The very
    first block a row sees sets its m_ref and is not counted.  With tau = 0
    this is the classic always-rescale scheme; for any tau the result is exact
    because acc and l carry the same factor.

    Returns o, lse, and (rescale_events, decisions): the number of (group,
    block) steps that rescaled and the number of steps that could have.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    B, HQ, NQ, _ = q.shape
    _, HKV, NK, _ = k.shape
    D = v.shape[-1]
    c = scale * LOG2E
    o = np.zeros((B, HQ, NQ, D))
    lse = np.full((B, HQ, NQ), -np.inf)
    events = 0
    decisions = 0
    vis_all = _visible(NQ, NK, causal)
    for b in range(B):
        for h in range(HQ):
            hk = kv_head_of(h, HQ, HKV)
            m_ref = np.full(NQ, -np.inf)
            m_run = np.full(NQ, -np.inf)
            l = np.zeros(NQ)
            acc = np.zeros((NQ, D))
            for j0 in range(0, NK, bc):
                j1 = min(NK, j0 + bc)
                t = c * (q[b, h] @ k[b, hk, j0:j1].T)
                t = np.where(vis_all[:, j0:j1], t, -np.inf)
                m_run = np.maximum(m_run, t.max(axis=1))
                for g0 in range(0, NQ, group):
                    g = slice(g0, min(NQ, g0 + group))
                    first = ~np.isfinite(m_ref[g]) & np.isfinite(m_run[g])
                    m_ref[g] = np.where(first, m_run[g], m_ref[g])
                    started = np.isfinite(m_ref[g])
                    if not started.any():
                        continue
                    grow = np.where(started & ~first, m_run[g] - m_ref[g], 0.0)
                    if (started & ~first).any():
                        decisions += 1
                        if (grow > tau).any():
                            events += 1
                            alpha = np.where(started, np.exp2(m_ref[g] - m_run[g]), 1.0)
                            acc[g] *= alpha[:, None]
                            l[g] *= alpha
                            m_ref[g] = np.where(started, m_run[g], m_ref[g])
                mr = np.where(np.isfinite(m_ref), m_ref, 0.0)
                p = np.exp2(t - mr[:, None])
                l += p.sum(axis=1)
                acc += p @ v[b, hk, j0:j1]
            live = l > 0
            o[b, h][live] = acc[live] / l[live][:, None]
            lse[b, h][live] = (m_ref[live] + np.log2(l[live])) / LOG2E
    return o, lse, (events, decisions)


def attention_keys_fp64(q, k, v, scale: float, causal: bool, k0: int, k1: int):
    """The definition over the keys [k0, k1) only, each key visible to a query
    exactly when it is in the full problem: o [B, Hq, Nq, d] normalised by the
    part's own sum, lse [B, Hq, Nq] of the part; a row that sees none of these
    keys gets o = 0 and lse = -inf."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    B, HQ, NQ, _ = q.shape
    _, HKV, NK, _ = k.shape
    if not 0 <= k0 <= k1 <= NK:
        raise ValueError("key range out of bounds")
    o = np.zeros((B, HQ, NQ, v.shape[-1]), dtype=np.float64)
    lse = np.full((B, HQ, NQ), -np.inf, dtype=np.float64)
    vis = _visible(NQ, NK, causal)[:, k0:k1]
    for b in range(B):
        for h in range(HQ):
            hk = kv_head_of(h, HQ, HKV)
            s = scale * (q[b, h] @ k[b, hk, k0:k1].T)
            p, m, l = _softmax_rows(s, vis)
            live = l > 0
            o[b, h][live] = (p[live] @ v[b, hk, k0:k1]) / l[live][:, None]
            lse[b, h][live] = m[live] + np.log(l[live])
    return o, lse


def merge_fp64(o_parts, lse_parts):
    """Combine attention over disjoint key sets: parts o_s (normalised by their
    own sums) and lse_s, stacked on axis 0.  With L = ln sum_s exp(lse_s):
    o = sum_s exp(lse_s - L) o_s and lse = L; rows where every part is -inf get
    o = 0 and lse = -inf."""
    o_parts = np.asarray(o_parts, dtype=np.float64)
    lse_parts = np.asarray(lse_parts, dtype=np.float64)
    m = lse_parts.max(axis=0)
    m_safe = np.where(np.isfinite(m), m, 0.0)
    w = np.exp(lse_parts - m_safe[None])          # -inf parts weigh 0
    tot = w.sum(axis=0)
    live = tot > 0
    lse = np.where(live, m_safe + np.log(np.where(live, tot, 1.0)), -np.inf)
    o = np.einsum("s...,s...d->...d", w, o_parts)
    o = np.where(live[..., None], o / np.where(live, tot, 1.0)[..., None], 0.0)
    return o, lse


def attention_backward_fp64(q, k, v, do, scale: float, causal: bool):
    """Gradients of the definition for an upstream gradient do = dL/dO.

    With P = softmax(S) (rows normalised, masked entries 0), O = P V:
      dV = P^T dO,  dP = dO V^T,  dS = P o (dP - D) with D_i = sum_j P_ij dP_ij
      (= sum_c dO_ic O_ic),  dQ = scale dS K,  dK = scale dS^T Q.
    GQA: the gradients of a key/value head sum over its query heads.  The
    pages print no backward algorithm; these are the derivatives of the
    definition they give ("FlashAttention (SV)", section "Problematik med
    standard-attention"), written out.  Returns (dq, dk, dv) in fp64.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    do = np.asarray(do, dtype=np.float64)
    B, HQ, NQ, _ = q.shape
    _, HKV, NK, _ = k.shape
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    vis = _visible(NQ, NK, causal)
    for b in range(B):
        for h in range(HQ):
            hk = kv_head_of(h, HQ, HKV)
            s = scale * (q[b, h] @ k[b, hk].T)
            p, m, l = _softmax_rows(s, vis)
            live = l > 0
            pn = np.zeros_like(p)
            pn[live] = p[live] / l[live][:, None]
            dv[b, hk] += pn.T @ do[b, h]
            dp = do[b, h] @ v[b, hk].T
            dd = (pn * dp).sum(axis=1, keepdims=True)
            ds = pn * (dp - dd)
            dq[b, h] = scale * (ds @ k[b, hk])
            dk[b, hk] += scale * (ds.T @ q[b, h])
    return dq, dk, dv
