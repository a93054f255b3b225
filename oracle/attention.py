"""CPU fp64 oracle for the exact attention forward.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or run
this file: only the tests, the smoke check and the benchmark's CPU-baseline leg
use it.  It shares no code with the HIP library and imports nothing but numpy.

What it computes.  The pages define attention as a softmax over the key axis of
the scaled query-key dot products, applied as weights to the value rows
("Flash Attention", wiki.ai-engineering.at, section "Das Grundproblem";
"Flash Attention: ускорить attention в 6 раз без потери точности", johe.ru,
sections "Введение: проблема attention" and "Проблема 1: O(n²) промежуточная
память").  The tiled method is claimed to reach the same result as that plain
definition, up to the rounding of the input precision (johe.ru, section
"Почему это точно?"; ZimaSpace, "Wie reduziert Flash Attention den
Speicherverkehr während der lokalen Inferenz?", section "Flash Attention teilt
das Problem in On-Chip-Arbeitssätze auf").  So the oracle is the plain
definition, written out per query row in float64:

  1. visible keys J(i): all keys, or keys j <= i + (Nk - Nq) under the causal
     mask (the pages only name masking, ZimaSpace section "Kernel-Fusion hält
     mehr Schritte der Attention-Kette in einem Ausführungspfad"; the causal
     reading is key j visible to query i iff j <= i when there are as many
     queries as keys, and, with fewer queries than keys, the queries are the
     last Nq positions of the sequence, as when new tokens attend to a kept
     KV cache (ZimaSpace, section "Weniger IO bedeutet nicht, dass der
     KV-Cache entfällt"));
  2. scores s_ij = scale * sum_d q_id k_jd (contraction over the head dim);
  3. m_i = max_j s_ij over J(i) (the max subtraction of the online-softmax
     section keeps exp finite and does not change the softmax);
  4. p_ij = exp(s_ij - m_i), l_i = sum_j p_ij over J(i);
  5. o_i = sum_j (p_ij / l_i) v_j;
  6. lse_i = m_i + ln l_i, the natural log-sum-exp of the scaled scores
     (not on the pages; it is the per-row statistic the kernel also returns).

Rows are batched into matrix products of independent rows; each row's max,
exp, sum and division involve that row alone, so batching does not change the
definition.
"""
from __future__ import annotations

import numpy as np

__all__ = ["attention_ref", "attention_ref_bhnd", "merge_ref"]


def _rows_per_chunk(n_keys: int) -> int:
    return int(max(1, min(256, (1 << 23) // max(1, n_keys))))


def attention_ref(q, k, v, causal: bool = False, scale: float | None = None,
                  rows=None, return_p: bool = False):
    """Exact attention of one head in float64.

    q: [Nq, D] queries, k: [Nk, D] keys, v: [Nk, Dv] values (any real dtype;
    widened exactly to float64).  With causal=True, Nq must not exceed Nk and
    key j is visible to query i iff j <= i + (Nk - Nq).  ``rows`` selects a
    subset of query rows (default: all).  scale defaults to 1/sqrt(D).

    Returns (o [R, Dv], lse [R]) in float64, and the normalised weights
    p [R, Nk] as a third value when return_p is set.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    if q.ndim != 2 or k.ndim != 2 or v.ndim != 2:
        raise ValueError("q, k, v must be 2-D [rows, dim]")
    if q.shape[1] != k.shape[1] or k.shape[0] != v.shape[0]:
        raise ValueError("shape mismatch")
    n_q, d = q.shape
    n_k = k.shape[0]
    if causal and n_q > n_k:
        raise ValueError("causal attention needs at least as many keys as queries")
    if scale is None:
        scale = 1.0 / np.sqrt(d)
    scale = float(scale)
    rows = np.arange(n_q, dtype=np.int64) if rows is None else np.asarray(rows, dtype=np.int64)

    o = np.empty((rows.size, v.shape[1]), dtype=np.float64)
    lse = np.empty(rows.size, dtype=np.float64)
    p_all = np.empty((rows.size, n_k), dtype=np.float64) if return_p else None
    key_idx = np.arange(n_k, dtype=np.int64)
    step = _rows_per_chunk(n_k)
    for c0 in range(0, rows.size, step):
        r = rows[c0:c0 + step]
        # step 2: scores, contracting q and k over the head dimension
        s = scale * (q[r] @ k.T)
        # step 1: keys outside J(i) take no part in max, sum or output
        if causal:
            s[key_idx[None, :] > r[:, None] + (n_k - n_q)] = -np.inf
        # step 3
        m = s.max(axis=1)
        # step 4
        p = np.exp(s - m[:, None])
        l = p.sum(axis=1)
        # step 5
        o[c0:c0 + step] = (p @ v) / l[:, None]
        # step 6
        lse[c0:c0 + step] = m + np.log(l)
        if return_p:
            p_all[c0:c0 + step] = p / l[:, None]
    if return_p:
        return o, lse, p_all
    return o, lse


def attention_ref_bhnd(q, k, v, causal: bool = False, scale: float | None = None):
    """attention_ref applied to every (b, h) of [B, H, N, D] arrays.

    Returns (o [B, H, N, D], lse [B, H, N]) in float64.
    """
    q = np.asarray(q)
    k = np.asarray(k)
    v = np.asarray(v)
    B, H, N, _ = q.shape
    o = np.empty(q.shape[:3] + (v.shape[3],), dtype=np.float64)
    lse = np.empty((B, H, N), dtype=np.float64)
    for b in range(B):
        for h in range(H):
            o[b, h], lse[b, h] = attention_ref(q[b, h], k[b, h], v[b, h], causal, scale)
    return o, lse


def merge_ref(o_parts, lse_parts):
    """Attention over a union of disjoint key sets from the results over each set.

    o_parts: [S, R, Dv] normalised outputs of the S parts, lse_parts: [S, R]
    their log-sum-exps (-inf for a part in which a row sees no key).  Returns
    (o [R, Dv], lse [R]) in float64.

    The online-softmax update of "Flash Attention" (wiki.ai-engineering.at,
    section "Lösung: Online Softmax") folds one block of keys into the running
    (max, sum, output) of the keys seen so far; applied to the summaries of
    whole parts it is the merge.  Written with lse_s = m_s + ln l_s and the
    normalised o_s = (unnormalised o_s) / l_s:
        lse = ln sum_s exp(lse_s)
        o   = sum_s exp(lse_s - lse) o_s
    The maximum of the lse_s is subtracted before exponentiating, as in the
    online-softmax section, so nothing overflows.
    """
    o_parts = np.asarray(o_parts, dtype=np.float64)
    lse_parts = np.asarray(lse_parts, dtype=np.float64)
    if o_parts.ndim != 3 or lse_parts.shape != o_parts.shape[:2]:
        raise ValueError("o_parts [S, R, Dv] and lse_parts [S, R] expected")
    m = lse_parts.max(axis=0)
    if not np.all(np.isfinite(m)):
        raise ValueError("every row needs at least one part with a visible key")
    seen = np.isfinite(lse_parts)
    w = np.where(seen, np.exp(np.where(seen, lse_parts, 0.0) - m[None, :]), 0.0)
    o_parts = np.where(seen[:, :, None], o_parts, 0.0)   # a part without keys adds nothing
    tot = w.sum(axis=0)
    lse = m + np.log(tot)
    o = np.einsum("sr,srd->rd", w / tot[None, :], o_parts)
    return o, lse
