"""CPU fp64 tiled online-softmax reference for the exact attention forward.

TEST INFRASTRUCTURE ONLY (same rules as oracle/attention.py: only tests, the
smoke check and the benchmark's CPU-baseline leg use it; no product code).

It runs the online-softmax recurrence of "Flash Attention"
(wiki.ai-engineering.at), section "Lösung: Online Softmax": the state starts as
running max m = -inf, running sum l = 0 and unnormalised output o = 0; each
block of keys updates

    m_new = max(m, rowmax(S_blk))
    l     = exp(m - m_new) * l + rowsum(exp(S_blk - m_new))
    o     = o * exp(m - m_new) + exp(S_blk - m_new) @ V_blk
    m     = m_new

The page stops there; the result it calls exact needs the final division
o / l (reading adopted: the only one under which the tiled result equals plain
attention, johe.ru "Почему это точно?").  A row that has seen only masked keys
so far still has m = -inf; its state is left untouched by such a block instead
of evaluating exp(-inf - (-inf)).

Block size and block order are free: the pages say the tile size follows the
hardware (ZimaSpace, section "Flash Attention teilt das Problem in
On-Chip-Arbeitssätze auf") and that only the order of computation differs from
plain attention (johe.ru, section "Почему это точно?").  This function runs any
block size (also ones that do not divide N) in any order; the tests use it to
check the recurrence itself against the plain definition.
"""
from __future__ import annotations

import numpy as np

__all__ = ["tiled_ref"]


def tiled_ref(q, k, v, causal: bool = False, scale: float | None = None,
              block: int = 64, order: str | list = "asc", seed: int = 0):
    """Online-softmax attention of one head in float64, processed in key blocks.

    order: "asc", "desc", "random" (seeded by ``seed``) or an explicit list of
    block indices.  Returns (o [Nq, Dv], lse [Nq]).
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    n_q, d = q.shape
    n_k = k.shape[0]
    if causal and n_q != n_k:
        raise ValueError("causal attention here needs as many queries as keys")
    if scale is None:
        scale = 1.0 / np.sqrt(d)
    n_blocks = (n_k + block - 1) // block
    if isinstance(order, str):
        if order == "asc":
            blocks = list(range(n_blocks))
        elif order == "desc":
            blocks = list(range(n_blocks))[::-1]
        elif order == "random":
            blocks = list(np.random.default_rng(seed).permutation(n_blocks))
        else:
            raise ValueError(order)
    else:
        blocks = list(order)

    m = np.full(n_q, -np.inf)
    l = np.zeros(n_q)
    o = np.zeros((n_q, v.shape[1]))
    qi = np.arange(n_q)[:, None]
    for j in blocks:
        j0, j1 = j * block, min(n_k, (j + 1) * block)
        s = scale * (q @ k[j0:j1].T)
        if causal:
            s[np.arange(j0, j1)[None, :] > qi] = -np.inf
        m_new = np.maximum(m, s.max(axis=1))
        live = np.isfinite(m_new)  # rows with at least one visible key so far
        m_safe = np.where(live, m_new, 0.0)
        alpha = np.where(live, np.exp(np.where(live, m, -np.inf) - m_safe), 1.0)
        e = np.where(live[:, None], np.exp(s - m_safe[:, None]), 0.0)
        l = alpha * l + e.sum(axis=1)
        o = o * alpha[:, None] + e @ v[j0:j1]
        m = m_new
    # the final division the page leaves implicit
    return o / l[:, None], m + np.log(l)
