"""CPU fp64 oracle for the gradients of the exact attention forward.

TEST INFRASTRUCTURE ONLY (same rules as oracle/attention.py: only tests, the
smoke check and the benchmark's CPU-baseline leg use it; no product code).

The pages say only that a second pass computes the gradients over the same
chunks, in reverse order, without storing the score matrix ("Flash Attention:
ускорить attention в 6 раз без потери точности", johe.ru, section "Стадии
вычисления", the second pass).  The gradients themselves follow from the
forward definition (oracle/attention.py) by the chain rule; with an upstream
gradient dO of the output O (LSE receives no gradient), per head:

  1. P = softmax over visible keys of s = scale * Q K^T (masked keys weigh 0),
     O = P V;
  2. dV = P^T dO                          (O is linear in V);
  3. dP = dO V^T                          (the same product, for the weights);
  4. Delta_i = sum_j P_ij dP_ij = sum_d dO_id O_id;
  5. dS = P * (dP - Delta)                (the softmax Jacobian, row by row:
                                            d p_j / d s_k = p_j (1[j=k] - p_k));
  6. dQ = scale * dS K,  dK = scale * dS^T Q   (s is bilinear in Q and K).

Everything is float64 matrix algebra on one head; masked entries of P are 0,
so they contribute nothing to dS, dQ or dK.
"""
from __future__ import annotations

import numpy as np

from .attention import attention_ref

__all__ = ["attention_bwd_ref"]


def attention_bwd_ref(q, k, v, do, causal: bool = False, scale: float | None = None):
    """Gradients (dq [Nq, D], dk [Nk, D], dv [Nk, Dv]) of attention_ref's output o
    with respect to q, k, v, for the upstream gradient do [Nq, Dv]; float64."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    do = np.asarray(do, dtype=np.float64)
    if scale is None:
        scale = 1.0 / np.sqrt(q.shape[1])
    scale = float(scale)
    if do.shape != (q.shape[0], v.shape[1]):
        raise ValueError("do must have the shape of the output [Nq, Dv]")
    # step 1: the forward's normalised weights and output
    o, _, p = attention_ref(q, k, v, causal, scale, return_p=True)
    # steps 2-3
    dv = p.T @ do
    dp = do @ v.T
    # step 4
    delta = np.sum(do * o, axis=1)
    # step 5
    ds = p * (dp - delta[:, None])
    # step 6
    dq = scale * (ds @ k)
    dk = scale * (ds.T @ q)
    return dq, dk, dv
