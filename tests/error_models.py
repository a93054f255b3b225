"""Error bounds of the GPU path, written from its arithmetic and evaluated in
float64 from the inputs alone (never from a device result).

Each function bounds |device - oracle| element by element for one head.  The
bounds are first order in the unit roundoff u of the 16-bit type (bf16:
2^-8, fp16: 2^-11): every rounding the kernels perform is a relative error of
at most u on the rounded quantity, and the error of each output is the sum of
those errors carried through the linear algebra that follows them.  The fp32
accumulations of the matrix instructions (unit roundoff 2^-24) are far below
these terms and are covered by the factor KAPPA = 2 the tests apply.

A rounding to the 16-bit type errs by at most u |x| + ETA, the absolute part
for the smallest values: ETA = 2^-126 for bf16 (the kernels' fp32 arithmetic
flushes results below fp32's smallest normal, 2^-126, to zero, and bf16 has
fp32's exponent range), and 2^-25 for fp16 (half the spacing of its
subnormals, where tiny weights and dS entries fall).

Backward (the exact derivatives of O, as oracle.attention_bwd_ref defines
them; dV = P^T dO, dP = dO V^T, Delta = rowsum(dO * O), dS = P * (dP - Delta),
dQ = scale dS K, dK = scale dS^T Q).  The kernels round to the 16-bit type:
  * P, as the operand of dV = P^T dO                 -> u * P^T |dO|
  * O, stored by the forward and read for Delta      -> |dDelta_i| <= u A_i,
    A_i = 2 sum_d |dO_id| (P|V|)_id (the forward's O carries at most its own
    rounding and that of the weights it summed: 2u (P|V|))
  * dS, as the operand of dQ and dK                  -> u |dS| + u P A  (with
    the Delta error carried through dS = P (dP - Delta))
  * the stored gradients                             -> u |g|
so, with S = u (|dS| + diag(A) P) + ETA M (M: 1 on visible pairs, else 0):
  |ddQ| <= |scale| S |K| + u |dQ| + ETA,   |ddK| <= |scale| S^T |Q| + u |dK| + ETA,
  |ddV| <= (u P + ETA M)^T |dO| + u |dV| + ETA.

FP8 forward (E4M3 inputs with MX block scales, compared with the exact
attention of the values they denote).  Beyond the bf16 contract, which covers
P and O rounded to bf16: the scaled FP8 matrix instruction's sums are not
specified to fp32 accuracy, and a score error e moves the row's weights by a
relative 2|e| at most, O by 2|e| max|v| and LSE by |e|.  Assumption (stated,
not fitted): each 64-product sum of the instruction is accurate to
EPS_FP8 = 2^-10 of the sum of its products' magnitudes, so score (i, j) carries
at most E_ij = EPS_FP8 |scale| sum_d |q_id k_jd|.  Per row, E_i = max over the
visible keys; the bounds are the bf16 ones plus 2 E_i max_j |v_jd| (O) and E_i
(LSE).
"""
from __future__ import annotations

import numpy as np

from oracle import attention_ref

KAPPA = 2.0
U16 = {"bf16": 2.0 ** -8, "f16": 2.0 ** -11}
ETA16 = {"bf16": 2.0 ** -126, "f16": 2.0 ** -25}
EPS_FP8 = 2.0 ** -10


def _visible(nq: int, nk: int, causal: bool):
    if not causal:
        return None
    i = np.arange(nq)[:, None] + (nk - nq)
    return np.arange(nk)[None, :] <= i


def backward_bounds(q, k, v, do, causal: bool, scale: float, dtype: str):
    """Element-wise bounds (bq, bk, bv) on |dq|, |dk|, |dv| errors of one head
    (before the factor KAPPA)."""
    u, eta = U16[dtype], ETA16[dtype]
    q, k, v, do = (np.asarray(x, dtype=np.float64) for x in (q, k, v, do))
    o, _, p = attention_ref(q, k, v, causal, scale, return_p=True)
    vis = _visible(q.shape[0], k.shape[0], causal)
    m = np.ones_like(p) if vis is None else vis.astype(np.float64)
    dp = do @ v.T
    delta = np.sum(do * o, axis=1)
    ds = p * (dp - delta[:, None])
    dq = scale * (ds @ k)
    dk = scale * (ds.T @ q)
    dv = p.T @ do
    a = 2.0 * np.sum(np.abs(do) * (p @ np.abs(v)), axis=1)
    s = u * (np.abs(ds) + a[:, None] * p) + eta * m
    sc = abs(float(scale))
    bq = sc * (s @ np.abs(k)) + u * np.abs(dq) + eta
    bk = sc * (s.T @ np.abs(q)) + u * np.abs(dk) + eta
    bv = (u * p + eta * m).T @ np.abs(do) + u * np.abs(dv) + eta
    return bq, bk, bv


def fp8_row_terms(qd, kd, vd, causal: bool, scale: float, rows=None):
    """Per query row: the score-error bound E_i and the O term 2 E_i max_j|v_jd|
    ([rows, D]) of the FP8 forward (dequantised inputs, float64)."""
    qd, kd, vd = (np.asarray(x, dtype=np.float64) for x in (qd, kd, vd))
    if rows is not None:
        qsel = qd[rows]
    else:
        rows = np.arange(qd.shape[0])
        qsel = qd
    mag = np.abs(qsel) @ np.abs(kd).T  # sum_d |q_id k_jd|
    vis = _visible(qd.shape[0], kd.shape[0], causal)
    if vis is not None:
        mag = np.where(vis[rows], mag, 0.0)
    e = EPS_FP8 * abs(float(scale)) * mag.max(axis=1)
    vmax = np.empty((len(rows), vd.shape[1]))
    if vis is None:
        vmax[:] = np.abs(vd).max(axis=0)
    else:
        # visible keys of row i are a prefix: running max over keys
        run = np.maximum.accumulate(np.abs(vd), axis=0)
        last = np.minimum(np.asarray(rows) + (kd.shape[0] - qd.shape[0]), kd.shape[0] - 1)
        vmax[:] = run[last]
    return e, 2.0 * e[:, None] * vmax
