"""Pins for the attention oracle: checks that do not come from the oracle itself.

Each pin takes an attention function with the oracle's signature
``attn(q, k, v, causal, scale, rows=None, return_p=False)`` and raises
AssertionError when the function disagrees with something the pages or plain
mathematics fix: hand-worked values, closed forms, invariants, an independent
library routine, a differently-formulated brute force.  tests/test_oracle_pins.py
runs them on the oracle; tests/test_oracle_mutants.py runs them on copies of the
oracle with planted mistakes and requires every mistake to be caught.
"""
from __future__ import annotations

import json
import math
import os

import numpy as np

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "worked_examples.json")
TOL = 1e-12


def _val(x):
    if isinstance(x, list) and len(x) == 2 and x[0] == "ln":
        return math.log(x[1])
    if isinstance(x, list):
        return [_val(e) for e in x]
    return float(x)


def _rng(seed):
    return np.random.default_rng(seed)


def _close(a, b, tol=TOL, what=""):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    assert a.shape == b.shape, f"{what}: shape {a.shape} vs {b.shape}"
    assert np.all(np.isfinite(a)), f"{what}: non-finite values"
    err = np.max(np.abs(a - b)) if a.size else 0.0
    assert err <= tol * max(1.0, float(np.max(np.abs(b))) if b.size else 1.0), f"{what}: max err {err}"


# P1 -------------------------------------------------------------------------
def pin_worked_examples(attn):
    """Hand-computed cases (tests/golden/worked_examples.json)."""
    with open(GOLDEN) as f:
        cases = json.load(f)["cases"]
    for c in cases:
        q, k, v = (np.array(_val(c[x])) for x in ("q", "k", "v"))
        for causal, key in ((False, "noncausal"), (True, "causal")):
            o, lse = attn(q, k, v, causal, c["scale"])[:2]
            _close(o, _val(c[key]["o"]), what=f"{c['name']} {key} o")
            _close(lse, _val(c[key]["lse"]), what=f"{c['name']} {key} lse")


# P3 -------------------------------------------------------------------------
def pin_uniform_scores(attn):
    """Q = 0: every visible key scores 0, so o_i is the mean of the visible v_j
    and lse_i = ln |J(i)|.  Identical key rows: same, with lse shifted by the score."""
    g = _rng(3)
    n, d = 37, 8
    v = g.standard_normal((n, 5))
    counts = np.arange(1, n + 1)
    prefix_mean = np.cumsum(v, axis=0) / counts[:, None]
    for causal in (False, True):
        o, lse = attn(np.zeros((n, d)), g.standard_normal((n, d)), v, causal, 0.3)[:2]
        if causal:
            _close(o, prefix_mean, what="uniform causal o")
            _close(lse, np.log(counts), what="uniform causal lse")
        else:
            _close(o, np.broadcast_to(v.mean(axis=0), o.shape), what="uniform o")
            _close(lse, np.full(n, math.log(n)), what="uniform lse")
    q = g.standard_normal((n, d))
    krow = g.standard_normal(d)
    k = np.tile(krow, (n, 1))
    scale = 0.7
    o, lse = attn(q, k, v, False, scale)[:2]
    _close(o, np.broadcast_to(v.mean(axis=0), o.shape), what="identical keys o")
    _close(lse, scale * (q @ krow) + math.log(n), what="identical keys lse")


# P4 -------------------------------------------------------------------------
def pin_weights_are_a_distribution(attn):
    """The returned weights are >= 0, sum to 1 over the visible keys, are 0 on
    masked keys, and o equals weights @ v."""
    g = _rng(4)
    n, d = 41, 16
    q, k, v = g.standard_normal((3, n, d))
    for causal in (False, True):
        o, lse, p = attn(q, k, v, causal, 0.25, return_p=True)
        assert np.all(p >= 0)
        _close(p.sum(axis=1), np.ones(n), what="weights sum")
        if causal:
            assert np.all(np.triu(p, 1) == 0), "masked weights not zero"
        _close(o, p @ v, what="o = p v")


# P5 -------------------------------------------------------------------------
def pin_constant_values(attn):
    g = _rng(5)
    n, d = 29, 12
    q = g.standard_normal((n, d)) * 3
    k = g.standard_normal((n, d)) * 3
    c = g.standard_normal(7)
    for causal in (False, True):
        o, _ = attn(q, k, np.tile(c, (n, 1)), causal, 1 / math.sqrt(d))[:2]
        _close(o, np.tile(c, (n, 1)), what="constant v")


# P6 -------------------------------------------------------------------------
def pin_key_permutation(attn):
    """Non-causal attention is a function of the set of (key, value) pairs."""
    g = _rng(6)
    n, d = 33, 9
    q, k, v = g.standard_normal((3, n, d))
    perm = g.permutation(n)
    o1, l1 = attn(q, k, v, False, 0.4)[:2]
    o2, l2 = attn(q, k[perm], v[perm], False, 0.4)[:2]
    _close(o1, o2, what="perm o")
    _close(l1, l2, what="perm lse")
    # ... and each query row is computed on its own
    rows = g.permutation(n)[:10]
    o3, l3 = attn(q[rows], k, v, False, 0.4)[:2]
    _close(o3, o1[rows], what="row independence o")
    _close(l3, l1[rows], what="row independence lse")


# P7 -------------------------------------------------------------------------
def pin_dominant_score(attn):
    """A key aligned with the query at large norm takes (almost) all the weight.

    Bound: |o_i - v_*| <= sum_{j != *} w_ij |v_j - v_*| with w_ij computed in
    closed form from the score gaps."""
    g = _rng(7)
    n, d = 24, 16
    q = g.standard_normal((n, d))
    k = 0.1 * g.standard_normal((n, d))
    v = g.standard_normal((n, d))
    i, jstar = 5, 17
    k[jstar] = 50.0 * q[i] / np.linalg.norm(q[i])
    scale = 1.0 / math.sqrt(d)
    o, _ = attn(q, k, v, False, scale)[:2]
    s = scale * (k @ q[i])
    gaps = s - s[jstar]
    w_other = np.exp(gaps) / np.exp(gaps).sum()
    bound = float(np.sum(np.delete(w_other, jstar)[:, None] * np.abs(np.delete(v, jstar, 0) - v[jstar]), axis=0).max())
    assert bound < 1e-3
    assert np.max(np.abs(o[i] - v[jstar])) <= bound * 1.0001 + 1e-14


# P8 -------------------------------------------------------------------------
def pin_score_shift(attn):
    """Adding the same constant c*scale to every score of a row leaves o unchanged
    and adds c*scale to lse.  With c*scale = 1000 an exp without max
    subtraction overflows float64."""
    g = _rng(8)
    n, d = 21, 8
    q, k, v = g.standard_normal((3, n, d))
    scale = 0.5
    c = 1000.0 / scale
    q2 = np.concatenate([q, np.full((n, 1), c)], axis=1)
    k2 = np.concatenate([k, np.ones((n, 1))], axis=1)
    for causal in (False, True):
        o1, l1 = attn(q, k, v, causal, scale)[:2]
        o2, l2 = attn(q2, k2, v, causal, scale)[:2]
        _close(o2, o1, tol=1e-11, what="shift o")
        _close(l2, l1 + 1000.0, tol=1e-12, what="shift lse")


# P9 -------------------------------------------------------------------------
def pin_torch_sdpa(attn):
    """torch's CPU float64 scaled_dot_product_attention computes the same map
    (the pages name it as PyTorch's attention entry point)."""
    import torch
    import torch.nn.functional as F
    from torch.nn.attention import SDPBackend, sdpa_kernel
    g = _rng(9)
    for n, d, causal, scale in ((50, 16, False, 0.25), (64, 32, True, 1 / math.sqrt(32)), (7, 4, True, -0.8)):
        q, k, v = g.standard_normal((3, n, d))
        o, lse = attn(q, k, v, causal, scale)[:2]
        t = [torch.from_numpy(x)[None, None] for x in (q, k, v)]
        # torch's fused CPU kernel returns NaN for a negative scale under a causal
        # mask; its plain math backend does not, so that backend is the pin.
        with sdpa_kernel(SDPBackend.MATH):
            ot = F.scaled_dot_product_attention(*t, is_causal=causal, scale=scale)[0, 0].numpy()
        _close(o, ot, tol=1e-12, what="sdpa o")
        st = torch.from_numpy(q) @ torch.from_numpy(k).T * scale
        if causal:
            st = st.masked_fill(torch.triu(torch.ones(n, n, dtype=torch.bool), 1), float("-inf"))
        _close(lse, torch.logsumexp(st, dim=1).numpy(), tol=1e-12, what="logsumexp lse")


# P10 ------------------------------------------------------------------------
def pin_mpmath_bruteforce(attn):
    """50-digit brute force with each weight formed on its own as
    w_ij = 1 / sum_k exp(s_ik - s_ij)  (no max, no shared normaliser)."""
    import mpmath as mp
    mp.mp.dps = 50
    g = _rng(10)
    for n, d, causal in ((5, 3, False), (6, 2, True), (4, 4, False)):
        q, k, v = g.standard_normal((3, n, d))
        scale = 0.9
        o, lse = attn(q, k, v, causal, scale)[:2]
        for i in range(n):
            J = range(i + 1) if causal else range(n)
            s = {j: mp.mpf(scale) * mp.fsum(mp.mpf(q[i, t]) * mp.mpf(k[j, t]) for t in range(d)) for j in J}
            for col in range(d):
                acc = mp.fsum(v[j, col] / mp.fsum(mp.e ** (s[kk] - s[j]) for kk in J) for j in J)
                assert abs(float(acc) - o[i, col]) <= 1e-13, "mpmath o"
            ref_lse = mp.log(mp.fsum(mp.e ** s[j] for j in J))
            assert abs(float(ref_lse) - lse[i]) <= 1e-13, "mpmath lse"


# P12 ------------------------------------------------------------------------
def pin_causal_prefix(attn):
    """Causal row 0 sees key 0 only (o_0 = v_0, lse_0 = s_00); causal row i equals
    non-causal attention over keys 0..i."""
    g = _rng(12)
    n, d = 19, 8
    q, k, v = g.standard_normal((3, n, d))
    scale = 0.45
    o, lse = attn(q, k, v, True, scale)[:2]
    _close(o[0], v[0], what="causal row 0 o")
    _close(lse[0], scale * (q[0] @ k[0]), what="causal row 0 lse")
    for i in (1, 7, n - 1):
        oi, li = attn(q[i:i + 1], k[:i + 1], v[:i + 1], False, scale)[:2]
        _close(o[i], oi[0], what=f"prefix row {i} o")
        _close(lse[i], li[0], what=f"prefix row {i} lse")


# P13 ------------------------------------------------------------------------
def pin_linear_in_values(attn):
    g = _rng(13)
    n, d = 26, 10
    q, k, v1, v2 = g.standard_normal((4, n, d))
    a, b = 0.7, -2.5
    for causal in (False, True):
        o1 = attn(q, k, v1, causal, 0.3)[0]
        o2 = attn(q, k, v2, causal, 0.3)[0]
        o12 = attn(q, k, a * v1 + b * v2, causal, 0.3)[0]
        _close(o12, a * o1 + b * o2, tol=1e-12, what="linearity")


# P14 ------------------------------------------------------------------------
def pin_causal_query_suffix(attn):
    """With fewer queries than keys the queries are the last positions of the
    sequence: causal attention of Q against K equals the last Nq rows of the
    square causal attention whose query rows are [P; Q], whatever P is; a single
    query therefore sees every key."""
    g = _rng(14)
    nk, d = 23, 8
    k, v = g.standard_normal((2, nk, d))
    scale = 0.4
    for nq in (1, 5, 22, nk):
        q = g.standard_normal((nq, d))
        full_q = np.concatenate([g.standard_normal((nk - nq, d)), q])
        o_full, lse_full = attn(full_q, k, v, True, scale)[:2]
        o, lse = attn(q, k, v, True, scale)[:2]
        _close(o, o_full[nk - nq:], what=f"suffix nq={nq} o")
        _close(lse, lse_full[nk - nq:], what=f"suffix nq={nq} lse")
    q1 = g.standard_normal((1, d))
    o_c, l_c = attn(q1, k, v, True, scale)[:2]
    o_n, l_n = attn(q1, k, v, False, scale)[:2]
    _close(o_c, o_n, what="single query o")
    _close(l_c, l_n, what="single query lse")


ALL_PINS = [
    pin_worked_examples,
    pin_uniform_scores,
    pin_weights_are_a_distribution,
    pin_constant_values,
    pin_key_permutation,
    pin_dominant_score,
    pin_score_shift,
    pin_torch_sdpa,
    pin_mpmath_bruteforce,
    pin_causal_prefix,
    pin_linear_in_values,
    pin_causal_query_suffix,
]
