"""The backward error model (tests/error_models.py) against a simulation of the
kernels' roundings on the CPU: the gradients recomputed in float64 with P, the
forward's output, dS and the stored gradients rounded to bf16 (or fp16) where
the kernels round them stay within the model's element-wise bound; the bound
is not vacuous (within a modest factor of the simulated errors), and a model
without its Delta term (which the peaked inputs need) is caught."""
import numpy as np
import pytest

import fa_inputs as fi
from oracle import attention_bwd_ref, attention_ref
from tests import error_models as em


def _round(x, dtype):
    x = np.asarray(x, dtype=np.float64)
    if dtype == "bf16":
        return fi.bf16_round(x.astype(np.float32)).astype(np.float64)
    if dtype == "b6":  # a planted coarser rounding: 6 significant bits
        m, e = np.frexp(x)
        return np.ldexp(np.round(m * 64.0) / 64.0, e)
    return x.astype(np.float16).astype(np.float64)


def _simulated(q, k, v, do, causal, scale, dtype, round_dp=False, p_dtype=None):
    """The gradients with the kernels' 16-bit roundings, float64 otherwise."""
    o, _, p = attention_ref(q, k, v, causal, scale, return_p=True)
    pr = _round(p, p_dtype or dtype)
    # the forward: P rounded as the operand, normalised by the rounded sum, O stored rounded
    o_fwd = _round((pr @ v) / pr.sum(axis=1, keepdims=True), dtype)
    dp = do @ v.T
    if round_dp:
        dp = _round(dp, dtype)
    delta = np.sum(do * o_fwd, axis=1)
    ds = _round(p * (dp - delta[:, None]), dtype)
    return _round(scale * (ds @ k), dtype), _round(scale * (ds.T @ q), dtype), _round(pr.T @ do, dtype)


def _inputs(seed, n, d, spread):
    g = np.random.default_rng(seed)
    x = g.standard_normal((4, n, d)).astype(np.float32)
    x[:2] *= spread
    return [fi.bf16_round(t).astype(np.float64) for t in x]


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("spread", [1.0, 4.0])
@pytest.mark.parametrize("causal", [False, True])
def test_model_bounds_the_simulated_roundings(causal, spread, dtype):
    q, k, v, do = _inputs(31 + int(spread) + causal, 96, 32, spread)
    scale = 1 / np.sqrt(32)
    ref = attention_bwd_ref(q, k, v, do, causal, scale)
    sim = _simulated(q, k, v, do, causal, scale, dtype)
    bounds = em.backward_bounds(q, k, v, do, causal, scale, dtype)
    for g, r, b in zip(sim, ref, bounds):
        assert np.all(np.abs(g - r) <= em.KAPPA * b + 1e-300)


@pytest.mark.parametrize("spread", [1.0, 4.0])
def test_bound_is_not_vacuous(spread):
    """The worst-case bound stays within a modest factor of the simulated
    errors (rounding errors of random sign partly cancel; the bound adds their
    magnitudes): for each gradient some element reaches 3 % of it."""
    q, k, v, do = _inputs(40, 96, 32, spread)
    scale = 1 / np.sqrt(32)
    ref = attention_bwd_ref(q, k, v, do, True, scale)
    sim = _simulated(q, k, v, do, True, scale, "bf16")
    bounds = em.backward_bounds(q, k, v, do, True, scale, "bf16")
    for g, r, b in zip(sim, ref, bounds):
        assert float((np.abs(g - r) / (em.KAPPA * b + 1e-300)).max()) >= 0.03


def test_delta_term_is_needed():
    """Without the term for Delta formed from the stored O, the bound fails on
    peaked inputs: the model is not loose enough to pass by accident."""
    q, k, v, do = _inputs(41, 96, 32, 4.0)
    scale = 1 / np.sqrt(32)
    ref = attention_bwd_ref(q, k, v, do, True, scale)
    sim = _simulated(q, k, v, do, True, scale, "bf16")
    u = em.U16["bf16"]
    _, _, p = attention_ref(q, k, v, True, scale, return_p=True)
    o = p @ v
    ds = p * ((do @ v.T) - np.sum(do * o, axis=1)[:, None])
    bq = u * (scale * (np.abs(ds) @ np.abs(k)) + np.abs(ref[0]))
    assert float((np.abs(sim[0] - ref[0]) / (em.KAPPA * bq + 1e-300)).max()) > 1.0


def test_fp8_row_terms_prefix_and_full():
    """The FP8 terms: E_i over the visible keys only, and max_j |v_jd| over them."""
    g = np.random.default_rng(3)
    q, k, v = g.standard_normal((3, 40, 64))
    e_c, t_c = em.fp8_row_terms(q, k, v, True, 0.125)
    e_n, t_n = em.fp8_row_terms(q, k, v, False, 0.125)
    mag = np.abs(q) @ np.abs(k).T
    for i in (0, 7, 39):
        assert np.isclose(e_c[i], em.EPS_FP8 * 0.125 * mag[i, :i + 1].max())
        assert np.allclose(t_c[i], 2 * e_c[i] * np.abs(v[:i + 1]).max(axis=0))
    assert np.allclose(e_n, em.EPS_FP8 * 0.125 * mag.max(axis=1))
    assert np.all(e_c <= e_n + 1e-15)
