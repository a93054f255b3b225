"""Pins for the gradient oracle (oracle.attention_bwd_ref), none of which reuses
its closed form: central finite differences of the forward oracle, torch's
float64 autograd through its math attention, and two invariants of the
definition.  Planted mistakes in copies of the gradient each fail a pin.
"""
import math

import numpy as np
import pytest

from oracle import attention_bwd_ref, attention_ref


def _rng(seed):
    return np.random.default_rng(seed)


def _case(seed, nq=7, nk=9, d=5, dv=4, causal=False):
    g = _rng(seed)
    if causal:
        nk = max(nk, nq)
    return (g.standard_normal((nq, d)), g.standard_normal((nk, d)), g.standard_normal((nk, dv)),
            g.standard_normal((nq, dv)))


def _loss(q, k, v, do, causal, scale):
    return float(np.sum(attention_ref(q, k, v, causal, scale)[0] * do))


def pin_finite_differences(bwd):
    """Each gradient entry against a central difference of <o(q,k,v), do>."""
    for causal in (False, True):
        q, k, v, do = _case(1, causal=causal)
        scale = 0.6
        grads = bwd(q, k, v, do, causal, scale)
        for x, gx in zip((q, k, v), grads):
            num = np.empty_like(x)
            for idx in np.ndindex(*x.shape):
                h = 1e-6
                old = x[idx]
                x[idx] = old + h
                lp = _loss(q, k, v, do, causal, scale)
                x[idx] = old - h
                lm = _loss(q, k, v, do, causal, scale)
                x[idx] = old
                num[idx] = (lp - lm) / (2 * h)
            assert np.allclose(gx, num, rtol=1e-6, atol=1e-7), f"finite differences causal={causal}"


def pin_torch_autograd(bwd):
    """torch float64 autograd of softmax(scale q k^T + mask) v, written with its
    own softmax and matmul (not the oracle)."""
    import torch
    for causal, (nq, nk) in ((False, (11, 13)), (True, (12, 12)), (True, (3, 10))):
        g = _rng(2 + nq)
        q, k, v, do = (g.standard_normal(s) for s in ((nq, 8), (nk, 8), (nk, 6), (nq, 6)))
        scale = 1 / math.sqrt(8)
        tq, tk, tv = (torch.tensor(x, dtype=torch.float64, requires_grad=True) for x in (q, k, v))
        s = scale * (tq @ tk.T)
        if causal:
            allowed = torch.arange(nk)[None, :] <= torch.arange(nq)[:, None] + (nk - nq)
            s = s.masked_fill(~allowed, float("-inf"))
        o = torch.softmax(s, dim=-1) @ tv
        o.backward(torch.tensor(do, dtype=torch.float64))
        for name, ours, ref in zip("qkv", bwd(q, k, v, do, causal, scale), (tq.grad, tk.grad, tv.grad)):
            assert np.allclose(ours, ref.numpy(), rtol=1e-10, atol=1e-12), f"autograd d{name} causal={causal}"


def pin_invariants(bwd):
    """Adding one vector to every key shifts each row's scores by a constant, so
    the key gradients sum to zero; each row's weights sum to one, so the value
    gradients sum to the summed upstream gradient."""
    for causal in (False, True):
        q, k, v, do = _case(3, nq=10, nk=10, causal=causal)
        _, dk, dv = bwd(q, k, v, do, causal, 0.45)
        assert np.allclose(dk.sum(axis=0), 0.0, atol=1e-12), "sum of dK"
        assert np.allclose(dv.sum(axis=0), do.sum(axis=0), atol=1e-12), "sum of dV"


PINS = [pin_finite_differences, pin_torch_autograd, pin_invariants]


@pytest.mark.parametrize("pin", PINS, ids=lambda p: p.__name__)
def test_gradient_oracle_passes(pin):
    pin(attention_bwd_ref)


def _mutant(kind):
    def bwd(q, k, v, do, causal=False, scale=None):
        q, k, v, do = (np.asarray(x, np.float64) for x in (q, k, v, do))
        if scale is None:
            scale = 1 / np.sqrt(q.shape[1])
        o, _, p = attention_ref(q, k, v, causal, scale, return_p=True)
        dv = (do.T @ p).T if kind == "dv_transposed_weights" else p.T @ do
        if kind == "dv_transposed_weights" and p.shape[0] == p.shape[1]:
            dv = p @ do
        dp = do @ v.T
        delta = np.sum(do * o, axis=1)
        if kind == "no_delta":
            delta = 0 * delta
        if kind == "delta_from_values":
            delta = np.sum(do * v[: do.shape[0]] if v.shape[0] >= do.shape[0] else do, axis=1)
        ds = p * (dp - delta[:, None])
        if kind == "ds_sign":
            ds = -ds
        dq = scale * (ds @ k)
        dk = scale * (ds.T @ q)
        if kind == "no_scale":
            dq, dk = ds @ k, ds.T @ q
        if kind == "dk_from_keys":
            dk = scale * (ds.T @ np.resize(k, q.shape))
        return dq, dk, dv
    return bwd


@pytest.mark.parametrize("kind", ["dv_transposed_weights", "no_delta", "delta_from_values", "ds_sign",
                                  "no_scale", "dk_from_keys"])
def test_gradient_mutant_is_caught(kind):
    failed = 0
    for pin in PINS:
        try:
            pin(_mutant(kind))
        except AssertionError:
            failed += 1
    assert failed, f"mutant {kind} passed every pin"
