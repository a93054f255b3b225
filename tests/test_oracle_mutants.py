"""Mistakes planted in copies of the oracle, on the CPU: every one must fail a pin.

Each mutant is the plain definition with one plausible slip (a dropped term, a
wrong sign or index, a transposed operand, a wrong axis or log base).  The pins
in tests/oracle_pins.py must reject each of them, which shows they constrain
every step of the oracle and not only its overall shape.
"""
import numpy as np
import pytest

from tests.oracle_pins import ALL_PINS


def _make(scores=None, mask=None, maxsub=True, axis=1, normalise=True, lse_fn=None, values=None,
          scale_fn=None):
    def attn(q, k, v, causal, scale, rows=None, return_p=False):
        q = np.asarray(q, dtype=np.float64)
        k = np.asarray(k, dtype=np.float64)
        v = np.asarray(v, dtype=np.float64)
        if scale is None:
            scale = 1 / np.sqrt(q.shape[1])
        if scale_fn:
            scale = scale_fn(scale, q.shape[1])
        rows = np.arange(q.shape[0]) if rows is None else np.asarray(rows)
        s = scale * (scores(q[rows], k) if scores else q[rows] @ k.T)
        if causal:
            nq, nk = q.shape[0], k.shape[0]
            bad = mask(rows, nq, nk) if mask else (np.arange(nk)[None, :] > rows[:, None] + (nk - nq))
            s = np.where(bad, -np.inf, s)
        m = s.max(axis=axis, keepdims=True) if maxsub else np.zeros((1, 1))
        with np.errstate(all="ignore"):
            p = np.exp(s - m)
            l = p.sum(axis=axis, keepdims=True)
            w = p / l if normalise else p
            vv = values(k, v) if values else v
            o = w @ vv
            lse = lse_fn(m, l) if lse_fn else (m + np.log(l))
        lse = np.broadcast_to(lse, (len(rows), 1))[:, 0] if axis == 1 else np.log(np.exp(s).sum(1))
        if return_p:
            return o, lse, w
        return o, lse
    return attn


MUTANTS = {
    "reference_copy": None,  # sanity: the unmutated copy passes every pin
    "transposed_scores": _make(scores=lambda q, k: (k[: q.shape[0]] @ q.T).T if k.shape[0] >= q.shape[0] and q.shape[0] == k.shape[0] else q @ k.T * 1.0000001),
    "no_max_subtraction": _make(maxsub=False),
    "wrong_sign_scores": _make(scores=lambda q, k: -(q @ k.T)),
    "causal_excludes_diagonal": _make(mask=lambda r, nq, nk: np.arange(nk)[None, :] >= r[:, None] + (nk - nq)),
    "causal_upper_triangle": _make(mask=lambda r, nq, nk: np.arange(nk)[None, :] < r[:, None] + (nk - nq)),
    "causal_off_by_one": _make(mask=lambda r, nq, nk: np.arange(nk)[None, :] > r[:, None] + (nk - nq) + 1),
    "causal_offset_ignored": _make(mask=lambda r, nq, nk: np.arange(nk)[None, :] > r[:, None]),
    "causal_offset_reversed": _make(mask=lambda r, nq, nk: np.arange(nk)[None, :] > r[:, None] - (nk - nq)),
    "softmax_over_queries": _make(axis=0),
    "no_normalisation": _make(normalise=False),
    "scale_dropped": _make(scale_fn=lambda s, d: 1.0),
    "scale_without_sqrt": _make(scale_fn=lambda s, d: s * s),
    "lse_base2": _make(lse_fn=lambda m, l: (m + np.log(l)) / np.log(2.0)),
    "lse_without_max": _make(lse_fn=lambda m, l: np.log(l)),
    "values_replaced_by_keys": _make(values=lambda k, v: k[:, : v.shape[1]] if k.shape[1] >= v.shape[1] else v * 1.01),
    "values_reversed": _make(values=lambda k, v: v[::-1]),
}


def _passes_all(attn):
    failed = []
    for pin in ALL_PINS:
        try:
            pin(attn)
        except Exception as e:  # noqa: BLE001 - any failure counts as caught
            failed.append((pin.__name__, type(e).__name__))
    return failed


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name):
    if name == "reference_copy":
        assert _passes_all(_make()) == []
        return
    failed = _passes_all(MUTANTS[name])
    assert failed, f"mutant {name} passed every pin"
