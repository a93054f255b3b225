"""The oracle against its pins (closed forms, invariants, library routine, brute force)."""
import numpy as np
import pytest

from oracle import attention_ref, attention_ref_bhnd
from tests.oracle_pins import ALL_PINS


@pytest.mark.parametrize("pin", ALL_PINS, ids=lambda p: p.__name__)
def test_oracle_pin(pin):
    pin(attention_ref)


def test_heads_independent():
    """Changing one (b, h) slice leaves every other slice's result bit-identical."""
    g = np.random.default_rng(14)
    q, k, v = g.standard_normal((3, 2, 3, 17, 8))
    o1, l1 = attention_ref_bhnd(q, k, v, causal=True, scale=0.4)
    v2 = v.copy()
    v2[1, 2] += 1.0
    o2, l2 = attention_ref_bhnd(q, k, v2, causal=True, scale=0.4)
    mask = np.ones((2, 3), dtype=bool)
    mask[1, 2] = False
    assert np.array_equal(o1[mask], o2[mask]) and np.array_equal(l1, l2)
    assert not np.array_equal(o1[1, 2], o2[1, 2])


def test_rows_subset_matches_full():
    g = np.random.default_rng(15)
    q, k, v = g.standard_normal((3, 300, 16))
    rows = np.array([0, 1, 77, 255, 299])
    for causal in (False, True):
        o, l = attention_ref(q, k, v, causal, 0.25)
        os_, ls = attention_ref(q, k, v, causal, 0.25, rows=rows)
        np.testing.assert_allclose(os_, o[rows], rtol=0, atol=1e-13)
        np.testing.assert_allclose(ls, l[rows], rtol=0, atol=1e-13)


def test_single_key_and_single_row():
    v = np.array([[3.0, -1.0]])
    o, l = attention_ref(np.array([[0.5, 2.0]]), np.array([[1.0, 1.0]]), v, True, 0.5)
    np.testing.assert_array_equal(o, v)
    assert l[0] == pytest.approx(0.5 * 2.5, abs=1e-15)
