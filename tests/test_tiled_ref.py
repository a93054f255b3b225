"""The CPU online-softmax recurrence: a hand trace, and equality with the plain definition."""
import math

import numpy as np
import pytest

from oracle import attention_ref, tiled_ref


def test_recurrence_hand_trace():
    """Row 0 of the two-key worked example, one key per block, traced by hand:
    after key 0: m=0, l=1, o=4; after key 1: m=ln3, alpha=1/3, l=1/3+1=4/3,
    o=4/3+8=28/3, and o/l = 7, lse = ln3 + ln(4/3) = ln 4."""
    q = np.array([[math.log(3.0)]])
    k = np.array([[0.0], [1.0]])
    v = np.array([[4.0], [8.0]])
    o, lse = tiled_ref(q, k, v, False, 1.0, block=1)
    assert o[0, 0] == pytest.approx(7.0, abs=1e-14)
    assert lse[0] == pytest.approx(math.log(4.0), abs=1e-14)
    # the intermediate state after the first block only
    o1, l1 = tiled_ref(q, k[:1], v[:1], False, 1.0, block=1)
    assert o1[0, 0] == 4.0 and l1[0] == 0.0
    # reversed order reaches the same state
    o2, l2 = tiled_ref(q, k, v, False, 1.0, block=1, order="desc")
    assert o2[0, 0] == pytest.approx(7.0, abs=1e-14) and l2[0] == pytest.approx(math.log(4.0), abs=1e-14)


@pytest.mark.parametrize("block", [1, 3, 7, 64, 100])
@pytest.mark.parametrize("order", ["asc", "desc", "random"])
@pytest.mark.parametrize("causal", [False, True])
def test_tiled_equals_plain(block, order, causal):
    g = np.random.default_rng(block * 7 + len(order) + causal)
    n, d = 100, 16
    q, k, v = g.standard_normal((3, n, d)) * 2.0
    o_ref, l_ref = attention_ref(q, k, v, causal, 0.3)
    o, l = tiled_ref(q, k, v, causal, 0.3, block=block, order=order, seed=block)
    np.testing.assert_allclose(o, o_ref, rtol=0, atol=1e-12)
    np.testing.assert_allclose(l, l_ref, rtol=0, atol=1e-12)


def test_tiled_peaked_scores():
    """Scores spread over hundreds of units: rescaling by exp(m - m_new) must keep the sum."""
    g = np.random.default_rng(5)
    q, k, v = g.standard_normal((3, 70, 8)) * 8.0
    o_ref, l_ref = attention_ref(q, k, v, True, 1.0)
    o, l = tiled_ref(q, k, v, True, 1.0, block=9, order="random")
    np.testing.assert_allclose(o, o_ref, rtol=0, atol=1e-11)
    np.testing.assert_allclose(l, l_ref, rtol=1e-13, atol=0)
