"""Pins for the oracle's merge of partial attention results (oracle.merge_ref).

The merge must give attention over a union of disjoint key sets from the
results over each set.  Checked against the oracle's plain attention over the
whole key set (a different computation: one softmax over all keys), on
contiguous and scattered partitions, with parts in which some rows see no key,
and at magnitudes where exponentiating without the max would overflow.  Planted
mistakes in copies of the merge must each fail one of these checks.
"""
import numpy as np
import pytest

from oracle import attention_ref, merge_ref


def _parts(q, k, v, groups, scale):
    o, lse = [], []
    for idx in groups:
        oi, li = attention_ref(q, k[idx], v[idx], False, scale)
        o.append(oi)
        lse.append(li)
    return np.stack(o), np.stack(lse)


def _checks(merge):
    g = np.random.default_rng(21)
    nq, nk, d = 9, 40, 8
    q, k, v = g.standard_normal((nq, d)), g.standard_normal((nk, d)), g.standard_normal((nk, d))
    scale = 0.35
    o_all, lse_all = attention_ref(q, k, v, False, scale)
    perm = g.permutation(nk)
    partitions = [
        [np.arange(nk)],
        [np.arange(0, 17), np.arange(17, nk)],
        [np.arange(0, 5), np.arange(5, 30), np.arange(30, nk)],
        [perm[:11], perm[11:12], perm[12:]],
    ]
    for groups in partitions:
        o_p, lse_p = _parts(q, k, v, groups, scale)
        o, lse = merge(o_p, lse_p)
        assert np.allclose(o, o_all, rtol=0, atol=1e-12), f"partition of {len(groups)}: o"
        assert np.allclose(lse, lse_all, rtol=0, atol=1e-12), f"partition of {len(groups)}: lse"
    # a part in which every row, or some rows, see no key contributes nothing,
    # whatever its output holds
    o_p, lse_p = _parts(q, k, v, partitions[1], scale)
    empty_o = np.full((1, nq, d), np.nan)
    empty_l = np.full((1, nq), -np.inf)
    o, lse = merge(np.concatenate([o_p, empty_o]), np.concatenate([lse_p, empty_l]))
    assert np.allclose(o, o_all, atol=1e-12) and np.allclose(lse, lse_all, atol=1e-12), "empty part"
    # rows 0..3 see only the first part's keys: the second part is empty for them
    lse_half = lse_p.copy()
    o_half = o_p.copy()
    lse_half[1, :4] = -np.inf
    o_half[1, :4] = np.nan
    o, lse = merge(o_half, lse_half)
    o1, l1 = attention_ref(q[:4], k[partitions[1][0]], v[partitions[1][0]], False, scale)
    assert np.allclose(o[:4], o1, atol=1e-12) and np.allclose(lse[:4], l1, atol=1e-12), "row-wise empty part"
    assert np.allclose(o[4:], o_all[4:], atol=1e-12), "rows that see both parts"
    # large log-sum-exps: merging must not overflow
    shift = 900.0
    o, lse = merge(o_p, lse_p + shift)
    assert np.all(np.isfinite(o)) and np.allclose(lse, lse_all + shift, atol=1e-9), "large lse"
    assert np.allclose(o, o_all, atol=1e-12), "large lse: o"


def test_merge_ref_passes_checks():
    _checks(merge_ref)


def _mutant(kind):
    def merge(o_parts, lse_parts):
        o_parts = np.asarray(o_parts, np.float64)
        lse_parts = np.asarray(lse_parts, np.float64)
        seen = np.isfinite(lse_parts)
        o_parts = np.where(seen[:, :, None], o_parts, 0.0)
        m = lse_parts.max(axis=0)
        with np.errstate(all="ignore"):
            if kind == "no_max":
                w = np.where(seen, np.exp(lse_parts), 0.0)
                tot = w.sum(0)
                return np.einsum("sr,srd->rd", w / tot, o_parts), np.log(tot)
            w = np.where(seen, np.exp(np.where(seen, lse_parts, 0.0) - m), 0.0)
            if kind == "plain_mean":
                w = seen.astype(np.float64)
            if kind == "sign":
                w = np.where(seen, np.exp(m - np.where(seen, lse_parts, 0.0)), 0.0)
            tot = w.sum(0)
            lse = m + np.log(tot)
            if kind == "lse_max_only":
                lse = m
            if kind == "unnormalised":
                return np.einsum("sr,srd->rd", w, o_parts), lse
            return np.einsum("sr,srd->rd", w / tot, o_parts), lse
    return merge


@pytest.mark.parametrize("kind", ["no_max", "plain_mean", "sign", "lse_max_only", "unnormalised"])
def test_merge_mutant_is_caught(kind):
    with pytest.raises(AssertionError):
        _checks(_mutant(kind))
