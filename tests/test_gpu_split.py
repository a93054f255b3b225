"""fa_fwd_split against the fp64 oracle: key ranges merged by log-sum-exp, fewer
queries than keys (the queries being the last positions under the causal mask),
and the short-sequence and decode workloads it exists for.

Small shapes are compared on every element; the decode and chunked-prefill
workloads at full size on every row of every (or of seeded) heads.
"""
import numpy as np
import pytest
import torch

import exact_attention_65_amd as fa
import fa_inputs as fi
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu


def _run(q, k, v, causal, scale, n_splits):
    o, lse = fa.attention_forward_split(q, k, v, causal=causal, scale=scale, n_splits=n_splits)
    torch.cuda.synchronize()
    return o, lse


SHAPES = [(1, 1), (1, 64), (1, 777), (5, 300), (64, 64), (100, 1000), (130, 130), (257, 4096)]


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("n_splits", [1, 2, 7, fa.FA_SPLIT_AUTO])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("nq,nk", SHAPES)
def test_split_small_shapes(nq, nk, causal, n_splits, D):
    seed = 600 + 10 * SHAPES.index((nq, nk)) + D // 64
    w = fi.Workload(f"split_nq{nq}_nk{nk}_d{D}", seed, 1, 2, nk, D, "bf16", causal, NQ=nq)
    gu.log(f"[gpu] split nq={nq} nk={nk} D={D} causal={causal} n_splits={n_splits}")
    q, k, v = gu.workload_tensors(w)
    o, lse = _run(q, k, v, causal, w.scale, n_splits)
    gu.compare_heads(w, o, lse, [(0, 0), (0, 1)], what=f"{w.name} causal={causal} splits={n_splits}")


def test_split_outputs_written_and_deterministic():
    w = fi.Workload("split_nan_canary", 650, 2, 3, 999, 128, "bf16", True, NQ=333)
    q, k, v = gu.workload_tensors(w)
    runs = []
    for _ in range(2):
        o = torch.full_like(q, float("nan"))
        lse = torch.full((w.B, w.H, w.nq), float("nan"), device=q.device)
        fa.attention_forward_split(q, k, v, causal=True, scale=w.scale, n_splits=5, out=o, lse=lse)
        torch.cuda.synchronize()
        assert torch.isfinite(o.float()).all() and torch.isfinite(lse).all()
        runs.append((o.clone(), lse.clone()))
    assert torch.equal(runs[0][0], runs[1][0]) and torch.equal(runs[0][1], runs[1][1])


def test_split_matches_single_launch_kernel():
    """Square causal shape: the merged ranges agree with fa_fwd to the bf16 tolerance."""
    w = fi.CAUSAL_SWEEP[0]  # N = 512
    q, k, v = gu.workload_tensors(w)
    o1, l1 = gu.run(q, k, v, True, w.scale)
    o2, l2 = _run(q, k, v, True, w.scale, 4)
    assert (o1.float() - o2.float()).abs().max().item() <= 2e-2
    assert (l1 - l2).abs().max().item() <= 1e-3


@pytest.mark.parametrize("n_splits", [3, 8])
def test_split_short_causal_sweep(n_splits):
    """The short causal workloads split into key ranges (the automatic choice
    keeps them on one range; the split result must still be exact)."""
    for w in (fi.CAUSAL_SWEEP[0], fi.CAUSAL_SWEEP[1], fi.CAUSAL_SWEEP[0].with_variant(fi.PEAKED)):
        gu.log(f"[gpu] split workload {w.name}: {n_splits} ranges")
        q, k, v = gu.workload_tensors(w)
        o, lse = _run(q, k, v, True, w.scale, n_splits)
        gu.compare_heads(w, o, lse, [(0, h) for h in range(w.H)], what=w.name + " split")


def test_split_decode_workload():
    """One new token per head against 16384 cached keys: every head, every row."""
    w = fi.SPLIT_DECODE
    gu.log(f"[gpu] workload {w.name}")
    q, k, v = gu.workload_tensors(w)
    o, lse = _run(q, k, v, w.causal, w.scale, fa.FA_SPLIT_AUTO)
    del q, k, v
    gu.compare_heads(w, o, lse, [(b, h) for b in range(w.B) for h in range(w.H)], what=w.name)


def test_split_chunk_workload():
    """512 queries after a 7680-key prefix: 4 seeded heads, every row."""
    w = fi.SPLIT_CHUNK
    gu.log(f"[gpu] workload {w.name}")
    q, k, v = gu.workload_tensors(w)
    o, lse = _run(q, k, v, w.causal, w.scale, fa.FA_SPLIT_AUTO)
    del q, k, v
    gu.compare_heads(w, o, lse, fi.sample_heads(w, 4), what=w.name)
