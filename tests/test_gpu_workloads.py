"""HIP path vs the fp64 oracle on the five workloads at their full sizes, in the
launch configuration the benchmark times.  The fp32 workload, the bf16 N=4096
workload and every causal-sweep workload (both variants) are compared on every
head and every row; the B=32 prefill on 4 seeded (b, h) pairs, every row; the
N=131072 workload on 256 seeded rows per head plus its first and last rows.
"""
import numpy as np
import pytest
import torch

import fa_inputs as fi
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu


def _run_workload(w):
    gu.log(f"[gpu] workload {w.name}: B={w.B} H={w.H} N={w.N} D={w.D} {w.dtype} causal={w.causal} "
           f"variant={w.variant}")
    q, k, v = gu.workload_tensors(w)
    o, lse = gu.run(q, k, v, w.causal, w.scale)
    del q, k, v
    return o, lse


def test_fp32_small_all_elements():
    w = fi.FP32_SMALL
    o, lse = _run_workload(w)
    gu.compare_heads(w, o, lse, [(0, 0)])


def test_bf16_n4096_noncausal():
    """All 64 heads, every row."""
    w = fi.BF16_N4096
    o, lse = _run_workload(w)
    gu.compare_heads(w, o, lse, [(b, h) for b in range(w.B) for h in range(w.H)], what=w.name + " all rows")


@pytest.mark.parametrize("variant", [fi.PLAIN, fi.PEAKED])
@pytest.mark.parametrize("n", fi.CAUSAL_SWEEP_N)
def test_causal_sweep(n, variant):
    """All 32 heads, every row."""
    w = fi.CAUSAL_SWEEP[fi.CAUSAL_SWEEP_N.index(n)].with_variant(variant)
    o, lse = _run_workload(w)
    gu.compare_heads(w, o, lse, [(0, h) for h in range(w.H)], what=w.name + " all rows")


def test_causal_prefill_b32():
    """4 seeded (b, h) pairs, every row."""
    w = fi.CAUSAL_PREFILL
    o, lse = _run_workload(w)
    gu.compare_heads(w, o, lse, fi.sample_heads(w, 4))


def test_causal_long_context():
    """256 seeded rows per head (+ rows 0 and N-1); no workspace beyond O and LSE."""
    import exact_attention_65_amd as fa
    w = fi.CAUSAL_LONG
    st, sz = fa.fa_fwd_query(w.B, w.H, w.N, w.D, 1, fa.FA_DTYPE_BF16)
    assert st == fa.FA_OK and sz.workspace_bytes == 0
    q, k, v = gu.workload_tensors(w)
    torch.cuda.synchronize()
    before = torch.cuda.memory_allocated()
    torch.cuda.reset_peak_memory_stats()
    gu.log(f"[gpu] workload {w.name}")
    o, lse = gu.run(q, k, v, w.causal, w.scale)
    # the only allocations are O and LSE themselves
    assert torch.cuda.max_memory_allocated() - before <= sz.o_bytes + sz.lse_bytes + (4 << 20)
    del q, k, v
    gu.compare_heads(w, o, lse, [(0, h) for h in range(w.H)],
                     rows_for=lambda h: fi.sample_rows(w, h, 256), what=w.name + " sampled rows")
