"""Head dimensions 96 and 256 (bf16 and fp16 inputs) through fa_fwd and
fa_fwd_split against the fp64 oracle, at the bounds of the input type
(tests/gpu_util.py)."""
import pytest
import torch

import exact_attention_65_amd as fa
import fa_inputs as fi
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu

EDGE_N = [1, 65, 129, 300, 1000]


@pytest.mark.parametrize("D", [96, 256])
@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("N", EDGE_N)
def test_head_dim_edge_shapes(N, causal, dtype, D):
    w = fi.Workload(f"{dtype}_n{N}_d{D}", 1000 + EDGE_N.index(N) + D, 1, 2, N, D, dtype, causal)
    gu.log(f"[gpu] D={D} {dtype} N={N} causal={causal}")
    q, k, v = gu.workload_tensors(w)
    o, lse = gu.run(q, k, v, causal, w.scale)
    gu.compare_heads(w, o, lse, [(0, 0), (0, 1)], what=f"{w.name} causal={causal}")


@pytest.mark.parametrize("D", [96, 256])
@pytest.mark.parametrize("n_splits", [1, 3])
@pytest.mark.parametrize("nq,nk", [(1, 777), (100, 1000)])
def test_head_dim_split(nq, nk, n_splits, D):
    w = fi.Workload(f"bf16_split_nq{nq}_nk{nk}_d{D}", 1010 + nq % 5 + D, 1, 2, nk, D, "bf16", True, NQ=nq)
    q, k, v = gu.workload_tensors(w)
    o, lse = fa.attention_forward_split(q, k, v, causal=True, scale=w.scale, n_splits=n_splits)
    torch.cuda.synchronize()
    gu.compare_heads(w, o, lse, [(0, 0), (0, 1)], what=f"{w.name} splits={n_splits}")


@pytest.mark.parametrize("w", [fi.D256_N4096, fi.D96_N4096], ids=lambda w: w.name)
def test_head_dim_workload(w):
    """B=2, H=16, N=4096, D=256 (the headline's bytes with half the heads) and
    B=2, H=32, N=4096, D=96."""
    gu.log(f"[gpu] workload {w.name}")
    q, k, v = gu.workload_tensors(w)
    o, lse = gu.run(q, k, v, w.causal, w.scale)
    gu.compare_heads(w, o, lse, [(b, h) for b in range(w.B) for h in range(w.H)], what=w.name + " all rows")
