"""fp16 inputs through fa_fwd and fa_fwd_split against the fp64 oracle on the
same fp16-rounded inputs.

Tolerance (tests/gpu_util.py): max |dO| <= 5e-3, mean |dO| <= 5e-4, |dLSE| <=
1e-3.  The kernel is the bf16 one with fp16 operands: products exact, sums and
softmax in fp32, P and O rounded to fp16, whose unit roundoff 2^-11 is a
quarter of bf16's, so the bf16 bounds are divided by four.
"""
import pytest
import torch

import exact_attention_65_amd as fa
import fa_inputs as fi
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu

EDGE_N = [1, 17, 64, 65, 128, 129, 257, 1000]


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("N", EDGE_N)
def test_f16_edge_shapes(N, causal, D):
    w = fi.Workload(f"f16_n{N}_d{D}", 900 + 4 * EDGE_N.index(N) + D // 64, 1, 2, N, D, "f16", causal)
    gu.log(f"[gpu] f16 N={N} D={D} causal={causal}")
    q, k, v = gu.workload_tensors(w)
    assert q.dtype == torch.float16
    o, lse = gu.run(q, k, v, causal, w.scale)
    assert o.dtype == torch.float16
    gu.compare_heads(w, o, lse, [(0, 0), (0, 1)], what=f"{w.name} causal={causal}")


@pytest.mark.parametrize("scale", [-0.125, 0.0, 0.6])
def test_f16_other_scales(scale):
    w = fi.Workload("f16_scale_n300_d128", 940, 1, 2, 300, 128, "f16", True)
    q, k, v = gu.workload_tensors(w)
    o, lse = gu.run(q, k, v, True, scale)
    from oracle import attention_ref
    errs = []
    for h in range(2):
        o_ref, lse_ref = attention_ref(*fi.head_qkv(w, 0, h), True, scale)
        errs.append(gu.errors(o[0, h].float().cpu().numpy(), lse[0, h].cpu().numpy(), o_ref, lse_ref))
    err = dict(o_max=max(e["o_max"] for e in errs), o_mean=sum(e["o_mean"] for e in errs) / 2,
               lse_max=max(e["lse_max"] for e in errs), finite=all(e["finite"] for e in errs))
    gu.assert_within(err, "f16", f"{w.name} scale={scale}")


@pytest.mark.parametrize("n_splits", [1, 3, fa.FA_SPLIT_AUTO])
@pytest.mark.parametrize("nq,nk", [(1, 777), (100, 1000), (257, 4096)])
def test_f16_split(nq, nk, n_splits):
    w = fi.Workload(f"f16_split_nq{nq}_nk{nk}", 950 + nq % 7, 1, 2, nk, 128, "f16", True, NQ=nq)
    q, k, v = gu.workload_tensors(w)
    o, lse = fa.attention_forward_split(q, k, v, causal=True, scale=w.scale, n_splits=n_splits)
    torch.cuda.synchronize()
    gu.compare_heads(w, o, lse, [(0, 0), (0, 1)], what=f"{w.name} splits={n_splits}")


def test_f16_full_size_workload():
    w = fi.F16_N4096
    gu.log(f"[gpu] workload {w.name}")
    q, k, v = gu.workload_tensors(w)
    o, lse = gu.run(q, k, v, w.causal, w.scale)
    gu.compare_heads(w, o, lse, [(b, h) for b in range(w.B) for h in range(w.H)], what=w.name + " all rows")
