"""The two one-range 16-bit kernels at D = 128 against the fp64 oracle.

fa_fwd (and fa_fwd_split with one range) runs grids of at most one 128-row
workgroup per compute unit (B * H * ceil(Nq / 128) <= CU count) on a kernel
with 64 rows per workgroup and 16 per wave, and larger grids on the 128-row
kernel.  Each case runs the same heads twice: with H = 2, which takes the
64-row kernel, and with H just large enough for the 128-row kernel on this
device.  A head's inputs depend only on its (b, h) and the seed, so heads 0
and 1 are the same in both runs; both are checked against the oracle on heads
0, 1 and the last, every row and column.
"""
import math

import pytest
import torch

import exact_attention_65_amd as fa
import fa_inputs as fi
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu

EDGE_N = [1, 17, 64, 65, 129, 257, 1000]


def _cus() -> int:
    return torch.cuda.get_device_properties(0).multi_processor_count


def _head_counts(nq: int):
    """H for the 64-row kernel (2) and the smallest H that takes the 128-row one."""
    qblocks = math.ceil(nq / 128)
    big = _cus() // qblocks + 1
    assert 2 * qblocks <= _cus() < big * qblocks
    return 2, big


def _both_kernels(name, seed, nq, nk, dtype, causal, forward):
    results = {}
    for H in _head_counts(nq):
        w = fi.Workload(f"{name}_h{H}", seed, 1, H, nk, 128, dtype, causal, NQ=nq if nq != nk else 0)
        gu.log(f"[gpu] {w.name}: Nq={nq} Nk={nk} {dtype} causal={causal}")
        q, k, v = gu.workload_tensors(w)
        o, lse = forward(w, q, k, v)
        torch.cuda.synchronize()
        gu.compare_heads(w, o, lse, [(0, 0), (0, 1), (0, H - 1)], what=f"{w.name} causal={causal}")
        results[H] = (o[:, :2].float().cpu(), lse[:, :2].cpu())
    (o0, l0), (o1, l1) = results.values()
    gu.log(f"  heads 0-1, 64-row vs 128-row kernel: max|dO| {float((o0 - o1).abs().max()):.3e} "
           f"max|dLSE| {float((l0 - l1).abs().max()):.3e}")


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("N", EDGE_N)
def test_fwd_small_and_large_grids(N, causal, dtype):
    seed = 1100 + 2 * EDGE_N.index(N) + causal

    def forward(w, q, k, v):
        return fa.attention_forward(q, k, v, causal=causal, scale=w.scale)

    _both_kernels(f"grid_n{N}", seed, N, N, dtype, causal, forward)


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("nq,nk", [(5, 300), (100, 1000), (257, 4096), (512, 8192)])
def test_split_one_range_small_and_large_grids(nq, nk, causal):
    """Nq queries against Nk keys (the queries are the last Nq positions under
    the causal mask) through fa_fwd_split with one range."""
    seed = 1130 + nq % 11 + causal

    def forward(w, q, k, v):
        return fa.attention_forward_split(q, k, v, causal=causal, scale=w.scale, n_splits=1)

    _both_kernels(f"split1_nq{nq}_nk{nk}", seed, nq, nk, "bf16", causal, forward)


@pytest.mark.parametrize("scale", [-0.125, 0.0, 2.0])
def test_small_grid_unusual_scales(scale):
    """A negative scale (signs carried by Q), zero (uniform weights) and a large
    one (peaked rows, where the lazy reference moves) on the 64-row kernel."""
    w = fi.Workload("grid_scale_n300", 1150, 1, 2, 300, 128, "bf16", True)
    q, k, v = gu.workload_tensors(w)
    o, lse = fa.attention_forward(q, k, v, causal=True, scale=scale)
    torch.cuda.synchronize()
    from oracle import attention_ref
    errs = []
    for h in range(2):
        o_ref, lse_ref = attention_ref(*fi.head_qkv(w, 0, h), True, scale)
        errs.append(gu.errors(o[0, h].float().cpu().numpy(), lse[0, h].cpu().numpy(), o_ref, lse_ref))
    err = dict(o_max=max(e["o_max"] for e in errs), o_mean=sum(e["o_mean"] for e in errs) / 2,
               lse_max=max(e["lse_max"] for e in errs), finite=all(e["finite"] for e in errs))
    gu.assert_within(err, "bf16", f"{w.name} scale={scale}")


def test_small_grid_every_output_written():
    """Outputs prefilled with NaN: every row of every head of a ragged small
    grid (B = 3, H = 5, N = 200: 15 heads x 4 blocks of 64 rows) is written,
    and two calls give the same bits."""
    w = fi.Workload("grid_nan_b3_h5_n200", 1160, 3, 5, 200, 128, "bf16", True)
    q, k, v = gu.workload_tensors(w)
    outs = []
    for _ in range(2):
        o = torch.full_like(q, float("nan"))
        lse = torch.full(q.shape[:3], float("nan"), dtype=torch.float32, device=q.device)
        fa.attention_forward(q, k, v, causal=True, scale=w.scale, out=o, lse=lse)
        torch.cuda.synchronize()
        assert bool(torch.isfinite(o).all()) and bool(torch.isfinite(lse).all())
        outs.append((o.clone(), lse.clone()))
    assert torch.equal(outs[0][0], outs[1][0]) and torch.equal(outs[0][1], outs[1][1])
    gu.compare_heads(w, outs[0][0], outs[0][1], [(0, 0), (1, 2), (2, 4)], what=w.name)
