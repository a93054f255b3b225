"""The one-range 16-bit forward at D = 64, 96, 128 and 256 on its launch
forms, against the fp64 oracle.

fa_fwd (and fa_fwd_split with one range) runs grids of at most one 128-row
workgroup per compute unit (B * H * ceil(Nq / 128) <= CU count) on a kernel
with 64 rows per workgroup in slices of 16: at D = 64, 96 and 128 with two waves
per slice when its 64-row grid fits one workgroup per CU and one wave per
slice otherwise, at D = 256 always with two.  Larger grids run the 128-row
kernel, or at D = 256 the same 16-row-wave kernel in 128-row workgroups of
8 waves.  Each case runs the same heads with H = 2 (two waves per slice), with
the smallest H for one wave per slice (when the shape has one; at D = 256 a
second grid of two waves per slice) and with the smallest H for the 128-row
workgroups on this device.  A head's inputs depend only on its (b, h) and the
seed, so heads 0 and 1 are the same in every run; each run is checked against
the oracle on heads 0, 1 and the last, every row and column.
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
    """H for each launch form the shape has: two waves per slice, one wave per
    slice, the 128-row kernel."""
    cus = _cus()
    b64, b128 = math.ceil(nq / 64), math.ceil(nq / 128)
    hs = [2]
    assert 2 * b64 <= cus
    h1 = cus // b64 + 1
    if h1 * b128 <= cus:
        hs.append(h1)
    hs.append(cus // b128 + 1)
    return hs


def _both_kernels(name, seed, nq, nk, dtype, causal, forward, D=128):
    results = []
    for H in _head_counts(nq):
        w = fi.Workload(f"{name}_h{H}", seed, 1, H, nk, D, dtype, causal, NQ=nq if nq != nk else 0)
        gu.log(f"[gpu] {w.name}: Nq={nq} Nk={nk} {dtype} causal={causal}")
        q, k, v = gu.workload_tensors(w)
        o, lse = forward(w, q, k, v)
        torch.cuda.synchronize()
        gu.compare_heads(w, o, lse, [(0, 0), (0, 1), (0, H - 1)], what=f"{w.name} causal={causal}")
        results.append((H, o[:, :2].float().cpu(), lse[:, :2].cpu()))
    h0, o0, l0 = results[0]
    for h1, o1, l1 in results[1:]:
        gu.log(f"  heads 0-1, H={h0} vs H={h1}: max|dO| {float((o0 - o1).abs().max()):.3e} "
               f"max|dLSE| {float((l0 - l1).abs().max()):.3e}")


@pytest.mark.parametrize("D", [64, 96, 128, 256])
@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("N", EDGE_N)
def test_fwd_small_and_large_grids(N, causal, dtype, D):
    seed = 1100 + 2 * EDGE_N.index(N) + causal

    def forward(w, q, k, v):
        return fa.attention_forward(q, k, v, causal=causal, scale=w.scale)

    _both_kernels(f"grid_n{N}_d{D}", seed, N, N, dtype, causal, forward, D)


@pytest.mark.parametrize("D", [64, 96, 128, 256])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("nq,nk", [(5, 300), (100, 1000), (257, 4096), (512, 8192)])
def test_split_one_range_small_and_large_grids(nq, nk, causal, D):
    """Nq queries against Nk keys (the queries are the last Nq positions under
    the causal mask) through fa_fwd_split with one range."""
    seed = 1130 + nq % 11 + causal

    def forward(w, q, k, v):
        return fa.attention_forward_split(q, k, v, causal=causal, scale=w.scale, n_splits=1)

    _both_kernels(f"split1_nq{nq}_nk{nk}_d{D}", seed, nq, nk, "bf16", causal, forward, D)


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


@pytest.mark.parametrize("D", [64, 96, 128, 256])
@pytest.mark.parametrize("B,H", [(3, 5), (2, 40)])
def test_small_grid_every_output_written(B, H, D):
    """Outputs prefilled with NaN: every row of every head of a ragged small
    grid (N = 200: 4 blocks of 64 rows per head; 60 blocks take two waves per
    slice, 320 one wave per slice) is written, and two calls give the same
    bits."""
    w = fi.Workload(f"grid_nan_b{B}_h{H}_n200_d{D}", 1160, B, H, 200, D, "bf16", True)
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
    gu.compare_heads(w, outs[0][0], outs[0][1], [(0, 0), (1, 2), (B - 1, H - 1)], what=w.name)


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("causal", [False, True])
def test_d256_large_grid_every_output_written(causal, dtype):
    """D = 256 on a grid of more 128-row blocks than CUs (the 8-wave form):
    N = 333 (3 blocks per head, the last of 77 rows), outputs prefilled with
    NaN, every output written, two calls give the same bits, and heads at both
    ends of the grid match the oracle."""
    B, H = 3, _cus() // 9 + 1
    assert B * H * 3 > _cus()
    w = fi.Workload(f"grid_d256_{dtype}_b{B}_h{H}_n333", 1170 + causal, B, H, 333, 256, dtype, causal)
    gu.log(f"[gpu] {w.name}: causal={causal}")
    q, k, v = gu.workload_tensors(w)
    outs = []
    for _ in range(2):
        o = torch.full_like(q, float("nan"))
        lse = torch.full(q.shape[:3], float("nan"), dtype=torch.float32, device=q.device)
        fa.attention_forward(q, k, v, causal=causal, scale=w.scale, out=o, lse=lse)
        torch.cuda.synchronize()
        assert bool(torch.isfinite(o).all()) and bool(torch.isfinite(lse).all())
        outs.append((o.clone(), lse.clone()))
    assert torch.equal(outs[0][0], outs[1][0]) and torch.equal(outs[0][1], outs[1][1])
    gu.compare_heads(w, outs[0][0], outs[0][1], [(0, 0), (1, H // 2), (B - 1, H - 1)], what=w.name)
