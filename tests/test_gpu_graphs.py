"""Every entry point captured in a HIP graph (torch.cuda.CUDAGraph) and replayed
several times, with the program's own eager launches and synchronisations
between the replays: each replay must reproduce the eager result bit for bit.

The entry points allocate nothing and issue no memset, so a caller may capture
them; the kernels are deterministic, so replays and eager calls agree exactly.
"""
import numpy as np
import pytest
import torch

import exact_attention_65_amd as fa
import fa_inputs as fi
import fa_inputs.fp8 as f8
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu

REPLAYS = 3


def _check_replays(run, outs):
    """run(): launches into the tensors in outs on the current stream."""
    run()
    torch.cuda.synchronize()
    eager = [x.clone() for x in outs]
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        run()  # warm-up on the capture stream
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    with torch.cuda.graph(g, stream=s):
        run()
    for r in range(REPLAYS):
        for x in outs:
            x.fill_(float("nan") if x.is_floating_point() else 0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for a, b in zip(outs, eager):
            assert torch.equal(a.view(torch.uint8), b.view(torch.uint8)), f"replay {r} differs from eager"
        run()  # eager work between replays
        torch.cuda.synchronize()


@pytest.mark.parametrize("B,H,D", [(1, 4, 128), (2, 40, 128), (2, 40, 256)],
                         ids=["small_grid", "large_grid", "large_grid_d256"])
def test_graph_fa_fwd(B, H, D):
    """fa_fwd in a graph: a grid that takes the 64-row small-grid kernel (B=1
    H=4: 28 blocks of 128 rows), one that takes the 128-row kernel (B=2 H=40:
    560 blocks), and the same grid at D = 256 (the 16-row-wave kernel in
    128-row workgroups of 8 waves)."""
    w = fi.Workload(f"graph_fwd_b{B}_h{H}_d{D}", 1100, B, H, 777, D, "bf16", True)
    q, k, v = gu.workload_tensors(w)
    o = torch.empty_like(q)
    lse = torch.empty((B, H, 777), device="cuda")
    _check_replays(lambda: fa.attention_forward(q, k, v, causal=True, scale=w.scale, out=o, lse=lse), [o, lse])


def test_graph_fa_fwd_split():
    w = fi.Workload("graph_split", 1101, 2, 2, 3000, 128, "bf16", True, NQ=5)
    q, k, v = gu.workload_tensors(w)
    o = torch.empty_like(q)
    lse = torch.empty((2, 2, 5), device="cuda")
    st, sz, _ = fa.fa_fwd_split_query(2, 2, 5, 3000, 128, True, 6, fa.FA_DTYPE_BF16)
    assert st == fa.FA_OK
    ws = torch.empty(sz.workspace_bytes, dtype=torch.uint8, device="cuda")
    _check_replays(lambda: fa.attention_forward_split(q, k, v, causal=True, scale=w.scale, n_splits=6, out=o,
                                                      lse=lse, workspace=ws), [o, lse])


@pytest.mark.parametrize("D", [128, 256])
def test_graph_fa_bwd(D):
    """fa_bwd in a graph: at D = 128 the small grid takes the one-grid plan
    (Delta kernel, then both kinds of workgroup), at D = 256 the dq kernel
    and the 16-key dk/dv kernel."""
    w = fi.Workload(f"graph_bwd_d{D}", 1102, 1, 2, 600, D, "bf16", True)
    q, k, v = gu.workload_tensors(w)
    do = gu.to_device_bits(fi.full_tensor(w, fi.T_DO), "bf16")
    o, lse = fa.attention_forward(q, k, v, causal=True, scale=w.scale)
    grads = [torch.empty_like(q) for _ in range(3)]
    st, sz = fa.fa_bwd_query(1, 2, 600, D, True, fa.FA_DTYPE_BF16)
    ws = torch.empty(sz.workspace_bytes, dtype=torch.uint8, device="cuda")
    _check_replays(lambda: fa.attention_backward(q, k, v, o, lse, do, causal=True, scale=w.scale, dq=grads[0],
                                                 dk=grads[1], dv=grads[2], workspace=ws), grads)


def test_graph_fa_fwd_fp8():
    w = fi.Workload("graph_fp8", 1103, 1, 2, 500, 128, "fp8", False)
    (q, qs), (k, ks), (v, vs) = [tuple(torch.from_numpy(np.ascontiguousarray(x)).cuda() for x in f8.full_mx(w, t))
                                 for t in (fi.T_Q, fi.T_K, fi.T_V)]
    o = torch.empty((1, 2, 500, 128), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((1, 2, 500), device="cuda")
    _check_replays(lambda: fa.attention_forward_fp8(q, qs, k, ks, v, vs, causal=False, scale=w.scale, out=o,
                                                    lse=lse), [o, lse])
