"""fa_fwd_split_static (the split forward on the library's own scratch) against
fa_fwd_split with a caller workspace: two calls in a row, the second with a
smaller input, each equal bit for bit to the workspace path (same kernels, same
key ranges)."""
import numpy as np
import pytest
import torch

import exact_attention_65_amd as fa
import fa_inputs as fi
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu


def _inputs(w):
    q = gu.to_device_bits(fi.full_tensor(w, fi.T_Q), w.dtype)
    k = gu.to_device_bits(fi.full_tensor(w, fi.T_K), w.dtype)
    v = gu.to_device_bits(fi.full_tensor(w, fi.T_V), w.dtype)
    return q, k, v


def _both(w, n_splits):
    q, k, v = _inputs(w)
    dt = fa.FA_DTYPE_BF16 if w.dtype == "bf16" else fa.FA_DTYPE_F16
    st, sz, n = fa.fa_fwd_split_query(w.B, w.H, w.nq, w.N, w.D, w.causal, n_splits, dt)
    assert st == fa.FA_OK and sz.workspace_bytes <= fa.FA_STATIC_SCRATCH_BYTES
    s = torch.cuda.current_stream().cuda_stream
    o_ws = torch.full(q.shape, float("nan"), dtype=q.dtype, device=q.device)
    l_ws = torch.full(q.shape[:3], float("nan"), dtype=torch.float32, device=q.device)
    ws = torch.empty(max(1, sz.workspace_bytes), dtype=torch.uint8, device=q.device)
    st = fa.fa_fwd_split(q.data_ptr(), k.data_ptr(), v.data_ptr(), o_ws.data_ptr(), l_ws.data_ptr(), ws.data_ptr(),
                         ws.numel(), w.B, w.H, w.nq, w.N, w.D, w.causal, w.scale, n_splits, dt, s)
    assert st == fa.FA_OK
    o_st = torch.full_like(o_ws, float("nan"))
    l_st = torch.full_like(l_ws, float("nan"))
    st = fa.fa_fwd_split_static(q.data_ptr(), k.data_ptr(), v.data_ptr(), o_st.data_ptr(), l_st.data_ptr(),
                                w.B, w.H, w.nq, w.N, w.D, w.causal, w.scale, n_splits, dt, s)
    assert st == fa.FA_OK, fa.fa_status_str(st)
    torch.cuda.synchronize()
    return n, (o_ws, l_ws), (o_st, l_st)


@pytest.mark.parametrize("first,second", [
    # chunked prefill (4 ranges, 33.8 MB of partials), then a decode step (1 query row, 4 ranges)
    (("chunk", 4), ("decode", 4)),
    # two causal calls on the 128-row kernel's split path, the second smaller
    (("sq1024", 7), ("sq300", 3)),
])
def test_static_scratch_matches_workspace_path(first, second):
    shapes = {
        "chunk": fi.Workload("static_chunk", 961, 1, 32, 8192, 128, "bf16", True, NQ=512),
        "decode": fi.Workload("static_decode", 962, 4, 32, 16384, 128, "bf16", True, NQ=1),
        "sq1024": fi.Workload("static_sq1024", 963, 1, 8, 1024, 128, "bf16", True),
        "sq300": fi.Workload("static_sq300", 964, 1, 4, 300, 64, "bf16", True),
    }
    for name, n_splits in (first, second):
        w = shapes[name]
        gu.log(f"[gpu] fa_fwd_split_static {w.name}: B={w.B} H={w.H} Nq={w.nq} Nk={w.N} D={w.D} ranges={n_splits}")
        n, (o_ws, l_ws), (o_st, l_st) = _both(w, n_splits)
        assert n == n_splits
        assert torch.isfinite(o_st.float()).all() and torch.isfinite(l_st).all()
        assert torch.equal(o_st, o_ws) and torch.equal(l_st, l_ws), w.name
        # and both agree with the oracle on two heads (the split path's own parity bar)
        gu.compare_heads(w, o_st, l_st, [(0, 0), (w.B - 1, w.H - 1)], what=w.name + " static scratch")
