"""Causal grids whose (batch x head) count gives each XCD 2, 5 or 6 heads.

Under the causal mask the kernels order their work items per XCD, longest
first across groups of up to 4 heads, when B*H is a multiple of 8 (groups of 4,
2 or 1 heads depending on how many heads an XCD holds).  These cases check,
against the fp64 oracle on every head and row, that each (head, block) of such
grids is computed exactly once: every output is prefilled with NaN, so a block
that no workgroup takes fails, and a block taken twice with the wrong head
gives wrong values.
"""
import numpy as np
import pytest
import torch

import exact_attention_65_amd as fa
import fa_inputs as fi
from oracle import attention_bwd_ref
from tests import gpu_util as gu
from tests import error_models as em
from tests.test_gpu_backward import REL_FRO, _grad_errors
from tests.test_gpu_fp8 import _compare as fp8_compare
from tests.test_gpu_fp8 import _dev, _inputs as fp8_inputs

pytestmark = pytest.mark.gpu

# (B, H): B*H = 16 (2 heads per XCD), 40 (5: groups of 1), 48 (6: groups of 2)
HEAD_COUNTS = [(1, 16), (5, 8), (2, 24)]


def _nan_like(shape, dtype):
    return torch.full(shape, float("nan"), dtype=dtype, device="cuda")


def _all_heads(w):
    return [(b, h) for b in range(w.B) for h in range(w.H)]


@pytest.mark.parametrize("dtype", ["bf16", "f16", "f32"])
@pytest.mark.parametrize("bh", HEAD_COUNTS)
def test_forward_causal_head_groups(bh, dtype):
    B, H = bh
    w = fi.Workload(f"order_fwd_{dtype}_b{B}_h{H}", 960 + HEAD_COUNTS.index(bh), B, H, 300, 64, dtype, True)
    gu.log(f"[gpu] causal order forward {w.name}: B={B} H={H} N=300 D=64 {dtype}")
    q, k, v = gu.workload_tensors(w)
    o = _nan_like(q.shape, q.dtype)
    lse = _nan_like((B, H, w.N), torch.float32)
    fa.attention_forward(q, k, v, causal=True, scale=w.scale, out=o, lse=lse)
    torch.cuda.synchronize()
    gu.compare_heads(w, o, lse, _all_heads(w), what=w.name)


@pytest.mark.parametrize("splits", [2, 3])
def test_split_causal_head_groups(splits):
    B, H = 2, 24
    w = fi.Workload(f"order_split{splits}_b{B}_h{H}", 964, B, H, 300, 64, "bf16", True)
    gu.log(f"[gpu] causal order split {w.name}: B={B} H={H} N=300 D=64 ranges={splits}")
    q, k, v = gu.workload_tensors(w)
    o = _nan_like(q.shape, q.dtype)
    lse = _nan_like((B, H, w.N), torch.float32)
    fa.attention_forward_split(q, k, v, causal=True, scale=w.scale, n_splits=splits, out=o, lse=lse)
    torch.cuda.synchronize()
    gu.compare_heads(w, o, lse, _all_heads(w), what=w.name)


@pytest.mark.parametrize("bh", HEAD_COUNTS[1:])
def test_backward_causal_head_groups(bh):
    B, H = bh
    w = fi.Workload(f"order_bwd_b{B}_h{H}", 966 + HEAD_COUNTS.index(bh), B, H, 200, 64, "bf16", True)
    gu.log(f"[gpu] causal order backward {w.name}: B={B} H={H} N=200 D=64")
    q, k, v = gu.workload_tensors(w)
    do = gu.to_device_bits(fi.full_tensor(w, fi.T_DO), w.dtype)
    o, lse = fa.attention_forward(q, k, v, causal=True, scale=w.scale)
    grads = [_nan_like(q.shape, q.dtype) for _ in range(3)]
    fa.attention_backward(q, k, v, o, lse, do, causal=True, scale=w.scale, dq=grads[0], dk=grads[1], dv=grads[2])
    torch.cuda.synchronize()
    worst = {n: 0.0 for n in ("dq", "dk", "dv")}
    for b, h in _all_heads(w):
        qh, kh, vh = fi.head_qkv(w, b, h)
        doh = fi.head_tensor(w, b, h, fi.T_DO)
        refs = attention_bwd_ref(qh, kh, vh, doh, True, w.scale)
        bounds = em.backward_bounds(qh, kh, vh, doh, True, w.scale, w.dtype)
        for name, g, ref, bd in zip(("dq", "dk", "dv"), grads, refs, bounds):
            e = _grad_errors(g[b, h].float().cpu().numpy(), ref, bd)
            assert e["finite"], f"{w.name} {name} (b={b}, h={h}): non-finite gradient"
            assert e["fro"] <= REL_FRO and e["elem"] <= 1.0, f"{w.name} {name} (b={b}, h={h}): {e}"
            worst[name] = max(worst[name], e["elem"])
    gu.log(f"  {w.name}: worst error / bound " + " ".join(f"{n}={v:.3f}" for n, v in worst.items()))


def test_fp8_causal_head_groups():
    B, H = 2, 24
    w = fi.Workload(f"order_fp8_b{B}_h{H}", 969, B, H, 200, 64, "fp8", True)
    gu.log(f"[gpu] causal order fp8 {w.name}: B={B} H={H} N=200 D=64")
    inp = fp8_inputs(w)
    (q, qs), (k, ks), (v, vs) = inp
    o = _nan_like((B, H, w.N, w.D), torch.bfloat16)
    lse = _nan_like((B, H, w.N), torch.float32)
    fa.attention_forward_fp8(_dev(q), _dev(qs), _dev(k), _dev(ks), _dev(v), _dev(vs), causal=True, scale=w.scale,
                             out=o, lse=lse)
    torch.cuda.synchronize()
    fp8_compare(inp, o, lse, _all_heads(w), True, w.scale, w.name)
