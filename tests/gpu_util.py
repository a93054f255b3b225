"""Helpers of the GPU parity tests: seeded inputs on the device, the HIP call,
and the comparison with the fp64 oracle at the tolerances of the contract.

Tolerances (O against the oracle on the same rounded inputs; LSE absolute),
the contract's, fixed for every test:
  float32 inputs: max |dO| <= 1e-5, |dLSE| <= 1e-3
  bf16 inputs:    max |dO| <= 2e-2 and mean |dO| <= 2e-3, |dLSE| <= 1e-3
  fp16 inputs:    the bf16 bounds / 4 (fp16's unit roundoff is 2^-11 against
                  bf16's 2^-8: an eighth, kept at a quarter for margin)

An fp32 score carries a rounding error proportional to its magnitude, so fp32
stress inputs with large scores (a large scale, a +1000 shift) are built with
exactly representable scores (test_gpu_parity._inputs) rather than given a
looser bound.
"""
from __future__ import annotations

import json
import os
import sys

import numpy as np
import torch

import exact_attention_65_amd as fa
import fa_inputs as fi
from oracle import attention_ref

TOL = {
    "f32": dict(o_max=1e-5, o_mean=None, lse=1e-3),
    "bf16": dict(o_max=2e-2, o_mean=2e-3, lse=1e-3),
    # fp16 rounds P and O with unit roundoff 2^-11, an eighth of bf16's 2^-8 (a quarter kept)
    "f16": dict(o_max=5e-3, o_mean=5e-4, lse=1e-3),
}
TORCH_DT = {"f32": torch.float32, "bf16": torch.bfloat16, "f16": torch.float16}


def log(msg: str):
    sys.__stderr__.write(msg + "\n")
    sys.__stderr__.flush()


def record(entry: dict):
    path = os.environ.get("FA_PARITY_LOG")
    if path:
        with open(path, "a") as f:
            f.write(json.dumps(entry) + "\n")


def to_device_bits(arr: np.ndarray, dtype: str) -> torch.Tensor:
    """Raw element bits (uint16 for bf16, float32) -> device tensor of that dtype."""
    if dtype == "bf16":
        t = torch.from_numpy(np.ascontiguousarray(arr).view(np.int16)).view(torch.bfloat16)
    elif dtype == "f16":
        t = torch.from_numpy(np.ascontiguousarray(arr).view(np.float16))
    else:
        t = torch.from_numpy(np.ascontiguousarray(arr, dtype=np.float32))
    return t.cuda()


def to_device_values(x: np.ndarray, dtype: str) -> torch.Tensor:
    """float32 values exactly representable in dtype -> device tensor of that dtype."""
    if dtype == "bf16":
        return to_device_bits(fi.bf16_bits(np.asarray(x, dtype=np.float32)), dtype)
    if dtype == "f16":
        return to_device_bits(np.asarray(x, dtype=np.float32).astype(np.float16).view(np.uint16), dtype)
    return to_device_bits(np.asarray(x, dtype=np.float32), dtype)


def workload_tensors(w: fi.Workload):
    return tuple(to_device_bits(fi.full_tensor(w, t), w.dtype) for t in (fi.T_Q, fi.T_K, fi.T_V))


def run(q, k, v, causal, scale, stream=None):
    o, lse = fa.attention_forward(q, k, v, causal=causal, scale=scale, stream=stream)
    torch.cuda.synchronize()
    return o, lse


def errors(o_gpu, lse_gpu, o_ref, lse_ref):
    do = np.abs(np.asarray(o_gpu, dtype=np.float64) - o_ref)
    dl = np.abs(np.asarray(lse_gpu, dtype=np.float64) - lse_ref)
    return dict(o_max=float(do.max()) if do.size else 0.0, o_mean=float(do.mean()) if do.size else 0.0,
                lse_max=float(dl.max()) if dl.size else 0.0,
                finite=bool(np.all(np.isfinite(o_gpu)) and np.all(np.isfinite(lse_gpu))))


def assert_within(err: dict, dtype: str, what: str):
    t = dict(TOL[dtype])
    record(dict(case=what, dtype=dtype, **err))
    log(f"  {what}: max|dO|={err['o_max']:.3e} mean|dO|={err['o_mean']:.3e} max|dLSE|={err['lse_max']:.3e}")
    assert err["finite"], f"{what}: non-finite output"
    assert err["o_max"] <= t["o_max"], f"{what}: max|dO| {err['o_max']} > {t['o_max']}"
    if t["o_mean"] is not None:
        assert err["o_mean"] <= t["o_mean"], f"{what}: mean|dO| {err['o_mean']} > {t['o_mean']}"
    assert err["lse_max"] <= t["lse"], f"{what}: max|dLSE| {err['lse_max']} > {t['lse']}"


def compare_heads(w: fi.Workload, o, lse, heads, rows_for=None, what=""):
    """Oracle on the given (b, h) pairs (all rows, or rows_for(h)) vs the device result."""
    o_err, l_err = [], []
    n_el = 0
    mean_acc = 0.0
    for b, h in heads:
        q, k, v = fi.head_qkv(w, b, h)
        rows = None if rows_for is None else rows_for(h)
        o_ref, lse_ref = attention_ref(q, k, v, w.causal, w.scale, rows=rows)
        og = o[b, h].float().cpu().numpy()
        lg = lse[b, h].cpu().numpy()
        if rows is not None:
            og, lg = og[rows], lg[rows]
        e = errors(og, lg, o_ref, lse_ref)
        assert e["finite"], f"{what} (b={b}, h={h}): non-finite output"
        o_err.append(e["o_max"])
        l_err.append(e["lse_max"])
        mean_acc += e["o_mean"] * o_ref.size
        n_el += o_ref.size
    err = dict(o_max=max(o_err), o_mean=mean_acc / n_el, lse_max=max(l_err), finite=True)
    assert_within(err, w.dtype, what or w.name)
    return err
