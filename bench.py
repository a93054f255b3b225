#!/usr/bin/env python3
"""Benchmark of the exact-attention forward on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]
                    [--split S] [--backward] [--no-cpu-baseline] [--sweep]

A step is one fa_fwd call (the whole hot path: one kernel) over the workload's
synthetic inputs, already resident in device memory.  Prints ONE JSON line:
metric = forward TFLOP/s with 4*B*H*N^2*D FLOPs (halved when causal), the
roofline of the kernel (its FLOPs per launch over its mean launch time from HIP
events on the launch stream, against the bf16 dense MFMA peak), and the CPU
fp64 oracle timed on a bounded sample of the same workload on this host.

Workloads with fewer queries than keys (decode, chunked prefill), and any bf16
workload run with --split S (S key ranges; 0 = the library's choice), step
through fa_fwd_split: the range kernel and the merge kernel, both inside the
timed events.  Their roofline is the HBM one (GB/s of Q, K, V, O and LSE) when
the workload's arithmetic intensity is below the machine balance.

The FP8 workloads (fp8_b2_h32_n4096_d128 and fp8_b2_h16_n4096_d256: E4M3
inputs with MX block scales) step through fa_fwd_fp8; their roofline peak is
the combination of the fp8 and bf16 MFMA peaks (Q K^T runs on the first, P V
on the second).

With --backward a step is one fa_bwd call (its two kernels: dq with Delta, then
dk and dv; on small grids a Delta kernel, then one grid of both kinds of
workgroup) for a seeded upstream gradient, O and LSE having been computed by
fa_fwd before the timed region.  FLOPs are those of the five products of the
gradient, 10*B*H*N^2*D (halved when causal): 2.5 times the forward's, whatever
the kernels recompute.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "fwd attention TFLOP/s (4BHN²D, ÷2 causal) + % of bf16 MFMA peak, N=4096 D=128"
HEADLINE = "bf16_b2_h32_n4096_d128"
# MI355X published dense peaks (TFLOP/s): bf16 MFMA 2516.6 (= 2.5 PFLOP/s), fp8 5033.2, fp32 MFMA 157.3.
# The FP8 path runs Q K^T on the fp8 matrix cores and P V on the bf16 ones, half of the FLOPs each:
# its ceiling is the harmonic combination of the two peaks.
PEAK_FP8_MIXED = 1.0 / (0.5 / 5033.2 + 0.5 / 2516.6)
PEAK_TFLOPS = {"bf16": 2516.6, "f16": 2516.6, "f32": 157.3, "fp8": PEAK_FP8_MIXED}
PEAK_HBM_GBS = 8000.0  # MI355X HBM3E
KERNEL_SOURCES = ["exact_attention_65_amd/csrc/fa_fwd_kernel.hpp", "exact_attention_65_amd/csrc/fa_fwd.hip"]
BWD_FLOP_FACTOR = 2.5  # five N x N x D products against the forward's two
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_fa_fwd_bf16_d128_b2_h32_n4096.txt")


def code_only(src: str) -> str:
    """C++ source with comments removed and whitespace runs collapsed."""
    src = re.sub(r"/\*.*?\*/", " ", src, flags=re.S)
    src = re.sub(r"//[^\n]*", " ", src)
    return " ".join(src.split())


def kernel_hash() -> str:
    """Hash of the kernel sources with comments and whitespace removed, so that an
    edit of comments alone keeps the counter summary valid."""
    h = hashlib.sha256()
    for p in KERNEL_SOURCES:
        with open(os.path.join(ROOT, p), encoding="utf-8") as f:
            h.update(code_only(f.read()).encode())
    return h.hexdigest()[:16]


def read_traffic(workload: str):
    """HBM bytes per launch from the committed rocprofv3 counter summary, or None
    when there is none for this workload or the kernel source changed since."""
    if not os.path.exists(TRAFFIC_FILE):
        return None
    kv = {}
    with open(TRAFFIC_FILE) as f:
        for line in f:
            m = re.match(r"^(\w+):\s*(.+?)\s*$", line)
            if m:
                kv[m.group(1)] = m.group(2)
    if kv.get("workload") != workload or kv.get("kernel_source_sha256_16") != kernel_hash():
        return None
    try:
        return float(kv["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def host_info():
    """CPU model and the cores this process may run on."""
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return {"cpu": model, "cores_available": len(os.sched_getaffinity(0))}


# forward tolerances against the fp64 oracle: max |dO|, mean |dO|, max |dLSE|
FWD_TOL = {"bf16": (2e-2, 2e-3, 1e-3), "f16": (5e-3, 5e-4, 1e-3), "f32": (1e-5, None, 1e-3)}


def cpu_baseline(w, budget_s: float = 12.0, backward: bool = False, gpu_out=None):
    """The fp64 oracle on whole (b, h) heads of the workload until the budget is
    spent (the gradient oracle with --backward), on a BLAS pool of
    min(available cores, 16) threads.  With gpu_out = (O, LSE) as host float
    arrays, the heads it computes are also compared with the GPU's result."""
    import numpy as np
    import threadpoolctl
    import fa_inputs as fi
    from oracle import attention_bwd_ref, attention_ref
    cores = min(len(os.sched_getaffinity(0)), 16)
    heads = [(b, h) for b in range(w.B) for h in range(w.H)]
    done = 0
    t_total = 0.0
    err = {"max_abs_dO": 0.0, "sum_abs_dO": 0.0, "n_O": 0, "max_abs_dLSE": 0.0}
    with threadpoolctl.threadpool_limits(limits=cores):
        for b, h in heads:
            q, k, v = fi.head_qkv(w, b, h)
            do = fi.head_tensor(w, b, h, fi.T_DO) if backward else None
            if w.dtype == "fp8":
                import fa_inputs.fp8 as f8
                from oracle import attention_fp8_ref
                mx = [f8.head_mx(w, b, h, t) for t in (fi.T_Q, fi.T_K, fi.T_V)]
            t0 = time.perf_counter()
            if backward:
                attention_bwd_ref(q, k, v, do, w.causal, w.scale)
                ref = None
            elif w.dtype == "fp8":
                ref = attention_fp8_ref(*mx[0], *mx[1], *mx[2], w.causal, w.scale)
            else:
                ref = attention_ref(q, k, v, w.causal, w.scale)
            t_total += time.perf_counter() - t0
            done += 1
            if gpu_out is not None and ref is not None:
                d_o = np.abs(gpu_out[0][b, h].astype(np.float64) - ref[0])
                d_l = np.abs(gpu_out[1][b, h].astype(np.float64) - ref[1])
                err["max_abs_dO"] = max(err["max_abs_dO"], float(d_o.max()))
                err["sum_abs_dO"] += float(d_o.sum())
                err["n_O"] += d_o.size
                err["max_abs_dLSE"] = max(err["max_abs_dLSE"], float(d_l.max()))
            if t_total >= budget_s:
                break
    flops = w.flops / (w.B * w.H) * done * (BWD_FLOP_FACTOR if backward else 1.0)
    rec = {"value": flops / t_total / 1e12, "unit": "TFLOP/s", "cores": int(cores), "kind": "oracle",
           "sample": f"{done} of {len(heads)} (b,h) heads of {w.name}, every query row, numpy float64 "
                     f"on {cores} BLAS threads ({t_total:.2f} s)"}
    rec.update(host_info())
    parity = None
    if err["n_O"]:
        parity = {"heads": done, "rows": done * w.nq, "max_abs_dO": err["max_abs_dO"],
                  "mean_abs_dO": err["sum_abs_dO"] / err["n_O"], "max_abs_dLSE": err["max_abs_dLSE"]}
        tol = FWD_TOL.get(w.dtype)
        if tol is not None:
            parity["tolerance"] = {"max_abs_dO": tol[0], "mean_abs_dO": tol[1], "max_abs_dLSE": tol[2]}
            parity["pass"] = bool(parity["max_abs_dO"] <= tol[0] and parity["max_abs_dLSE"] <= tol[2]
                                  and (tol[1] is None or parity["mean_abs_dO"] <= tol[1]))
    return rec, parity


def settle(step, seconds: float) -> int:
    """Runs steps for about `seconds` before the warm-up.  After an idle spell the
    chip's launch times first rise by up to a third over some tens of
    milliseconds of load and then settle (power management); the timed steps are
    meant to see the settled state.  Returns the number of steps run."""
    import torch
    n = 0
    t_end = time.perf_counter() + seconds
    while time.perf_counter() < t_end:
        for _ in range(8):
            step()
        n += 8
        torch.cuda.synchronize()
    return n


def naive_context(q, k, v, w, fa_ms, stream, reps: int = 10):
    """Plain torch attention on the same inputs: S = scale Q K^T and P = softmax(S)
    materialised in device memory (the N x N round trip the tiled method avoids),
    then O = P V; both products in the input dtype with the library's fp32
    accumulation, the softmax in fp32.  Reported as context, never as a target."""
    import torch
    kt = k.transpose(-2, -1).contiguous()  # batched 16-bit products take a contiguous right operand
    mask = None
    if w.causal:
        mask = torch.ones(w.N, w.N, dtype=torch.bool, device=q.device).triu(1)

    def naive():
        s = torch.matmul(q, kt).float() * w.scale
        if mask is not None:
            s.masked_fill_(mask, float("-inf"))
        p = torch.softmax(s, dim=-1).to(q.dtype)
        del s
        return torch.matmul(p, v)

    naive()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(reps):
        naive()
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    del kt, mask
    torch.cuda.empty_cache()
    return {"kind": "plain torch attention (matmul, fp32 softmax, matmul), same GPU and inputs",
            "ms_per_call": round(ms, 4), "ratio_to_fa": round(ms / fa_ms, 2)}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default=HEADLINE)
    ap.add_argument("--split", type=int, default=None,
                    help="run through fa_fwd_split with this many key ranges (0 = library's choice)")
    ap.add_argument("--backward", action="store_true",
                    help="time fa_bwd (the gradients) instead of the forward")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--sweep", action="store_true", help="one line per workload instead of the headline")
    ap.add_argument("--naive-context", action="store_true",
                    help="also time plain torch attention (matmul, softmax, matmul with the N x N scores in "
                         "device memory) on the same inputs, as context only")
    ap.add_argument("--settle-s", type=float, default=0.3,
                    help="seconds of untimed steps before the warm-up, for the clock to settle after idle")
    ap.add_argument("--no-probe", action="store_true",
                    help="skip the clock stamps and the MFMA-rate probe")
    ap.add_argument("--calib-copy-mib", type=int, default=0,
                    help="first run a plain device copy of this many MiB (3 times), the known-size "
                         "reference that scales the HBM byte counters")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(json.dumps({"error": "this benchmark runs on exactly one GPU; the attention forward "
                                   "shards over (batch, head) with no exchange, so N GPUs run N "
                                   "independent copies", "n_gpus": args.gpus}))
        sys.exit(2)

    import numpy as np
    import torch
    import exact_attention_65_amd as fa
    import fa_inputs as fi
    from exact_attention_65_amd import probe

    stamps, wall_khz = None, None
    if not args.no_probe:
        stamps = torch.zeros((2, probe.STAMP_WORDS), dtype=torch.int64, device="cuda")
        wall_khz = probe.wallclock_khz()

    if args.calib_copy_mib > 0:
        n = args.calib_copy_mib << 20
        src = torch.ones(n, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    names = [w.name for w in fi.ALL_WORKLOADS + fi.SPLIT_WORKLOADS + fi.FP8_WORKLOADS + fi.BREADTH_WORKLOADS] \
        if args.sweep \
        else [args.workload]
    for name in names:
        w = fi.workload_by_name(name)
        split = args.split if args.split is not None else (fa.FA_SPLIT_AUTO if w.NQ > 0 else None)
        if args.backward:
            split = None
            if w.dtype not in ("bf16", "f16") or w.NQ > 0:
                continue  # the gradients take bf16 or fp16 (and are timed on square shapes)
        if w.dtype == "fp8":
            split = None
        if split is not None and w.dtype not in ("bf16", "f16"):
            continue
        dt = {"bf16": fa.FA_DTYPE_BF16, "f16": fa.FA_DTYPE_F16}.get(w.dtype, fa.FA_DTYPE_F32)
        tensors = []
        if w.dtype == "fp8":
            import fa_inputs.fp8 as f8
            scales = []
            for t in (fi.T_Q, fi.T_K, fi.T_V):
                codes, sc = f8.full_mx(w, t)
                tensors.append(torch.from_numpy(codes).cuda())
                scales.append(torch.from_numpy(sc).cuda())
            q, k, v = tensors
            qs, ks, vs = scales
            o = torch.empty(q.shape, dtype=torch.bfloat16, device=q.device)
        else:
            for t in (fi.T_Q, fi.T_K, fi.T_V):
                bits = fi.full_tensor(w, t)
                x = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16) if w.dtype == "bf16" \
                    else torch.from_numpy(bits.view(np.float16)) if w.dtype == "f16" else torch.from_numpy(bits)
                tensors.append(x.cuda())
                del bits, x
            q, k, v = tensors
            o = torch.empty_like(q)
        lse = torch.empty((w.B, w.H, w.nq), dtype=torch.float32, device=q.device)
        stream = torch.cuda.current_stream()
        sp = stream.cuda_stream
        n_ranges = 1
        if split is not None:
            st, sz, n_ranges = fa.fa_fwd_split_query(w.B, w.H, w.nq, w.N, w.D, w.causal, split, dt)
            if st != fa.FA_OK:
                raise fa.FaError(st)
            ws = torch.empty(max(1, sz.workspace_bytes), dtype=torch.uint8, device=q.device)

        if args.backward:
            bits = fi.full_tensor(w, fi.T_DO)
            do = (torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16) if w.dtype == "bf16"
                  else torch.from_numpy(bits.view(np.float16))).cuda()
            del bits
            fa.attention_forward(q, k, v, causal=w.causal, scale=w.scale, out=o, lse=lse)
            grads = [torch.empty_like(q) for _ in range(3)]
            st, sz = fa.fa_bwd_query(w.B, w.H, w.N, w.D, w.causal, dt)
            if st != fa.FA_OK:
                raise fa.FaError(st)
            ws = torch.empty(sz.workspace_bytes, dtype=torch.uint8, device=q.device)
        flops = w.flops * (BWD_FLOP_FACTOR if args.backward else 1.0)

        def step():
            if w.dtype == "fp8":
                st = fa.fa_fwd_fp8(q.data_ptr(), qs.data_ptr(), k.data_ptr(), ks.data_ptr(), v.data_ptr(),
                                   vs.data_ptr(), o.data_ptr(), lse.data_ptr(), w.B, w.H, w.N, w.D, w.causal,
                                   w.scale, sp)
            elif args.backward:
                st = fa.fa_bwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), do.data_ptr(),
                               lse.data_ptr(), grads[0].data_ptr(), grads[1].data_ptr(), grads[2].data_ptr(),
                               ws.data_ptr(), ws.numel(), w.B, w.H, w.N, w.D, w.causal, w.scale, dt, sp)
            elif split is None:
                st = fa.fa_fwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(),
                               w.B, w.H, w.N, w.D, w.causal, w.scale, dt, sp)
            else:
                st = fa.fa_fwd_split(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(),
                                     ws.data_ptr(), ws.numel(), w.B, w.H, w.nq, w.N, w.D, w.causal, w.scale,
                                     split, dt, sp)
            if st != fa.FA_OK:
                raise fa.FaError(st)

        settle_steps = settle(step, args.settle_s)
        for _ in range(args.warmup):
            step()
        torch.cuda.synchronize()

        # timed region: K back-to-back steps on the launch stream, an event after
        # each, so the per-launch durations come from the same launches as the mean;
        # clock stamps just outside the region give the mean shader clock over it
        evs = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        if stamps is not None:
            probe.stamp(stamps[0], sp)
        evs[0].record(stream)
        for i in range(args.steps):
            step()
            evs[i + 1].record(stream)
        if stamps is not None:
            probe.stamp(stamps[1], sp)
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        region_ms = evs[0].elapsed_time(evs[-1])
        ms_per_step = region_ms / args.steps
        launch_ms = np.array([evs[i].elapsed_time(evs[i + 1]) for i in range(args.steps)])
        clock = None
        if stamps is not None:
            torch.cuda.synchronize()
            st_host = stamps.cpu().tolist()
            clock = round(probe.clock_mhz(st_host[0], st_host[1], wall_khz), 1)

        tflops = flops / (ms_per_step * 1e-3) / 1e12
        peak = PEAK_TFLOPS[w.dtype]
        elt = {"bf16": 2, "f16": 2, "fp8": 1}.get(w.dtype, 4)
        alg_bytes = w.kv_bytes + w.B * w.H * w.nq * w.D * (elt + 2 if w.dtype == "fp8" else 2 * elt) \
            + 4.0 * w.B * w.H * w.nq + (3.0 * w.B * w.H * w.N * w.D / 32 if w.dtype == "fp8" else 0.0)
        hbm_bound = flops / alg_bytes < peak / PEAK_HBM_GBS * 1e3  # intensity below machine balance
        # the roofline is taken from the same timed launches as value
        if hbm_bound:
            gbs = alg_bytes / (ms_per_step * 1e-3) / 1e9
            roofline = {"bound": "hbm", "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                        "frac": round(gbs / PEAK_HBM_GBS, 4), "traffic": None}
        else:
            roofline = {"bound": "mfma", "achieved": round(tflops, 2), "peak": peak, "unit": "TFLOP/s",
                        "frac": round(tflops / peak, 4),
                        "traffic": read_traffic(w.name) if split is None and not args.backward else None}
        roofline["timing"] = "mean of the timed steps (the same launches as value)"
        rec = {
            "metric": "bwd attention TFLOP/s (10*D per visible (query, key) pair) of workload " + w.name
            if args.backward else METRIC if w.name == HEADLINE else
            "fwd attention TFLOP/s (4*D per visible (query, key) pair) of workload " + w.name,
            "value": round(tflops, 2),
            "unit": "TFLOP/s",
            "n_gpus": 1,
            "steps": args.steps,
            "warmup": args.warmup,
            "ms_per_step": round(ms_per_step, 5),
            "higher_is_better": True,
            "scaling": "weak",
            "vs_baseline": None,
            "dtype": "fp8_e4m3 (QK^T) + bf16 (PV)" if w.dtype == "fp8" else w.dtype,
            "data": "synthetic: seeded iid N(0,1) inputs"
                    + (" with Q, K x4 (peaked)" if w.variant == fi.PEAKED else "")
                    + (" rounded to bf16" if w.dtype == "bf16" else "")
                    + (" rounded to fp16" if w.dtype == "f16" else "")
                    + (" quantised to E4M3 with MX block scales (32 along D)" if w.dtype == "fp8" else ""),
            "config": {"workload": w.name, "B": w.B, "H": w.H, "N": w.N, "Nq": w.nq, "D": w.D,
                       "causal": w.causal, "scale": w.scale, "parallelism": "single GPU",
                       "entry_point": "fa_fwd_fp8 (E4M3 with MX block scales)" if w.dtype == "fp8" else
                       "fa_bwd (dq and dk/dv kernels, or both in one grid for small grids)" if args.backward else
                       "fa_fwd" if split is None else f"fa_fwd_split ({n_ranges} key ranges)",
                       "pct_of_peak": round(100 * tflops / peak, 2),
                       "wall_ms_per_step": round(wall * 1e3 / args.steps, 5),
                       "launch_ms_median": round(float(np.median(launch_ms)), 5),
                       "launch_ms_p90": round(float(np.percentile(launch_ms, 90)), 5),
                       "launch_ms_min": round(float(launch_ms.min()), 5),
                       "launch_ms_max": round(float(launch_ms.max()), 5),
                       "settle_steps": settle_steps,
                       "shader_clock_mhz": clock},
            "roofline": roofline,
        }
        if args.naive_context and w.dtype in ("bf16", "f16") and not args.backward and split is None:
            rec["context"] = naive_context(q, k, v, w, ms_per_step, stream)
        if not args.no_probe and not args.sweep:
            m = probe.mfma_rate(sp)
            rec["config"]["mfma_probe"] = {
                "kind": "register-only v_mfma_f32_32x32x16_bf16 loop, 2 waves per SIMD, all CUs",
                "tflops": round(m["tflops"], 1), "clock_mhz": round(m["clock_mhz"], 1)}
            if w.dtype in ("bf16", "f16") or args.backward:
                rec["config"]["pct_of_mfma_probe"] = round(100 * tflops / m["tflops"], 2)
        if not args.no_cpu_baseline and not args.sweep:
            gpu_out = None
            if not args.backward and split is None:
                gpu_out = (o.float().cpu().numpy(), lse.cpu().numpy())
            del q, k, v, o, lse
            torch.cuda.empty_cache()
            rec["cpu_baseline"], parity = cpu_baseline(w, backward=args.backward, gpu_out=gpu_out)
            if parity is not None:
                rec["parity_vs_oracle"] = parity
        print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
