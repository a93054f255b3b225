"""Binding of the measurement probes (include/fa_probe.h, libfa_probe_mi355x.so).

Used by the benchmark only: a clock stamp (shader-clock and constant-rate
counters) and a register-only bf16 MFMA loop, from which it reports the mean
shader clock over its timed launches and the matrix-core rate the chip attains.
"""
from __future__ import annotations

import ctypes
import os

from .build import PROBE_LIB_PATH

_LIB = None


def lib():
    global _LIB
    if _LIB is None:
        if not os.path.exists(PROBE_LIB_PATH):
            raise ImportError(f"{PROBE_LIB_PATH} is not built; run python -m exact_attention_65_amd.build")
        L = ctypes.CDLL(PROBE_LIB_PATH)
        vp = ctypes.c_void_p
        L.fa_probe_stamp.restype = ctypes.c_int
        L.fa_probe_stamp.argtypes = [vp, vp]
        L.fa_probe_mfma_query.restype = ctypes.c_int
        L.fa_probe_mfma_query.argtypes = [ctypes.c_int, ctypes.POINTER(ctypes.c_int), ctypes.POINTER(ctypes.c_double)]
        L.fa_probe_mfma.restype = ctypes.c_int
        L.fa_probe_mfma.argtypes = [ctypes.c_int, vp, vp]
        L.fa_probe_wallclock_khz.restype = ctypes.c_int
        L.fa_probe_wallclock_khz.argtypes = [ctypes.POINTER(ctypes.c_int)]
        _LIB = L
    return _LIB


def _check(rc: int, what: str) -> None:
    if rc != 0:
        raise RuntimeError(f"{what} failed with code {rc}")


def wallclock_khz() -> int:
    k = ctypes.c_int(0)
    _check(lib().fa_probe_wallclock_khz(ctypes.byref(k)), "fa_probe_wallclock_khz")
    return k.value


STAMP_BLOCKS = 2048  # FA_PROBE_STAMP_BLOCKS
STAMP_WORDS = 3 * STAMP_BLOCKS


def stamp(buf, stream) -> None:
    """Enqueue a stamp into buf (a contiguous int64 device tensor of STAMP_WORDS elements)."""
    if buf.numel() < STAMP_WORDS or buf.element_size() != 8 or not buf.is_contiguous():
        raise ValueError("stamp buffer must be a contiguous 64-bit tensor of STAMP_WORDS elements")
    _check(lib().fa_probe_stamp(buf.data_ptr(), stream), "fa_probe_stamp")


def clock_mhz(stamp0, stamp1, wall_khz: int) -> float:
    """Mean shader clock between two stamps (host copies of the stamp buffers),
    per compute unit from that unit's counter, then the median over the units."""
    def per_xcc(s):
        d = {}
        for b in range(STAMP_BLOCKS):
            t, r, x = (int(v) for v in s[3 * b:3 * b + 3])
            d.setdefault(x, (t, r))
        return d
    a, b = per_xcc(stamp0), per_xcc(stamp1)
    clk = sorted((b[x][0] - a[x][0]) / (b[x][1] - a[x][1]) * wall_khz / 1e3
                 for x in a if x in b and b[x][1] > a[x][1])
    return clk[len(clk) // 2] if clk else float("nan")


def mfma_rate(stream, iters: int = 4096, reps: int = 3):
    """bf16 MFMA rate of the register-only loop (best of reps) and the shader
    clock inside it: {"tflops", "ms", "clock_mhz", "blocks"}."""
    import torch
    blocks, flops = ctypes.c_int(0), ctypes.c_double(0.0)
    _check(lib().fa_probe_mfma_query(iters, ctypes.byref(blocks), ctypes.byref(flops)), "fa_probe_mfma_query")
    stamps = torch.zeros(4 * blocks.value, dtype=torch.int64, device="cuda")
    khz = wallclock_khz()
    best = None
    for _ in range(reps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(torch.cuda.current_stream())
        _check(lib().fa_probe_mfma(iters, stamps.data_ptr(), stream), "fa_probe_mfma")
        e1.record(torch.cuda.current_stream())
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1)
        s = stamps.view(blocks.value, 4).cpu().tolist()
        clk = sorted((r[2] - r[0]) / (r[3] - r[1]) * khz / 1e3 for r in s if r[3] > r[1])
        rec = {"tflops": flops.value / (ms * 1e-3) / 1e12, "ms": ms,
               "clock_mhz": clk[len(clk) // 2] if clk else float("nan"), "blocks": blocks.value}
        if best is None or rec["tflops"] > best["tflops"]:
            best = rec
    return best
