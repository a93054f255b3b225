"""Seeded synthetic inputs for the exact-attention forward.

This module is shared by the CPU oracle side (tests, the oracle timing in the
benchmark) and by the GPU side (tests, benchmark, smoke).  It holds no part of
the attention arithmetic: it only draws random numbers, rounds them to the
element type the kernel reads, and picks the seeded samples of (batch, head)
pairs and query rows that the large workloads are checked on.

Distribution.  The pages build their workloads from standard-normal tensors of
shape [batch, heads, seq_len, head_dim] ("Flash Attention: ускорить attention в
6 раз без потери точности", johe.ru, sections "Использование в коде" and
"Сравнение производительности").  Every (config, variant, b, h, tensor) slice
is drawn from its own numpy PCG64 stream keyed by a SeedSequence, so any slice
can be regenerated on its own, on any machine, bit for bit.

bf16 rounding is round-to-nearest-even, written out on the float32 bit
pattern (the same rounding torch uses for ``.to(torch.bfloat16)``; a CPU test
checks the two agree).
"""
from __future__ import annotations

import math
import os
from concurrent.futures import ProcessPoolExecutor
from dataclasses import dataclass, field

import numpy as np

# tensor ids inside the seed key; T_DO is the upstream gradient of the output
# (the gradients' input: standard normal like the others, never scaled by the
# peaked variant)
T_Q, T_K, T_V, T_DO = 0, 1, 2, 3
# variant ids
PLAIN, PEAKED = 0, 1
PEAK_FACTOR = 4.0  # exact in binary: multiplying before rounding loses nothing extra


@dataclass(frozen=True)
class Workload:
    """One synthetic workload: shapes, element type, mask and the seed key."""

    name: str
    seed_id: int
    B: int
    H: int
    N: int
    D: int
    dtype: str  # "f32", "bf16", "f16" or "fp8" (E4M3 codes with MX block scales: fa_inputs.fp8)
    causal: bool
    variant: int = PLAIN
    NQ: int = 0  # query rows per head; 0: as many as keys (N)

    @property
    def nq(self) -> int:
        return self.NQ if self.NQ > 0 else self.N

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.D)

    @property
    def flops(self) -> float:
        """Metric FLOPs of one forward: 4*B*H*D times the (query, key) pairs,
        N^2 (halved when causal) with as many queries as keys; with fewer
        queries, Nq*N, or under the causal mask Nq*(N - Nq) + Nq^2/2."""
        nq, nk = self.nq, self.N
        if nq == nk:
            pairs = nk * nk / (2.0 if self.causal else 1.0)
        else:
            pairs = nq * (nk - nq) + nq * nq / 2.0 if self.causal else float(nq * nk)
        return 4.0 * self.B * self.H * self.D * pairs

    @property
    def kv_bytes(self) -> float:
        """Bytes of K and V (the stream a decode step is bound by)."""
        return 2.0 * self.B * self.H * self.N * self.D * {"bf16": 2, "f16": 2, "fp8": 1}.get(self.dtype, 4)

    def rows(self, t: int) -> int:
        """Rows of tensor t in one head: nq for Q and dO, N for K and V."""
        return self.nq if t in (T_Q, T_DO) else self.N

    def with_variant(self, variant: int) -> "Workload":
        return Workload(self.name + ("_peaked" if variant == PEAKED else ""), self.seed_id,
                        self.B, self.H, self.N, self.D, self.dtype, self.causal, variant, self.NQ)


# The five workloads attention is checked and measured on.
FP32_SMALL = Workload("f32_b1_h1_n256_d64", 1, 1, 1, 256, 64, "f32", False)
BF16_N4096 = Workload("bf16_b2_h32_n4096_d128", 2, 2, 32, 4096, 128, "bf16", False)
CAUSAL_SWEEP_N = (512, 1024, 2048, 4096, 8192)
CAUSAL_SWEEP = tuple(
    Workload(f"bf16_causal_b1_h32_n{n}_d128", 30 + i, 1, 32, n, 128, "bf16", True)
    for i, n in enumerate(CAUSAL_SWEEP_N))
CAUSAL_PREFILL = Workload("bf16_causal_b32_h32_n4096_d128", 4, 32, 32, 4096, 128, "bf16", True)
CAUSAL_LONG = Workload("bf16_causal_b1_h8_n131072_d128", 5, 1, 8, 131072, 128, "bf16", True)

ALL_WORKLOADS = (FP32_SMALL, BF16_N4096) + CAUSAL_SWEEP + tuple(
    w.with_variant(PEAKED) for w in CAUSAL_SWEEP) + (CAUSAL_PREFILL, CAUSAL_LONG)

# Workloads of the split-key path (queries fewer than keys): one new token per
# head against a kept KV cache, and a 512-token chunk of a prompt whose first
# 7680 tokens are already in the cache.
SPLIT_DECODE = Workload("bf16_decode_b4_h32_nq1_nk16384_d128", 40, 4, 32, 16384, 128, "bf16", True, NQ=1)
SPLIT_CHUNK = Workload("bf16_chunk_b1_h32_nq512_nk8192_d128", 41, 1, 32, 8192, 128, "bf16", True, NQ=512)
SPLIT_WORKLOADS = (SPLIT_DECODE, SPLIT_CHUNK)


# FP8 inputs at the headline shape: Q, K, V drawn like the bf16 workload's and
# quantised to E4M3 with MX block scales (fa_inputs.fp8).
FP8_N4096 = Workload("fp8_b2_h32_n4096_d128", 6, 2, 32, 4096, 128, "fp8", False)
# and at head dimension 256 (the headline's element count with half the heads)
FP8_D256_N4096 = Workload("fp8_b2_h16_n4096_d256", 10, 2, 16, 4096, 256, "fp8", False)
FP8_WORKLOADS = (FP8_N4096, FP8_D256_N4096)
# fp16 inputs at the headline shape
F16_N4096 = Workload("f16_b2_h32_n4096_d128", 7, 2, 32, 4096, 128, "f16", False)
# head dimension 256: the headline's bytes with half the heads; head dimension 96
D256_N4096 = Workload("bf16_b2_h16_n4096_d256", 8, 2, 16, 4096, 256, "bf16", False)
D96_N4096 = Workload("bf16_b2_h32_n4096_d96", 9, 2, 32, 4096, 96, "bf16", False)
BREADTH_WORKLOADS = (F16_N4096, D256_N4096, D96_N4096)


def workload_by_name(name: str) -> Workload:
    for w in ALL_WORKLOADS + SPLIT_WORKLOADS + FP8_WORKLOADS + BREADTH_WORKLOADS:
        if w.name == name:
            return w
    raise KeyError(name)


# ---------------------------------------------------------------- rounding
def bf16_round(x: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bfloat16 (ties to even); returns float32.

    NaN stays NaN; values that overflow bf16 become +-inf like an IEEE rounding.
    """
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    lsb = (u >> 16) & 1
    r = ((u + 0x7FFF + lsb) >> 16) << 16
    out = r.astype(np.uint32).view(np.float32)
    nan = np.isnan(x)
    if nan.any():
        out = out.copy()
        out[nan] = np.nan
    return out


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """The uint16 bf16 bit patterns of float32 values that are exactly bf16."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32)
    if np.any(u & 0xFFFF):
        raise ValueError("values are not exactly representable in bf16")
    return (u >> 16).astype(np.uint16)


# ---------------------------------------------------------------- drawing
def _stream(seed_id: int, variant: int, b: int, h: int, t: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed_id, variant, b, h, t])))


def head_tensor(w: Workload, b: int, h: int, t: int) -> np.ndarray:
    """One [rows, D] slice of tensor t (T_Q/T_K/T_V/T_DO) as float32 values of w.dtype
    (rows = nq for Q and dO, N for K and V)."""
    x = _stream(w.seed_id, w.variant, b, h, t).standard_normal((w.rows(t), w.D), dtype=np.float32)
    if w.variant == PEAKED and t in (T_Q, T_K):
        x *= np.float32(PEAK_FACTOR)
    if w.dtype == "bf16":
        x = bf16_round(x)
    elif w.dtype == "f16":
        x = x.astype(np.float16).astype(np.float32)  # round to nearest even
    return x


def head_qkv(w: Workload, b: int, h: int):
    """(q, k, v) for one (b, h): float32 arrays [rows, D] holding exactly the kernel's inputs."""
    return tuple(head_tensor(w, b, h, t) for t in (T_Q, T_K, T_V))


def _fill_one(args):
    w, b, h, t, path, offset = args
    x = head_tensor(w, b, h, t)
    if w.dtype in ("bf16", "f16"):
        arr = np.memmap(path, dtype=np.uint16, mode="r+", offset=offset, shape=(w.rows(t), w.D))
        arr[:] = bf16_bits(x) if w.dtype == "bf16" else x.astype(np.float16).view(np.uint16)
    else:
        arr = np.memmap(path, dtype=np.float32, mode="r+", offset=offset, shape=(w.rows(t), w.D))
        arr[:] = x
    arr.flush()
    del arr
    return None


def full_tensor(w: Workload, t: int, workers: int | None = None) -> np.ndarray:
    """The whole [B, H, rows, D] tensor t, as raw element bits (uint16 for bf16, float32 for f32).

    Slices are drawn in parallel worker processes when the tensor is large.
    """
    dt = np.uint16 if w.dtype in ("bf16", "f16") else np.float32
    shape = (w.B, w.H, w.rows(t), w.D)
    n_slices = w.B * w.H
    slice_elems = w.rows(t) * w.D
    if workers is None:
        workers = min(16, len(os.sched_getaffinity(0)))
    if n_slices * slice_elems < (1 << 22) or workers <= 1:
        out = np.empty(shape, dtype=dt)
        for b in range(w.B):
            for h in range(w.H):
                x = head_tensor(w, b, h, t)
                out[b, h] = bf16_bits(x) if w.dtype == "bf16" else \
                    x.astype(np.float16).view(np.uint16) if w.dtype == "f16" else x
        return out
    import tempfile
    with tempfile.NamedTemporaryFile(dir="/dev/shm" if os.path.isdir("/dev/shm") else None,
                                     delete=True) as f:
        nbytes = n_slices * slice_elems * np.dtype(dt).itemsize
        f.truncate(nbytes)
        jobs = [(w, b, h, t, f.name, (b * w.H + h) * slice_elems * np.dtype(dt).itemsize)
                for b in range(w.B) for h in range(w.H)]
        with ProcessPoolExecutor(max_workers=workers) as ex:
            list(ex.map(_fill_one, jobs, chunksize=max(1, len(jobs) // (4 * workers))))
        out = np.fromfile(f.name, dtype=dt).reshape(shape)
    return out


# ---------------------------------------------------------------- sampling
def sample_heads(w: Workload, count: int) -> list[tuple[int, int]]:
    """Seeded (b, h) pairs, drawn without replacement, sorted."""
    g = _stream(w.seed_id, 0, 999, 0, 0)
    flat = g.choice(w.B * w.H, size=min(count, w.B * w.H), replace=False)
    return sorted((int(i) // w.H, int(i) % w.H) for i in flat)


def sample_rows(w: Workload, h: int, count: int, edges: bool = True) -> np.ndarray:
    """Seeded query rows of head h, without replacement, plus the first and last row, sorted."""
    g = _stream(w.seed_id, 0, 999, h, 1)
    rows = set(int(i) for i in g.choice(w.nq, size=min(count, w.nq), replace=False))
    if edges:
        rows |= {0, w.nq - 1}
    return np.array(sorted(rows), dtype=np.int64)
