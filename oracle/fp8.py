"""CPU fp64 oracle for attention on FP8 inputs with MX block scales.

TEST INFRASTRUCTURE ONLY (same rules as oracle/attention.py: only tests, the
smoke check and the benchmark's CPU-baseline leg use it; no product code).

The pages name FP8 support and block-scaled attention among the later
FlashAttention versions ("Flash Attention: ускорить attention в 6 раз без
потери точности", sections "Flash Attention 3" and "Flash Attention 4") and
say nothing more.  Reading: the inputs are OCP FP8 E4M3 codes with one OCP MX
E8M0 scale per 32 consecutive elements of a row (along the head dimension),
and the result is the exact attention (oracle/attention.py) of the values the
codes and scales denote.  The two formats, as their specifications define
them:

  E4M3 code (s, e, m) = bits (7, 6..3, 2..0):
      e > 0:  (-1)^s * 2^(e - 7) * (1 + m / 8)
      e = 0:  (-1)^s * 2^(-6) * (m / 8)
      e = 15 and m = 7: NaN (no infinities; the largest finite value is 448)
  E8M0 scale code c: 2^(c - 127); c = 255 is NaN.

Dequantisation multiplies each element's E4M3 value by its block's scale; all
of it is exact in float64.
"""
from __future__ import annotations

import numpy as np

from .attention import attention_ref

__all__ = ["e4m3_value", "e8m0_value", "mx_dequantize", "attention_fp8_ref", "MX_BLOCK"]

MX_BLOCK = 32


def e4m3_value(codes) -> np.ndarray:
    """float64 value of each E4M3 code (NaN for the two NaN codes)."""
    c = np.asarray(codes).astype(np.int64)
    sign = np.where((c >> 7) & 1, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = c & 0x7
    mag = np.where(e > 0, np.ldexp(1.0 + m / 8.0, e - 7), np.ldexp(m / 8.0, -6))
    mag = np.where((e == 0xF) & (m == 0x7), np.nan, mag)
    return sign * mag


def e8m0_value(codes) -> np.ndarray:
    """float64 value 2^(c - 127) of each E8M0 scale code (NaN for 255)."""
    c = np.asarray(codes).astype(np.int64)
    return np.where(c == 255, np.nan, np.ldexp(1.0, c - 127))


def mx_dequantize(codes, scales) -> np.ndarray:
    """[rows, D] E4M3 codes with [rows, D/32] E8M0 scales -> float64 values."""
    codes = np.asarray(codes)
    rows, d = codes.shape
    scales = np.asarray(scales)
    if d % MX_BLOCK or scales.shape != (rows, d // MX_BLOCK):
        raise ValueError("scales must be [rows, D/32]")
    block_scale = np.repeat(e8m0_value(scales), MX_BLOCK, axis=1)
    return e4m3_value(codes) * block_scale


def attention_fp8_ref(q8, q_scale, k8, k_scale, v8, v_scale, causal: bool = False, scale=None, rows=None):
    """(o, lse) of one head from FP8 codes and MX scales: attention_ref of the
    dequantised Q, K, V (scale defaults to 1/sqrt(D))."""
    q = mx_dequantize(q8, q_scale)
    k = mx_dequantize(k8, k_scale)
    v = mx_dequantize(v8, v_scale)
    return attention_ref(q, k, v, causal, scale, rows=rows)
