"""FP8 inputs: seeded draws quantised to OCP FP8 E4M3 codes with MX block scales.

Input generation only, shared by the oracle side and the GPU side; it holds no
attention arithmetic and no decoding (the oracle decodes codes with its own
implementation of the formats).

Formats (OCP 8-bit floating point and OCP Microscaling (MX) specifications):
  E4M3 code s eeee mmm: (-1)^s 2^(e-7) (1 + m/8) for e > 0, (-1)^s 2^-6 (m/8)
  for e = 0; s 1111 111 is NaN, so the largest finite magnitude is 448.
  E8M0 scale code c: 2^(c - 127) (255 is NaN, never produced here).
A block of 32 elements shares one E8M0 scale.  The element value is the E4M3
value times the block's scale.  Q, K and V are all blocked along the head
dimension: 32 consecutive d of one row share a scale, so a [rows, D] tensor
has [rows, D/32] scales.

Quantisation (the MX specification's shared-scale rule): the block's scale is
2^(floor(log2 amax) - 8), 8 being E4M3's largest exponent, and each element is
x / scale rounded to the nearest E4M3 value (ties to the even code), with
magnitudes above 448 clamped to 448.  An all-zero block gets scale 1.
"""
from __future__ import annotations

import numpy as np

from . import T_DO, T_K, T_Q, T_V, Workload, _stream

MX_BLOCK = 32
E4M3_MAX = 448.0
E8M0_ONE = 127


def _nonneg_table() -> np.ndarray:
    """Magnitudes of the non-negative finite codes 0 .. 126, ascending."""
    c = np.arange(127)
    e, m = c >> 3, c & 7
    return np.where(e == 0, m * 2.0 ** -9, (1.0 + m / 8.0) * 2.0 ** (e - 7.0))


_TABLE = _nonneg_table()


def e4m3_encode(y: np.ndarray) -> np.ndarray:
    """Nearest E4M3 code of each value (ties to the even code), magnitudes clamped to 448."""
    y = np.asarray(y, dtype=np.float64)
    a = np.minimum(np.abs(y), E4M3_MAX)
    hi = np.clip(np.searchsorted(_TABLE, a), 0, 126)
    lo = np.clip(hi - 1, 0, 126)
    dlo, dhi = a - _TABLE[lo], _TABLE[hi] - a
    code = np.where((dhi < dlo) | ((dhi == dlo) & (hi % 2 == 0)), hi, lo)
    return (code | np.where(y < 0, 0x80, 0)).astype(np.uint8)


def _block_scale_codes(amax: np.ndarray) -> np.ndarray:
    with np.errstate(divide="ignore"):
        e = np.floor(np.log2(np.where(amax > 0, amax, 1.0))) - 8
    code = np.clip(e + E8M0_ONE, 0, 254)
    return np.where(amax > 0, code, E8M0_ONE).astype(np.uint8)


def quantize_rows(x: np.ndarray):
    """[rows, D] values -> (codes [rows, D], scales [rows, D/32]): blocks along D."""
    rows, d = x.shape
    blocks = np.asarray(x, np.float64).reshape(rows, d // MX_BLOCK, MX_BLOCK)
    sc = _block_scale_codes(np.abs(blocks).max(axis=2))
    codes = e4m3_encode(blocks / np.exp2(sc.astype(np.float64) - E8M0_ONE)[:, :, None])
    return codes.reshape(rows, d), sc


def head_mx(w: Workload, b: int, h: int, t: int):
    """(codes [rows, D], scales [rows, D/32]) of tensor t (T_Q, T_K, T_V) for one
    (b, h): the standard normal draw of the bf16 workloads, quantised along D."""
    x = _stream(w.seed_id, w.variant, b, h, t).standard_normal((w.rows(t), w.D), dtype=np.float32)
    if w.variant == 1 and t in (T_Q, T_K):
        x = x * np.float32(4.0)
    return quantize_rows(x)


def full_mx(w: Workload, t: int):
    """Whole-tensor (codes [B, H, rows, D], scales) of tensor t."""
    pairs = [head_mx(w, b, hh, t) for b in range(w.B) for hh in range(w.H)]
    codes = np.stack([p[0] for p in pairs]).reshape(w.B, w.H, *pairs[0][0].shape)
    scales = np.stack([p[1] for p in pairs]).reshape(w.B, w.H, *pairs[0][1].shape)
    return codes, scales


__all__ = ["MX_BLOCK", "E4M3_MAX", "E8M0_ONE", "e4m3_encode", "quantize_rows", "head_mx",
           "full_mx", "T_Q", "T_K", "T_V", "T_DO"]
