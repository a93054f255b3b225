"""Pins for the FP8 oracle (oracle/fp8.py) that do not reuse its formulas:
torch's own float8_e4m3fn conversion for every code, values the OCP FP8
specification lists, powers of two for E8M0, a per-element loop for the block
layout, exact scale invariances of the attention, and agreement with the input
generator's independent encoder.  Planted mistakes each fail a pin.
"""
import numpy as np
import pytest
import torch

import fa_inputs as fi
import fa_inputs.fp8 as f8
from oracle import attention_ref
from oracle import fp8 as ofp8


def _torch_e4m3(codes):
    t = torch.from_numpy(np.asarray(codes, np.uint8).copy()).view(torch.float8_e4m3fn)
    return t.to(torch.float64).numpy()


def pin_every_code_against_torch(dec, *_):
    codes = np.arange(256, dtype=np.uint8)
    ours, ref = dec(codes), _torch_e4m3(codes)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(ours), nan), "NaN codes"
    assert np.array_equal(ours[~nan], ref[~nan]), "E4M3 values differ from torch float8_e4m3fn"


def pin_spec_values(dec, *_):
    # values listed for E4M3 by the OCP 8-bit floating point specification
    table = {0x00: 0.0, 0x01: 2.0 ** -9, 0x07: 0.875 * 2.0 ** -6, 0x08: 2.0 ** -6, 0x38: 1.0, 0x3C: 1.5,
             0x40: 2.0, 0x7E: 448.0, 0x77: 240.0, 0xB8: -1.0, 0xFE: -448.0, 0x81: -(2.0 ** -9)}
    for code, val in table.items():
        assert dec(np.array([code]))[0] == val, hex(code)
    assert np.isnan(dec(np.array([0x7F]))[0]) and np.isnan(dec(np.array([0xFF]))[0])
    assert dec(np.array([0x80]))[0] == 0.0 and np.signbit(dec(np.array([0x80]))[0])


def pin_e8m0(_, e8, *__):
    assert e8(np.array([127]))[0] == 1.0 and e8(np.array([128]))[0] == 2.0 and e8(np.array([126]))[0] == 0.5
    assert e8(np.array([0]))[0] == 2.0 ** -127 and e8(np.array([254]))[0] == 2.0 ** 127
    assert np.isnan(e8(np.array([255]))[0])


def pin_block_layout(dec, e8, deq):
    g = np.random.default_rng(3)
    codes = g.integers(0, 0x7F, (5, 96)).astype(np.uint8)
    scales = g.integers(100, 150, (5, 3)).astype(np.uint8)
    out = deq(codes, scales)
    for r in range(5):
        for c in range(96):
            want = _torch_e4m3([codes[r, c]])[0] * 2.0 ** (int(scales[r, c // 32]) - 127)
            assert out[r, c] == want, (r, c)


def pin_scale_invariances(dec, e8, deq):
    """Raising every Q block scale by one doubles the scores (so halving the
    softmax scale undoes it exactly); raising every V scale doubles O and
    leaves LSE alone."""
    w = fi.Workload("fp8_pin", 77, 1, 1, 70, 64, "fp8", True)
    (q8, qs), (k8, ks), (v8, vs) = (f8.head_mx(w, 0, 0, t) for t in (fi.T_Q, fi.T_K, fi.T_V))
    run = lambda qs_, vs_, sc: attention_ref(deq(q8, qs_), deq(k8, ks), deq(v8, vs_), True, sc)
    o0, l0 = run(qs, vs, 0.125)
    o1, l1 = run(qs + 1, vs, 0.0625)
    assert np.array_equal(o0, o1) and np.array_equal(l0, l1), "Q scale"
    o2, l2 = run(qs, vs + 1, 0.125)
    assert np.array_equal(o2, 2 * o0) and np.array_equal(l2, l0), "V scale"


def pin_generator_round_trip(dec, e8, deq):
    """The generator's encoder (a nearest-value search, written separately)
    maps every finite decoded value back to its code."""
    codes = np.array([c for c in range(256) if c & 0x7F != 0x7F and c != 0x80], dtype=np.uint8)
    assert np.array_equal(f8.e4m3_encode(dec(codes)), codes)


PINS = [pin_every_code_against_torch, pin_spec_values, pin_e8m0, pin_block_layout, pin_scale_invariances,
        pin_generator_round_trip]


@pytest.mark.parametrize("pin", PINS, ids=lambda p: p.__name__)
def test_fp8_oracle_passes(pin):
    pin(ofp8.e4m3_value, ofp8.e8m0_value, ofp8.mx_dequantize)


def test_attention_fp8_ref_is_attention_of_dequantised_inputs():
    w = fi.Workload("fp8_pin2", 78, 1, 1, 33, 64, "fp8", False)
    (q8, qs), (k8, ks), (v8, vs) = (f8.head_mx(w, 0, 0, t) for t in (fi.T_Q, fi.T_K, fi.T_V))
    o, lse = ofp8.attention_fp8_ref(q8, qs, k8, ks, v8, vs, False, 0.2)
    # dequantisation done here with torch's decoder and a per-block loop
    def deq(c, s):
        x = _torch_e4m3(c.reshape(-1)).reshape(c.shape)
        for j in range(s.shape[1]):
            x[:, 32 * j:32 * j + 32] *= 2.0 ** (s[:, j:j + 1].astype(np.int64) - 127)
        return x
    o2, l2 = attention_ref(deq(q8, qs), deq(k8, ks), deq(v8, vs), False, 0.2)
    assert np.array_equal(o, o2) and np.array_equal(lse, l2)


def _mutant(kind):
    def dec(codes):
        c = np.asarray(codes).astype(np.int64)
        sign = np.where((c >> 7) & 1, -1.0, 1.0)
        if kind == "sign_ignored":
            sign = 1.0
        e, m = (c >> 3) & 0xF, c & 7
        bias = 8 if kind == "bias_8" else 7
        sub = np.ldexp(m / 8.0, -6) if kind != "subnormal_as_normal" else np.ldexp(1 + m / 8.0, -7)
        mag = np.where(e > 0, np.ldexp(1.0 + m / 8.0, e - bias), sub)
        if kind == "mantissa_4bits":
            mag = np.where(e > 0, np.ldexp(1.0 + m / 16.0, e - 7), sub)
        mag = np.where((e == 15) & (m == 7), np.nan, mag)
        return sign * mag

    def e8(c):
        c = np.asarray(c).astype(np.int64)
        return np.where(c == 255, np.nan, np.ldexp(1.0, c - (128 if kind == "e8m0_bias_128" else 127)))

    def deq(codes, scales):
        blk = 16 if kind == "blocks_of_16" else 32
        s = np.repeat(e8(scales), 32, axis=1)
        if kind == "blocks_of_16":
            s = np.repeat(e8(scales), 16, axis=1)
            s = np.concatenate([s, s], axis=1)[:, :codes.shape[1]]
        if kind == "scale_per_row_first_block":
            s = np.repeat(e8(scales[:, :1]), codes.shape[1], axis=1)
        return dec(codes) * s
    return dec, e8, deq


@pytest.mark.parametrize("kind", ["sign_ignored", "bias_8", "subnormal_as_normal", "mantissa_4bits",
                                  "e8m0_bias_128", "blocks_of_16", "scale_per_row_first_block"])
def test_fp8_mutant_is_caught(kind):
    failed = 0
    for pin in PINS:
        try:
            pin(*_mutant(kind))
        except AssertionError:
            failed += 1
    assert failed, f"mutant {kind} passed every pin"
