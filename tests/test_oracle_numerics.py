"""Pins of the oracle's number formats (bf16 storage rounding and MXFP8).

Each check compares against something other than the oracle itself: the IEEE
bit layout, torch's own format conversions (library routines), or values
fixed by the definition of the format.
"""

import numpy as np
import pytest
import torch

from oracle import bf16, mx


# --------------------------------------------------------------------------- bf16

def test_bf16_decode_known_patterns():
    pats = np.array([0x3F80, 0xC000, 0x0000, 0x8000, 0x7F7F, 0x0001, 0x3EAB], dtype=np.uint16)
    want = [1.0, -2.0, 0.0, -0.0, (2 - 2 ** -7) * 2.0 ** 127, 2.0 ** -133,
            (1 + 0x2B / 128) * 2.0 ** -2]
    got = bf16.to_f64(pats)
    assert list(got) == want
    assert np.signbit(got[3])


def test_bf16_round_matches_torch_on_fp32_values():
    g = torch.Generator().manual_seed(5)
    v = torch.randn(200_000, generator=g, dtype=torch.float32) * 3.0
    v = torch.cat([v, v * 1e-30, v * 1e30])
    ref = v.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got = bf16.from_f64(v.numpy().astype(np.float64))
    assert np.array_equal(got, ref)


def test_bf16_round_is_direct_not_double():
    # 1 + 2^-8 is the midpoint of 1 and 1 + 2^-7: ties to even gives 1.
    # 1 + 2^-8 + 2^-30 is above the midpoint: direct rounding goes up, whereas
    # rounding to fp32 first would land on the midpoint and then go down.
    x = np.array([1 + 2 ** -8, 1 + 2 ** -8 + 2 ** -30, 1 + 3 * 2 ** -8, -(1 + 2 ** -8 + 2 ** -40)])
    want = np.array([1.0, 1 + 2 ** -7, 1 + 4 * 2 ** -8, -(1 + 2 ** -7)])
    assert np.array_equal(bf16.round_f64(x), want)


def test_bf16_round_error_bound():
    rng = np.random.default_rng(1)
    x = rng.standard_normal(100_000) * 10.0 ** rng.integers(-20, 20, 100_000)
    r = bf16.round_f64(x)
    assert np.all(np.abs(r - x) <= np.abs(x) * 2.0 ** -8)
    # and r is a bf16 value: its fp32 has 16 zero low bits
    assert np.all((r.astype(np.float32).view(np.uint32) & 0xFFFF) == 0)


# --------------------------------------------------------------------------- E4M3

def test_e4m3_table_matches_torch():
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    ref = codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = mx.e4m3_decode(np.arange(256))
    both_nan = np.isnan(ref) & np.isnan(got)
    assert np.array_equal(np.where(both_nan, 0, got), np.where(both_nan, 0, ref))
    assert np.count_nonzero(np.isnan(got)) == 2  # 0x7F and 0xFF
    assert got[0x7E] == 448.0 and got[0x01] == 2.0 ** -9 and got[0x08] == 2.0 ** -6


def test_e4m3_encode_matches_torch_in_range():
    g = torch.Generator().manual_seed(3)
    v = torch.randn(300_000, generator=g, dtype=torch.float64) * 2.0 ** torch.randint(-12, 9, (300_000,), generator=g)
    # fp32 inputs: torch converts through fp32, so only then is it a single rounding
    v = v.clamp(-448, 448).float()
    ref = v.to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    got = mx.e4m3_encode(v.numpy().astype(np.float64))
    assert np.array_equal(got, ref)


def test_e4m3_encode_saturates_and_keeps_sign():
    v = np.array([448.0, 449.0, 464.0, 500.0, 1e9, -1e9, -0.0, 0.0, -2.0 ** -11, 2.0 ** -10, 3 * 2.0 ** -11])
    want = np.array([0x7E, 0x7E, 0x7E, 0x7E, 0x7E, 0xFE, 0x80, 0x00, 0x80, 0x00, 0x01], dtype=np.uint8)
    assert np.array_equal(mx.e4m3_encode(v), want)


def test_e4m3_grid_round_trip():
    vals = mx.E4M3_VALUES[np.r_[0:0x7F, 0x80:0xFF]]
    assert np.array_equal(mx.e4m3_decode(mx.e4m3_encode(vals)), vals)


# --------------------------------------------------------------------------- MX blocks

def test_mx_scale_rule_closed_form():
    amax = np.array([1.0, 448.0, 447.0, 2.0 ** -20, 0.0, 3.0, 2.0 ** 200, 2.0 ** -200])
    # X = floor(log2 amax) - 8, clamped to [-127, 127]; zero block -> -127
    want = np.array([-8, 0, 0, -28, -127, -7, 127, -127])
    assert np.array_equal(mx.scale_exponent(amax), want)


def test_mx_quantize_block_properties():
    rng = np.random.default_rng(7)
    v = rng.standard_normal((64, 256)) * 2.0 ** rng.integers(-6, 6, (64, 1))
    codes, scales = mx.quantize(v)
    assert codes.shape == v.shape and scales.shape == (64, 8)
    q = mx.dequantize(codes, scales)
    blocks = v.reshape(64, 8, 32)
    X = scales.astype(np.int64) - 127
    amax = np.abs(blocks).max(-1)
    # the largest element of each block lands in [256, 512) before saturation
    assert np.all((amax / 2.0 ** X >= 256) & (amax / 2.0 ** X < 512))
    # element error: half a spacing in its binade (relative 2^-4), or the
    # saturation loss above 448, or half the subnormal spacing 2^-10 (scaled)
    err = np.abs(q - v).reshape(64, 8, 32)
    a = np.abs(blocks) / 2.0 ** X[..., None]
    bound = np.maximum(np.maximum(a * 2.0 ** -4, 2.0 ** -10), a - 448.0) * 2.0 ** X[..., None]
    assert np.all(err <= bound)
    # zero block
    c0, s0 = mx.quantize(np.zeros((1, 32)))
    assert s0[0, 0] == 0 and np.all(c0 == 0)


def test_mx_lossless_on_grid_values():
    rng = np.random.default_rng(9)
    codes = rng.integers(0, 0x7F, (16, 64)).astype(np.uint8)
    codes[:, ::32] = 0x7E  # one 448 per block pins the scale at 2^X
    codes |= (rng.integers(0, 2, (16, 64)) * 0x80).astype(np.uint8)
    X = rng.integers(-20, 20, (16, 2))
    v = mx.dequantize(codes, (X + 127).astype(np.uint8))
    c2, s2 = mx.quantize(v)
    assert np.array_equal(s2, (X + 127).astype(np.uint8))
    assert np.array_equal(mx.dequantize(c2, s2), v)
