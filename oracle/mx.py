"""MXFP8 (E4M3 elements, E8M0 block scale, 32 elements per block) for the oracle.

The MoK paper (§3.4 "MXFP8 Support") runs the routed experts in MXFP8 and cites
the OCP Microscaling format without spelling it out.  This module takes the
reading written down in the design doc:

* a block is 32 consecutive elements along the contraction (K) axis;
* the shared scale is a power of two 2^X stored as the byte X + 127 (E8M0),
  with X = floor(log2(amax)) - 8, where 8 is the exponent of the largest
  E4M3 normal (448 = 1.75 * 2^8), clamped to [-127, 127];
* an all-zero block gets the byte 0x00 (X = -127) and zero elements;
* each element v / 2^X is rounded to the nearest E4M3 value, ties to even,
  saturating at +-448 (E4M3 "FN": no infinities, 0x7F/0xFF are NaN).

E4M3 values: sign, 4 exponent bits (bias 7), 3 mantissa bits.  Normals are
(1 + m/8) * 2^(e-7) for e in 1..15 (with e=15, m=7 being NaN), subnormals are
m/8 * 2^-6 = m * 2^-9.
"""

from __future__ import annotations

import numpy as np

BLOCK = 32
E4M3_MAX = 448.0
E4M3_EMAX = 8


def _e4m3_table() -> np.ndarray:
    """fp64 value of each of the 256 E4M3FN codes (NaN codes -> nan)."""
    vals = np.empty(256, dtype=np.float64)
    for code in range(256):
        s = -1.0 if code & 0x80 else 1.0
        e = (code >> 3) & 0xF
        m = code & 0x7
        if e == 0xF and m == 0x7:
            vals[code] = np.nan
        elif e == 0:
            vals[code] = s * m * 2.0 ** -9
        else:
            vals[code] = s * (1.0 + m / 8.0) * 2.0 ** (e - 7)
    return vals


E4M3_VALUES = _e4m3_table()


def e4m3_decode(codes: np.ndarray) -> np.ndarray:
    return E4M3_VALUES[np.asarray(codes, dtype=np.uint8)]


def e4m3_encode(v: np.ndarray) -> np.ndarray:
    """Round fp64 values to E4M3FN codes: nearest, ties to even, saturate at 448."""
    v = np.asarray(v, dtype=np.float64)
    if not np.all(np.isfinite(v)):
        raise ValueError("non-finite input to the E4M3 encoder")
    sign = np.signbit(v)
    a = np.minimum(np.abs(v), E4M3_MAX)
    _, e = np.frexp(a)  # a in [2^(e-1), 2^e)
    q = np.maximum(e - 4, -9)  # spacing 2^(e-4) in a binade (4 significant bits), 2^-9 below 2^-6
    r = np.rint(a / np.ldexp(1.0, q)) * np.ldexp(1.0, q)
    r = np.minimum(r, E4M3_MAX)  # a tie just under 448 can only round to 448 itself
    # the code of r from the format's definition: below 2^-6 a subnormal
    # m * 2^-9; otherwise r = (1 + m/8) * 2^(E-7) with biased exponent E
    f, ex = np.frexp(r)  # r = f * 2^ex, f in [0.5, 1)
    normal = r >= 2.0 ** -6
    code = np.where(normal, ((ex + 6) << 3) | np.rint((2.0 * f - 1.0) * 8.0).astype(np.int64),
                    np.rint(r * 2.0 ** 9).astype(np.int64)).astype(np.uint8)
    assert np.all(E4M3_VALUES[code] == r)  # the table decodes it back exactly
    # the sign is kept also when the value rounds to zero (-0 is code 0x80)
    return np.where(sign, code | np.uint8(0x80), code).astype(np.uint8)


def scale_exponent(amax: np.ndarray) -> np.ndarray:
    """Shared exponent X of a block with largest magnitude amax."""
    amax = np.asarray(amax, dtype=np.float64)
    out = np.full(amax.shape, -127, dtype=np.int64)
    nz = amax > 0
    _, e = np.frexp(amax[nz])  # amax in [2^(e-1), 2^e): floor(log2 amax) = e - 1
    out[nz] = np.clip(e - 1 - E4M3_EMAX, -127, 127)
    return out


def quantize(v: np.ndarray):
    """MX-quantise along the last axis (length a multiple of 32).

    Returns (codes uint8 same shape, scale bytes uint8 [..., n/32]).
    """
    v = np.asarray(v, dtype=np.float64)
    n = v.shape[-1]
    if n % BLOCK:
        raise ValueError("last axis must be a multiple of 32")
    blocks = v.reshape(v.shape[:-1] + (n // BLOCK, BLOCK))
    X = scale_exponent(np.abs(blocks).max(axis=-1))
    scaled = blocks / np.ldexp(1.0, X)[..., None]  # exact: power-of-two scaling
    codes = e4m3_encode(scaled).reshape(v.shape)
    return codes, (X + 127).astype(np.uint8)


def dequantize(codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """fp64 values of MX data (exact)."""
    codes = np.asarray(codes, dtype=np.uint8)
    n = codes.shape[-1]
    vals = e4m3_decode(codes).reshape(codes.shape[:-1] + (n // BLOCK, BLOCK))
    X = np.asarray(scales, dtype=np.int64) - 127
    return (vals * np.ldexp(1.0, X)[..., None]).reshape(codes.shape)


def round_f64(v: np.ndarray) -> np.ndarray:
    """The value v takes after MX quantisation along the last axis."""
    return dequantize(*quantize(v))
