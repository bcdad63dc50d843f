"""bf16 bit patterns <-> fp64 for the oracle.

bf16 is the top half of an IEEE-754 binary32: 1 sign bit, 8 exponent bits,
7 stored mantissa bits.  Widening to fp64 is exact.  Narrowing rounds to the
nearest bf16 with ties to even, directly from fp64 (no intermediate fp32
rounding, which would round twice).
"""

from __future__ import annotations

import numpy as np


def to_f64(u16: np.ndarray) -> np.ndarray:
    """Exact fp64 value of bf16 bit patterns (uint16 array)."""
    u = np.asarray(u16, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return u.view(np.float32).astype(np.float64)


def round_f64(x: np.ndarray) -> np.ndarray:
    """Round fp64 values to the nearest bf16 value (ties to even); returns fp64.

    bf16 has 8 significant bits, so for |x| in [2^e, 2^(e+1)) the spacing is
    2^(e-7); below the smallest normal 2^-126 the spacing stays 2^-133.
    Values beyond the largest finite bf16 are not expected here and raise.
    """
    x = np.asarray(x, dtype=np.float64)
    if not np.all(np.isfinite(x)):
        raise ValueError("non-finite value cannot be stored as a finite bf16")
    _, e = np.frexp(x)  # x = m * 2^e with 0.5 <= |m| < 1, so |x| in [2^(e-1), 2^e)
    q = np.maximum(e - 8, -133)  # exponent of the spacing for that binade
    scale = np.ldexp(1.0, q)
    r = np.rint(x / scale) * scale  # x / scale is exact (power-of-two scaling)
    if np.any(np.abs(r) > 3.3895313892515355e38):
        raise ValueError("value out of bf16 range")
    return r


def from_f64(x: np.ndarray) -> np.ndarray:
    """bf16 bit patterns of round_f64(x)."""
    r = round_f64(x).astype(np.float32)  # exact: a bf16 value is an fp32 value
    return (r.view(np.uint32) >> np.uint32(16)).astype(np.uint16)
