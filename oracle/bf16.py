"""bfloat16 <-> float64 for the oracle (test infrastructure only).

bf16: 1 sign bit, 8 exponent bits (bias 127), 7 stored significand bits; the
top 16 bits of an IEEE binary32. Finite values are m * 2**(e - 7) with an
8-bit significand m in [128, 255] for normals (e in [-126, 127]) and
m * 2**-133 with m in [1, 127] for subnormals.
"""
from __future__ import annotations

import numpy as np


def decode(bits) -> np.ndarray:
    """bf16 bit patterns (uint16) -> exact float64 values."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    with np.errstate(invalid="ignore"):
        return b.view(np.float32).astype(np.float64)


def round_rne(v) -> np.ndarray:
    """float64 -> bf16 bits with ONE rounding, to nearest, ties to even.

    The quantum of |v| is 2**(e-7) for its binary exponent e >= -126 and
    2**-133 below (bf16 subnormals); |v| / quantum is rounded with
    ``numpy.rint`` (ties to even) and scaled back, which is exact in float64.
    Results at or above 2**128 become infinity; NaN becomes the quiet NaN 0x7FC0.
    """
    v = np.asarray(v, dtype=np.float64)
    a = np.abs(v)
    _, e2 = np.frexp(a)                       # a = f * 2**e2, f in [0.5, 1)
    e = e2.astype(np.int64) - 1               # a in [2**e, 2**(e+1))
    e = np.maximum(e, -126)                   # subnormal range shares the 2**-133 quantum
    q = np.ldexp(1.0, (e - 7).astype(np.int32))
    with np.errstate(over="ignore", invalid="ignore"):
        r = np.rint(a / q) * q
        r = np.where(np.isfinite(a), r, a)
        r = np.copysign(r, v)
        f32 = r.astype(np.float32)            # exact: r is a bf16 value (or overflows to inf)
    bits = (f32.view(np.uint32) >> 16).astype(np.uint16)
    return np.where(np.isnan(v), np.uint16(0x7FC0), bits)


def to_ordered(bits) -> np.ndarray:
    """Map bf16 bits to integers ordered like the values, +0 and -0 both to 0."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.int64)
    mag = b & 0x7FFF
    return np.where(b & 0x8000, -mag, mag)


def ulp_distance(a_bits, b_bits) -> np.ndarray:
    """Number of bf16 lattice steps between two bf16 values (finite inputs)."""
    return np.abs(to_ordered(a_bits) - to_ordered(b_bits))
