"""bf16 rounding for the oracle (float64 in, float64 or bits out).

Rounding is round-to-nearest, ties to even, taken directly from float64 (never
through float32, which would round twice).  bf16 has float32's exponent range
and 8 significant bits: normal numbers from 2^-126, subnormals in steps of
2^-133, the largest finite value (2 - 2^-7) * 2^127, and values at or past the
midpoint to 2^128 round to infinity.  Signs of zeros are kept, so a negative
value that underflows gives -0: TensorFold PR #1183, squashed commit bodies
(the bf16 u16-bit tests), fix that bf16(-2^-135) is -0, bits 0x8000.

The ordered key puts every bf16 pattern on one integer line, -0 just below +0,
as the same page's range checks order their ends.
"""
from __future__ import annotations

import numpy as np

_MAX_FINITE = (2.0 - 2.0 ** -7) * 2.0 ** 127


def round_f64(x) -> np.ndarray:
    """Value of bf16_RNE(x) as float64 (inf for overflow, nan for nan)."""
    x = np.asarray(x, dtype=np.float64)
    out = np.array(x, dtype=np.float64, copy=True)
    fin = np.isfinite(x) & (x != 0)
    if np.any(fin):
        xf = x[fin]
        _, e = np.frexp(xf)              # |x| = m * 2^e, m in [0.5, 1)
        expo = np.maximum(e - 1, -126)   # floor(log2|x|), clamped to normals
        quantum = np.ldexp(1.0, expo - 7)
        r = np.round(xf / quantum) * quantum   # np.round: ties to even
        r = np.where(np.abs(r) >= 2.0 ** 128, np.copysign(np.inf, xf), r)
        out[fin] = r
    return out


def bits_from_f64(x) -> np.ndarray:
    """bf16 bits (uint16) of bf16_RNE(x)."""
    r = round_f64(x)
    b = (r.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    b[np.isnan(r)] = 0x7FC0
    return b


def f64_from_bits(b) -> np.ndarray:
    """Exact float64 value of bf16 bit patterns."""
    b = np.asarray(b, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def is_nan_bits(b) -> np.ndarray:
    b = np.asarray(b, dtype=np.uint16)
    return ((b & 0x7F80) == 0x7F80) & ((b & 0x007F) != 0)


def ordered(b) -> np.ndarray:
    """Monotone integer key of bf16 bits: -0 sorts one step below +0."""
    b = np.asarray(b, dtype=np.uint16).astype(np.int32)
    mag = b & 0x7FFF
    return np.where(b & 0x8000, 0x7FFF - mag, 0x8000 + mag)


def max_finite() -> float:
    return _MAX_FINITE
