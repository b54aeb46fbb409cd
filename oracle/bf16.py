"""Exact bf16 conversions for the oracle (test infrastructure only).

bf16 is the upper half of an IEEE binary32 word: 1 sign bit, 8 exponent
bits, 7 stored mantissa bits (8 significant bits). Widening is exact;
narrowing from fp64 rounds once, to nearest with ties to even, directly from
the fp64 value (no intermediate fp32 rounding).
"""
import numpy as np


def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns (uint16) -> exact fp64 values."""
    b = np.asarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def f64_to_bf16(x: np.ndarray) -> np.ndarray:
    """fp64 -> bf16 bit patterns, round to nearest, ties to even.

    For a finite normal x = m * 2**e with 0.5 <= |m| < 1, the value
    ldexp(x, 8 - e) lies in [128, 256) and its integer part holds exactly the
    8 significant bits bf16 keeps; rint() on it is the correctly rounded
    (ties-to-even) choice. The rounded value is exactly representable in
    binary32, so the final cast is exact. Subnormal, infinite and NaN values
    are outside the oracle's contract and rejected.
    """
    x = np.asarray(x, dtype=np.float64)
    if not np.all(np.isfinite(x)):
        raise ValueError("non-finite value in bf16 rounding")
    m, e = np.frexp(x)
    r = np.ldexp(np.rint(np.ldexp(m, 8)), e - 8)
    nz = r != 0
    if np.any(np.abs(r[nz]) < np.ldexp(1.0, -126)):
        raise ValueError("bf16 subnormal outside the oracle's contract")
    if np.any(np.abs(r) >= np.ldexp(1.0, 128)):
        raise ValueError("bf16 overflow")
    return (r.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
