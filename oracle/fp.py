"""Rounding helpers of the oracle: bf16 <-> float32/float64, ulps, exact fp32 rounding.

bf16 is the upper half of an IEEE binary32 (8 significant bits).  Rounding to it is
round-to-nearest-even; a NaN stays a NaN (quiet bit set).
"""
from __future__ import annotations

from fractions import Fraction

import numpy as np


def bf16_to_f32(bits) -> np.ndarray:
    """bf16 bit patterns -> float32 values (exact widening)."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def bf16_to_f64(bits) -> np.ndarray:
    return bf16_to_f32(bits).astype(np.float64)


def f32_to_bf16(x) -> np.ndarray:
    """float32 -> bf16 bits, round to nearest even; NaN -> quiet NaN with the same sign."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    nan = np.isnan(np.asarray(x, dtype=np.float32))
    lsb = (u >> np.uint64(16)) & np.uint64(1)
    r = ((u + np.uint64(0x7FFF) + lsb) >> np.uint64(16)) & np.uint64(0xFFFF)
    q = ((u >> np.uint64(16)) | np.uint64(0x40)) & np.uint64(0xFFFF)
    return np.where(nan, q, r).astype(np.uint16)


def f64_to_bf16(x) -> np.ndarray:
    """float64 -> bf16 bits with ONE rounding (no detour through float32, which would
    round twice).  Round to nearest even on 8 significant bits; subnormal spacing 2^-133;
    overflow to +-inf."""
    x = np.asarray(x, dtype=np.float64)
    out = np.empty(x.shape, dtype=np.float64)
    fin = np.isfinite(x)
    xf = np.where(fin, x, 0.0)
    mant, ex = np.frexp(xf)                          # xf = mant * 2**ex, 0.5 <= |mant| < 1
    ex = np.maximum(ex, -125)                        # below 2^-126 the spacing is fixed
    q = np.rint(np.ldexp(xf, 8 - ex))                # integer count of units of 2^(ex-8)
    val = np.ldexp(q, ex - 8)
    val = np.where(np.abs(val) >= 2.0 ** 128 * (1 - 2.0 ** -9), np.copysign(np.inf, xf), val)
    out[...] = np.where(fin, val, x)
    f = out.astype(np.float32)                       # exact: val has <= 8 significant bits
    return f32_to_bf16(f)


def ulp_bf16(mag) -> np.ndarray:
    """Spacing of bf16 numbers at magnitude |mag| (2^(floor(log2|mag|) - 7), 2^-133 below 2^-126)."""
    m = np.abs(np.asarray(mag, dtype=np.float64))
    m = np.where(m < 2.0 ** -126, 2.0 ** -126, m)
    _, ex = np.frexp(m)
    return np.ldexp(1.0, ex - 1 - 7)


def ulp_f32(mag) -> np.ndarray:
    m = np.abs(np.asarray(mag, dtype=np.float64))
    m = np.where(m < 2.0 ** -126, 2.0 ** -126, m)
    _, ex = np.frexp(m)
    return np.ldexp(1.0, ex - 1 - 23)


def f32_from_fraction(q: Fraction) -> np.float32:
    """Exact round-to-nearest-even of a rational to binary32 (normal range only)."""
    if q == 0:
        return np.float32(0.0)
    sign = -1 if q < 0 else 1
    a = abs(q)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    if Fraction(2) ** e > a:
        e -= 1
    while Fraction(2) ** (e + 1) <= a:
        e += 1
    # a in [2^e, 2^(e+1)); 24 significant bits -> unit 2^(e-23)
    scaled = a / (Fraction(2) ** (e - 23))
    n = scaled.numerator // scaled.denominator
    rem = scaled - n
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and n % 2 == 1):
        n += 1
    return np.float32(sign * float(Fraction(n) * Fraction(2) ** (e - 23)))


def f32_bits(x) -> int:
    return int(np.asarray(x, dtype=np.float32).view(np.uint32))
