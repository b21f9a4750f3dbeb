"""Exact-arithmetic helpers for the pin tests (no code shared with the oracle).

Everything here works on Python integers and fractions.Fraction, so results are
exact; rounding to binary32 is done by the textbook rule (nearest, ties to even
significand) on the exact value.
"""
from __future__ import annotations

import math
import struct
from fractions import Fraction

F32_EMIN = -126          # smallest normal exponent
F32_MANT = 23            # stored significand bits


def f32_bits(x: float) -> int:
    return struct.unpack("<I", struct.pack("<f", x))[0]


def f32_from_bits(b: int) -> float:
    return struct.unpack("<f", struct.pack("<I", b & 0xFFFFFFFF))[0]


def floor_log2(q: Fraction) -> int:
    """Largest e with 2^e <= q, for q > 0, exactly."""
    n, d = q.numerator, q.denominator
    e = n.bit_length() - d.bit_length()
    # 2^e <= n/d  <=>  n * 2^-e >= d
    if e >= 0:
        if n < (d << e):
            e -= 1
    else:
        if (n << -e) < d:
            e -= 1
    return e


def ceil_log2(q: Fraction) -> int:
    """Smallest e with 2^e >= q, for q > 0, exactly."""
    e = floor_log2(q)
    return e if Fraction(2) ** e == q else e + 1


def round_to_f32(q: Fraction, negative_zero: bool = False) -> float:
    """Nearest binary32 value to the exact rational q (ties to even
    significand), as a Python float.  Subnormals are handled; results beyond
    the largest finite value are not expected here and raise."""
    if q == 0:
        return -0.0 if negative_zero else 0.0
    neg = q < 0
    a = -q if neg else q
    e = max(floor_log2(a), F32_EMIN)
    quantum = Fraction(2) ** (e - F32_MANT)
    n = a / quantum
    k = math.floor(n)
    rem = n - k
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and k % 2 == 1):
        k += 1
    val = k * quantum
    if val >= Fraction(2) ** 128:
        raise OverflowError("value beyond binary32 range")
    out = float(val)                # exact: val is a binary32 value
    return -out if neg else out


def bf16_value(bits: int) -> Fraction:
    """Exact value of a finite bf16 bit pattern."""
    return Fraction(f32_from_bits(bits << 16))
