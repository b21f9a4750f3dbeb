"""CPU checks of facts the gfx950 kernels rely on (no GPU, no oracle code):
the silu32 table's closed-form regions and its rounding margin."""
from __future__ import annotations

import decimal
from fractions import Fraction

import numpy as np

import libref
from exact import floor_log2

# design constants of the SwiGLU kernel's table (bf16 magnitude bits)
SILU_LO, SILU_HI = 0x3280, 0x4300          # 2^-26 and 128


def _bf16(bits):
    return float(np.array([bits << 16], np.uint32).view(np.float32)[0])


def test_closed_forms_outside_the_table():
    table = libref.silu32_table()                        # 60-digit reference
    for b in range(65536):
        if (b & 0x7F80) == 0x7F80:
            continue
        mag, neg = b & 0x7FFF, b >> 15
        g = np.float32(_bf16(b))
        want = table[b].view(np.uint32)
        if mag < SILU_LO:
            assert (g * np.float32(0.5)).view(np.uint32) == want, hex(b)
        elif mag > SILU_HI:
            expect = np.float32(-0.0) if neg else g
            assert expect.view(np.uint32) == want, hex(b)


def test_table_values_keep_a_margin_from_fp32_midpoints():
    """For 2^-6 <= |g| <= 128 the exact silu(g) never comes within 2^-20 fp32
    ulp of a point halfway between two fp32 values (subnormal results
    included), while an fp64 evaluation errs by under 2^-26 fp32 ulp; so one
    fp64 -> fp32 rounding gives the correctly rounded value."""
    ctx = decimal.Context(prec=50, Emax=10**6, Emin=-10**6)
    worst = 1.0
    for mag in range(SILU_LO, SILU_HI + 1):
        for neg in (0, 1):
            g = _bf16((neg << 15) | mag)
            if abs(g) < 2.0 ** -6:
                continue
            dg = decimal.Decimal(g)
            v = Fraction(ctx.divide(dg, ctx.add(1, ctx.exp(-dg))))
            av = abs(v)
            if av < Fraction(2) ** -151:
                continue                  # below a quarter of the smallest subnormal: rounds to -0 by far
            e = max(floor_log2(av), -126)
            ulp = Fraction(2) ** (e - 23)
            k = av / ulp                          # position in ulps
            frac = k - (k.numerator // k.denominator)
            worst = min(worst, float(abs(frac - Fraction(1, 2))))
    assert worst > 2.0 ** -20, worst



def _pow2_by_division(a: np.ndarray, d: float) -> np.ndarray:
    """Biased exponent of 2^ceil(log2(fl32(a / d))) read from the quotient's fields."""
    s = (a / np.float32(d)).astype(np.float32).view(np.uint32)
    return (s >> 23) + ((s & 0x7FFFFF) != 0)


def _pow2_by_fields(a: np.ndarray, qd: str) -> np.ndarray:
    """The kernels' division-free form: from a's own exponent and mantissa."""
    b = a.view(np.uint32)
    e, m = b >> 23, b & 0x7FFFFF
    if qd == "e4m3":                       # D = 7 * 2^6: round up past mantissa 1.75
        return e - 8 + (m > 0x600000)
    return e - 2 + (m > 0x400000)          # D = 3 * 2: round up past mantissa 1.5


def _pow2_by_carry(a: np.ndarray, qd: str) -> np.ndarray:
    """The one-addition form the fused RMSNorm cast uses: 2^23 - T - 1 added
    to a's bits carries into the exponent field exactly when the significand
    field passes T, and the same addition takes off the 8 (E4M3) or 2 (E2M1);
    the mask keeps the exponent field."""
    b = a.view(np.uint32).astype(np.uint64)
    add = ((0x1FFFFF - (8 << 23)) if qd == "e4m3" else (0x3FFFFF - (2 << 23))) % (1 << 32)   # as a uint32
    s_bits = ((b + np.uint64(add)) & 0xFFFFFFFF) & 0x7F800000
    return (s_bits >> 23).astype(np.uint32)


def test_pow2_scale_without_division():
    """fl32(a/448) and fl32(a/6) are powers of two only when the exact
    quotients are, so ceil(log2) of the rounded quotient follows from a's
    fields (compared, or by one carrying addition): checked for every fp32
    significand at exponents spanning the floored range [1e-4, FLT_MAX], and
    at the floor itself."""
    mant = np.arange(1 << 23, dtype=np.uint32)
    floor_bits = np.float32(1e-4).view(np.uint32)
    for field in (113, 114, 120, 127, 128, 150, 200, 253, 254):
        bits = (np.uint32(field) << 23) | mant
        if field == 113:
            bits = bits[bits >= floor_bits]
        a = bits.view(np.float32)
        for qd, d in (("e4m3", 448.0), ("e2m1", 6.0)):
            want = _pow2_by_division(a, d)
            got = _pow2_by_fields(a, qd)
            assert np.array_equal(got, want), (field, qd, int(np.argmax(got != want)))
            carry = _pow2_by_carry(a, qd)
            assert np.array_equal(carry, want), (field, qd, int(np.argmax(carry != want)))
