"""Independent reference for pinning the oracle: the cast composed from library
routines, vectorised, sharing nothing with ``oracle/``.

Each step of the method is mapped onto a routine whose behaviour is fixed by its
own documentation rather than by this project:
  * |x| max over a group          -> numpy ``abs`` + ``max`` (exact);
  * scale = a / D, v = x / s      -> numpy float32 division (IEEE, nearest-even);
  * 2^ceil(log2 s)                -> numpy ``frexp`` / ``ldexp`` (exact);
  * UE8M0 byte of a power of two  -> torch ``float8_e8m0fnu`` cast;
  * saturating RNE to e4m3        -> numpy ``clip`` then torch ``float8_e4m3fn``
                                     cast (nearest-even, keeps the sign of zero;
                                     it does not saturate by itself, hence clip);
  * RNE to e2m1                   -> numpy ``round`` (half to even) on the
                                     binade's quantum 0.5 / 1 / 2;
  * silu32(g)                     -> ``decimal`` exp at 60 digits, then exact
                                     rounding to binary32 (tests/exact.py).
"""
from __future__ import annotations

import decimal
import functools
from fractions import Fraction

import numpy as np
import torch

from exact import round_to_f32

D_OF = {"e4m3": np.float32(448.0), "e2m1": np.float32(6.0)}
FLOOR = np.float32(1e-4)


def widen(bits: np.ndarray) -> np.ndarray:
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def pow2_ceil(s: np.ndarray) -> np.ndarray:
    m, e = np.frexp(s.astype(np.float32))         # s = m * 2^e, m in [0.5, 1)
    c = np.where(m == np.float32(0.5), e - 1, e)  # ceil(log2 s)
    return np.ldexp(np.float32(1.0), c).astype(np.float32)


def ue8m0_bytes(s_pow2: np.ndarray) -> np.ndarray:
    t = torch.from_numpy(np.ascontiguousarray(s_pow2, dtype=np.float32))
    return t.to(torch.float8_e8m0fnu).view(torch.uint8).numpy()


def e4m3_codes(v: np.ndarray) -> np.ndarray:
    c = np.clip(v.astype(np.float32), np.float32(-448.0), np.float32(448.0))
    return torch.from_numpy(np.ascontiguousarray(c)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def e2m1_codes(v: np.ndarray) -> np.ndarray:
    v = v.astype(np.float32)
    a = np.minimum(np.abs(v), np.float32(6.0))
    q = np.where(a < 2, np.float32(0.5), np.where(a < 4, np.float32(1.0), np.float32(2.0)))
    val = (np.round(a / q) * q).astype(np.float32)
    # value -> code from the format's fields: below 1 the subnormal code is
    # 2*val; from 1 up, code = (exponent+1) << 1 | mantissa bit.
    with np.errstate(divide="ignore"):
        e = np.floor(np.log2(np.where(val >= 1, val, 1))).astype(np.int32)
    mbit = (val / np.ldexp(np.float32(1), e) - 1 == 0.5).astype(np.uint8)
    code = np.where(val < 1, (2 * val).astype(np.uint8), (((e + 1) << 1) | mbit).astype(np.uint8))
    return (code | np.where(np.signbit(v), 8, 0)).astype(np.uint8)


@functools.lru_cache(maxsize=1)
def silu32_table() -> np.ndarray:
    """fp32 nearest to g / (1 + e^-g) for every bf16 bit pattern g (NaN for
    non-finite g), by 60-digit decimal arithmetic and exact rounding."""
    ctx = decimal.Context(prec=60, Emax=10**6, Emin=-10**6)
    out = np.full(65536, np.nan, dtype=np.float32)
    for b in range(65536):
        if (b & 0x7F80) == 0x7F80:
            continue                       # Inf / NaN
        g = float(widen(np.array([b], dtype=np.uint16))[0])
        if g >= 1000.0:
            # g/(1+e^-g) = g*(1 - t), t < e^-1000: rounds to g itself.
            out[b] = g
            continue
        if g <= -1000.0:
            # |g| e^g/(1+e^g) < 4e38 * e^-1000 << 2^-150: rounds to -0.
            out[b] = -0.0
            continue
        dg = decimal.Decimal(g)
        val = ctx.divide(dg, ctx.add(decimal.Decimal(1), ctx.exp(-dg)))
        out[b] = round_to_f32(Fraction(val), negative_zero=(g < 0 or (g == 0 and b == 0x8000)))
    return out


def swiglu_h(gate_up_bits: np.ndarray) -> np.ndarray:
    rows, c2 = gate_up_bits.shape
    cols = c2 // 2
    sg = silu32_table()[gate_up_bits[:, :cols].astype(np.int64)]
    u = widen(gate_up_bits[:, cols:])
    return (sg * u).astype(np.float32)


def cast_values(x: np.ndarray, group: int, out_dtype: str, round_pow2: bool, scale_fmt: str):
    """Cast fp32 values x [rows, cols] -> (codes, scales) in the oracle's layout."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    rows, cols = x.shape
    ng = cols // group
    xg = x.reshape(rows, ng, group)
    amax = np.abs(xg).max(axis=2) if rows else np.zeros((0, ng), np.float32)
    a = np.maximum(amax, FLOOR)
    s = (a / D_OF[out_dtype]).astype(np.float32)
    if round_pow2:
        s = pow2_ceil(s)
    v = (xg / s[:, :, None]).astype(np.float32).reshape(rows, cols)
    if out_dtype == "e4m3":
        q = e4m3_codes(v)
    else:
        n = e2m1_codes(v)
        q = (n[:, 0::2] | (n[:, 1::2] << 4)).astype(np.uint8)
    if scale_fmt == "f32":
        scales = s
    else:
        scales = np.ascontiguousarray(ue8m0_bytes(s)).view(np.int32).reshape(rows, ng // 4)
    return q, scales


def per_token_cast(x_bits, group=128, out_dtype="e4m3", round_pow2=False, scale_fmt="f32"):
    return cast_values(widen(x_bits), group, out_dtype, round_pow2, scale_fmt)


def swiglu_per_token_cast(gate_up_bits, group=128, out_dtype="e4m3", round_pow2=False,
                          scale_fmt="f32"):
    return cast_values(swiglu_h(gate_up_bits), group, out_dtype, round_pow2, scale_fmt)


def decode_e4m3(codes: np.ndarray) -> np.ndarray:
    t = torch.from_numpy(np.ascontiguousarray(codes, dtype=np.uint8)).view(torch.float8_e4m3fn)
    return t.to(torch.float32).numpy()


def decode_e2m1_nibbles(n: np.ndarray) -> np.ndarray:
    mag = np.array([0, 0.5, 1, 1.5, 2, 3, 4, 6], dtype=np.float32)[n & 7]
    return np.where(n & 8, -mag, mag).astype(np.float32)


def f32_to_bf16_bits(v: np.ndarray) -> np.ndarray:
    """torch's fp32 -> bf16 cast (nearest, ties to even) as uint16 bits."""
    t = torch.from_numpy(np.ascontiguousarray(v, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def per_token_dequant(q, scales, cols, group, in_dtype, scale_fmt, out="bf16"):
    """Codes + scales -> fl32(value * s) (torch float8 decode / the E2M1 table,
    numpy fp32 multiply), then torch's bf16 cast when out == "bf16"."""
    rows = q.shape[0]
    if in_dtype == "e4m3":
        val = decode_e4m3(q)
    else:
        n = np.empty((rows, cols), dtype=np.uint8)
        n[:, 0::2] = q & 0xF
        n[:, 1::2] = q >> 4
        val = decode_e2m1_nibbles(n)
    if scale_fmt == "f32":
        s = np.asarray(scales, dtype=np.float32)
    else:
        e = np.ascontiguousarray(scales).view(np.uint8).reshape(rows, cols // group).astype(np.int32)
        s = np.ldexp(np.float32(1.0), e - 127).astype(np.float32)
    y = (val * np.repeat(s, group, axis=1)).astype(np.float32)
    return y if out == "f32" else f32_to_bf16_bits(y)


def per_token_cast_back(x_bits, group, out_dtype, round_pow2):
    q, s = per_token_cast(x_bits, group, out_dtype, round_pow2, "f32")
    return per_token_dequant(q, s, x_bits.shape[1], group, out_dtype, "f32", "bf16")


def block_cast_values(x: np.ndarray, block_rows: int, block_cols: int, out_dtype: str, round_pow2: bool,
                      scale_fmt: str):
    """Cast fp32 values x [rows, cols] with one scale per block of block_rows x
    block_cols elements (last block row partial) -> (codes, scales)."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    rows, cols = x.shape
    nbr, nbc = -(-rows // block_rows), cols // block_cols
    amax = np.zeros((nbr, nbc), np.float32)
    for bi in range(nbr):
        sl = np.abs(x[bi * block_rows:(bi + 1) * block_rows]).reshape(-1, nbc, block_cols)
        amax[bi] = sl.max(axis=(0, 2))
    s = (np.maximum(amax, FLOOR) / D_OF[out_dtype]).astype(np.float32)
    if round_pow2:
        s = pow2_ceil(s)
    s_full = np.repeat(np.repeat(s, block_rows, axis=0)[:rows], block_cols, axis=1)
    v = (x / s_full).astype(np.float32)
    if out_dtype == "e4m3":
        q = e4m3_codes(v)
    else:
        n = e2m1_codes(v)
        q = (n[:, 0::2] | (n[:, 1::2] << 4)).astype(np.uint8)
    if scale_fmt == "f32":
        return q, s
    return q, np.ascontiguousarray(ue8m0_bytes(s)).view(np.int32).reshape(nbr, nbc // 4)


def per_block_cast(x_bits, block_rows=128, block_cols=128, out_dtype="e4m3", round_pow2=False, scale_fmt="f32"):
    return block_cast_values(widen(x_bits), block_rows, block_cols, out_dtype, round_pow2, scale_fmt)


def sum_squares_exact_f32(x_bits: np.ndarray) -> np.ndarray:
    """Per row: the exact sum of squares (Python integers on the bf16 values'
    integer significands) rounded to binary32 by tests/exact.py."""
    from exact import round_to_f32
    out = np.empty(x_bits.shape[0], dtype=np.float32)
    for r in range(x_bits.shape[0]):
        total = Fraction(0)
        for v in widen(x_bits[r]).astype(np.float64):
            if v != 0.0:
                total += Fraction(float(v)) ** 2
        try:
            out[r] = round_to_f32(total)
        except OverflowError:
            out[r] = np.inf
    return out


def rmsnorm(x_bits: np.ndarray, w_bits, eps: float, ss: np.ndarray | None = None) -> np.ndarray:
    """RMSNorm forward as numpy float32 operations (IEEE, nearest-even) on the
    exactly rounded sum of squares: fp32 y [rows, cols]."""
    rows, cols = x_bits.shape
    ss = sum_squares_exact_f32(x_bits) if ss is None else ss
    with np.errstate(over="ignore", invalid="ignore", divide="ignore"):
        t = (ss / np.float32(cols)).astype(np.float32)
        t = (t + np.float32(eps)).astype(np.float32)
        r = (np.float32(1.0) / np.sqrt(t)).astype(np.float32)
        y = (widen(x_bits) * r[:, None]).astype(np.float32)
        if w_bits is not None:
            y = (y * widen(np.asarray(w_bits))[None, :]).astype(np.float32)
    return y
