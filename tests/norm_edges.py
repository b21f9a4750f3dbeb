"""Rows on which RMSNorm's output y equals chosen bf16 values exactly, for
testing the fused cast's rounding edges through the RMSNorm path.

A row of C columns (C a multiple of 256) ends with C/256 anchor values
2^(M+4); every other column is a test value t with |t| <= 896.  The exact
sum of squares is C * 2^(2M) plus at most C * 896^2 < 2^34, far below half
an fp32 unit of C * 2^(2M) (2^(2M + log2 C - 24)), so ss rounds to C * 2^(2M);
ss / C = 2^(2M) absorbs eps = 1e-6, sqrt gives 2^M and r = 2^-M, all exact.
Test columns carry the weight 2^M, so y = (t * 2^-M) * 2^M = t exactly (no
step leaves the fp32 normal range); the anchors carry weight 1 (y = 16).

Each scale group of test columns starts with D * 2^k (D = 448 for E4M3, 6
for E2M1), which makes the group's maximum D * 2^k and its scale 2^k for
fp32 and power-of-two scales alike; the other G - 1 columns hold every
finite bf16 magnitude from 2^(k-14) (E4M3) or 2^(k-5) (E2M1) up to D * 2^k,
with both signs, plus +0 and -0.  At scale 2^k these are every E4M3 / E2M1
code's value, every midpoint between two codes (ties to even), the
subnormal codes and the values that round to zero.  Groups whose maximum
falls below 1e-4 exercise the floored scale.

Only bit patterns are built here; nothing of the method's arithmetic.
"""
from __future__ import annotations

import numpy as np

M = 30                      # every row's root mean square is 2^M


def _bf16(v: float) -> int:
    b = int(np.float32(v).view(np.uint32))
    assert b & 0xFFFF == 0, "not a bf16 value"
    return b >> 16


def edge_values(dt: str, k: int) -> tuple[int, np.ndarray]:
    """The group maximum's bf16 bits and the test values (bf16 bits) for scale 2^k."""
    d = 448.0 if dt == "e4m3" else 6.0
    top = _bf16(d * 2.0 ** k)
    low = _bf16(2.0 ** (k - (14 if dt == "e4m3" else 5)))
    mags = np.arange(low, top + 1, dtype=np.uint16)           # positive bf16 order = bit order
    vals = np.concatenate([mags, mags | np.uint16(0x8000), np.array([0x0000, 0x8000], np.uint16)])
    return top, vals


def edge_rows(cols: int, group: int, dt: str, ks=range(-24, 2)) -> tuple[np.ndarray, np.ndarray]:
    """x (bf16 bits [rows, cols]) and weight (bf16 bits [cols]) as described above."""
    assert cols % 256 == 0 and cols % group == 0
    anchors = cols // 256
    reserved = -(-anchors // group) * group                   # trailing groups without test values
    ngroups = (cols - reserved) // group
    per_row = ngroups * (group - 1)
    rows = []
    for k in ks:
        top, vals = edge_values(dt, k)
        assert d_fits(dt, k)
        n = -(-vals.size // per_row) * per_row
        vals = np.concatenate([vals, np.zeros(n - vals.size, np.uint16)])
        for chunk in vals.reshape(-1, per_row):
            x = np.zeros(cols, np.uint16)
            body = x[:ngroups * group].reshape(ngroups, group)
            body[:, 0] = top
            body[:, 1:] = chunk.reshape(ngroups, group - 1)
            x[cols - anchors:] = _bf16(2.0 ** (M + 4))
            rows.append(x)
    w = np.full(cols, _bf16(2.0 ** M), np.uint16)
    w[cols - reserved:] = _bf16(1.0)
    return np.stack(rows), w


def d_fits(dt: str, k: int) -> bool:
    """The test values stay within the magnitude the construction allows."""
    return (448.0 if dt == "e4m3" else 6.0) * 2.0 ** k <= 896.0


def edge_columns(cols: int, group: int) -> np.ndarray:
    """Mask of the columns whose y equals x (all but the reserved tail)."""
    anchors = cols // 256
    reserved = -(-anchors // group) * group
    mask = np.zeros(cols, bool)
    mask[:cols - reserved] = True
    return mask
