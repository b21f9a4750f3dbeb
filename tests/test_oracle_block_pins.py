"""Pins of the oracle's per-block and per-channel casts (CPU only).

  * whole tensors   -> tests/libref.py's block cast (numpy block max, numpy
                       fp32 division, torch float8 / e8m0 casts, numpy
                       half-to-even rounding for E2M1)
  * reductions      -> a block of one row and G channels is the per-token cast
                       with group G; per-channel is the per-token cast of the
                       transposed tensor with one group per row
  * exact example   -> a 3 x 4 tensor worked by hand in exact rationals
"""
from __future__ import annotations

import numpy as np
import pytest

import libref
import oracle
from activation_quantization_token_amd import inputs

VARIANTS = [("e4m3", False, "f32"), ("e4m3", True, "ue8m0"), ("e2m1", True, "ue8m0"), ("e2m1", False, "f32")]


@pytest.mark.parametrize("dt,p2,sf", VARIANTS)
@pytest.mark.parametrize("br,bc", [(128, 128), (32, 32), (16, 64), (1, 16), (64, 1 * 128)])
@pytest.mark.parametrize("rows", [1, 37, 130])
def test_per_block_vs_library_composition(dt, p2, sf, br, bc, rows):
    cols = 4 * bc * (2 if bc < 128 else 1)
    x = inputs.generate_small(br + bc + rows, rows, cols, "student_t3" if rows % 2 else "normal")
    got = oracle.per_block_cast(x, br, bc, dt, p2, sf)
    want = libref.per_block_cast(x, br, bc, dt, p2, sf)
    assert np.array_equal(got[0], want[0])
    assert np.array_equal(got[1].view(np.uint32), want[1].view(np.uint32))


@pytest.mark.parametrize("dt,p2,sf", VARIANTS)
@pytest.mark.parametrize("group", [16, 32, 64, 128])
def test_block_of_one_row_is_per_token(dt, p2, sf, group):
    x = inputs.generate_small(group, 9, 8 * group, "student_t3")
    a = oracle.per_block_cast(x, 1, group, dt, p2, sf)
    b = oracle.per_token_cast(x, group, dt, p2, sf)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


def _nibbles(q: np.ndarray) -> np.ndarray:
    n = np.empty((q.shape[0], q.shape[1] * 2), np.uint8)
    n[:, 0::2], n[:, 1::2] = q & 0xF, q >> 4
    return n


@pytest.mark.parametrize("dt,p2,sf", VARIANTS)
@pytest.mark.parametrize("rows,cols", [(64, 256), (128, 512)])
def test_per_channel_is_per_token_of_transpose(dt, p2, sf, rows, cols):
    x = inputs.generate_small(rows + cols, rows, cols, "student_t3")
    q, s = oracle.per_channel_cast(x, dt, p2, sf)
    qt, st = oracle.per_token_cast(np.ascontiguousarray(x.T), rows, dt, p2, "f32")
    if dt == "e4m3":
        assert np.array_equal(q, qt.T)
    else:
        assert np.array_equal(_nibbles(q), _nibbles(qt).T)
    if sf == "f32":
        assert np.array_equal(s.view(np.uint32), st.reshape(-1).view(np.uint32))
    else:
        e8 = (st.reshape(-1).view(np.uint32) >> 23).astype(np.uint8)
        assert np.array_equal(s.view(np.uint8), e8)


def test_exact_worked_example():
    """3 x 4 bf16 values, blocks of 2 rows x 2 channels, e4m3, fp32 scales.
    Block (0,0) holds {1, -3, 0.5, 2}: amax 3, s = fl32(3/448); block (0,1)
    holds {448, 0, -0, 7}: s = 1, codes are the values; the partial block row
    (row 2) holds {1e-6, -1e-6} -> amax floored to 1e-4 and {0, 100}."""
    vals = np.array([[1.0, -3.0, 448.0, 0.0],
                     [0.5, 2.0, -0.0, 7.0],
                     [1e-6, -1e-6, 0.0, 100.0]], np.float32)
    bits = (vals.view(np.uint32) >> 16).astype(np.uint16)  # all exact in bf16 except 1e-6
    q, s = oracle.per_block_cast(bits, 2, 2, "e4m3", False, "f32")
    x = libref.widen(bits)
    s00 = np.float32(3.0) / np.float32(448.0)
    assert s[0, 0] == s00 and s[0, 1] == np.float32(1.0)
    s10 = np.float32(1e-4) / np.float32(448.0)
    s11 = np.float32(100.0) / np.float32(448.0)
    assert s[1, 0] == s10 and s[1, 1] == s11
    # block (0,1), s = 1: 448 -> 0x7E, 0 -> 0x00, -0 -> 0x80, 7 -> 0x4E (1.75 * 2^2)
    assert q[0, 2] == 0x7E and q[0, 3] == 0x00 and q[1, 2] == 0x80 and q[1, 3] == 0x4E
    # -3 / s00 = -448 exactly? fl32(3/448) * 448 need not be 3; the quotient
    # lies within one ulp of 448 and saturates to the largest code.
    assert q[0, 1] == 0xFE
    # 1e-6 (as bf16) / fl32(1e-4/448): about 4.47 -> nearest e4m3 4.5 = 0x49
    v = x[2, 0] / s10
    assert 4.25 < v < 4.75 and q[2, 0] == 0x49 and q[2, 1] == 0xC9
    # 100 / fl32(100/448) rounds to 448 -> 0x7E
    assert q[2, 3] == 0x7E and q[2, 2] == 0x00


def test_per_block_rejects_bad_shapes():
    x = inputs.generate_small(0, 4, 96)
    for args in ((128, 64, "e4m3", False, "f32"), (128, 32, "e4m3", False, "ue8m0"),
                 (0, 32, "e4m3", False, "f32")):
        with pytest.raises(ValueError):
            oracle.per_block_cast(x, *args)
