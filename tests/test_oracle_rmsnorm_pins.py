"""Pins of the oracle's RMSNorm forward and its fused cast (CPU only).

  * sum of squares -> the exact rational sum (Python integers / Fraction)
                      rounded by tests/exact.py, on random rows of wide
                      dynamic range and on rows built to land on or next to
                      rounding midpoints, in the subnormal range and past the
                      largest binary32 value
  * y              -> numpy float32 division, sqrt and products on that sum
                      (tests/libref.py), with and without a weight
  * fused cast     -> the library-composed cast of that y
  * special rows   -> a row of one repeated value, an all-zero row
"""
from __future__ import annotations

import numpy as np
import pytest

import libref
import oracle
from activation_quantization_token_amd import inputs


def bf16(vals) -> np.ndarray:
    """bf16 bits of values that bf16 holds exactly."""
    a = np.asarray(vals, dtype=np.float32)
    b = a.view(np.uint32)
    assert np.all((b & 0xFFFF) == 0), "value not exact in bf16"
    return (b >> 16).astype(np.uint16)


def wide_rows(seed: int, rows: int, cols: int) -> np.ndarray:
    """bf16 bits of values spread over most of the bf16 exponent range."""
    rng = np.random.default_rng(seed)
    exp = rng.integers(-132, 62, size=(rows, cols))
    mant = rng.integers(0, 128, size=(rows, cols))
    sign = rng.integers(0, 2, size=(rows, cols))
    vals = np.ldexp(1.0 + mant / 128.0, exp) * np.where(sign, -1.0, 1.0)
    bits = libref.f32_to_bf16_bits(vals.astype(np.float32))
    return bits


@pytest.mark.parametrize("kind", ["normal", "student_t3", "wide"])
def test_sum_squares_exact(kind):
    if kind == "wide":
        x = wide_rows(7, 24, 300)
        x[::3, ::2] = 0
    else:
        x = inputs.generate_small(5, 12, 7168 if kind == "normal" else 2048, kind)
    got = oracle.sum_squares(x)
    want = libref.sum_squares_exact_f32(x)
    assert np.array_equal(got.view(np.uint32), want.view(np.uint32))


MIDPOINT_ROWS = [
    ([1.0, 2.0 ** -12], 1.0),                                   # 1 + 2^-24: tie -> even (1)
    ([1.0, 2.0 ** -12, 2.0 ** -40], 1.0 + 2.0 ** -23),          # just above the tie
    ([1.0 + 2.0 ** -7, 2.0 ** -12], None),                      # odd significand at the tie
    ([2.0 ** -75], 0.0),                                        # 2^-150: tie -> even (0)
    ([2.0 ** -75, 2.0 ** -80], 2.0 ** -149),                    # just above it
    ([2.0 ** -75, 2.0 ** -100], 2.0 ** -149),                   # above it by less than 24 bits resolve
    ([2.0 ** -70, 2.0 ** -75], None),                           # subnormal sum
    ([2.0 ** 63] * 2, 2.0 ** 127),
    ([2.0 ** 63] * 4, float("inf")),                            # 2^128: past the largest value
    ([-(2.0 ** 20), 3.0, 2.0 ** -30, -(2.0 ** -133)], None),    # smallest subnormal bf16
]


@pytest.mark.parametrize("vals,expect", MIDPOINT_ROWS)
def test_sum_squares_rounding_cases(vals, expect):
    x = bf16(vals)[None, :]
    got = oracle.sum_squares(x)[0]
    want = libref.sum_squares_exact_f32(x)[0]
    assert got.view(np.uint32) == want.view(np.uint32)
    if expect is not None:
        assert got == np.float32(expect)


@pytest.mark.parametrize("weighted", [False, True])
@pytest.mark.parametrize("eps", [1e-6, 1e-5, 0.5])
def test_rmsnorm_vs_library_composition(weighted, eps):
    x = inputs.generate_small(11, 16, 1024, "student_t3")
    x[3] = libref.f32_to_bf16_bits(libref.widen(x[3]) * np.float32(2.0 ** -12))   # ss near eps
    x[4] = 0
    w = inputs.generate_small(12, 1, 1024, "normal")[0] if weighted else None
    want = libref.rmsnorm(x, w, eps)
    got = oracle.rmsnorm(x, w, eps, "f32")
    assert np.array_equal(got.view(np.uint32), want.view(np.uint32))
    got16 = oracle.rmsnorm(x, w, eps, "bf16")
    assert np.array_equal(got16, libref.f32_to_bf16_bits(want))


@pytest.mark.parametrize("group,dt,p2,sf", [(128, "e4m3", False, "f32"), (128, "e4m3", True, "ue8m0"),
                                          (32, "e2m1", True, "ue8m0"), (16, "e4m3", True, "f32")])
def test_rmsnorm_cast_vs_composition(group, dt, p2, sf):
    x = inputs.generate_small(21, 9, 2048, "normal")
    w = inputs.generate_small(22, 1, 2048, "student_t3")[0]
    y = libref.rmsnorm(x, w, 1e-6)
    want = libref.cast_values(y, group, dt, p2, sf)
    got = oracle.rmsnorm_cast(x, w, 1e-6, group, dt, p2, sf)
    assert np.array_equal(got[0], want[0])
    assert np.array_equal(got[1].view(np.uint32), want[1].view(np.uint32))


def test_rmsnorm_of_a_constant_row():
    """x_j = a for all j: ss = fl32(C a^2) (exact here), r = 1/sqrt(a^2 + eps)."""
    a, cols, eps = np.float32(3.0), 512, np.float32(1e-6)
    x = np.full((1, cols), bf16([a])[0], dtype=np.uint16)
    ss = np.float32(cols) * a * a
    t = np.float32(np.float32(ss / np.float32(cols)) + eps)
    r = np.float32(np.float32(1.0) / np.float32(np.sqrt(t)))
    y = oracle.rmsnorm(x, None, float(eps), "f32")
    assert np.all(y == np.float32(a * r))


def test_rmsnorm_zero_row_keeps_signed_zeros():
    x = np.zeros((1, 256), dtype=np.uint16)
    x[0, 1::2] = 0x8000
    y = oracle.rmsnorm(x, None, 1e-6, "f32")
    assert np.all(y == 0) and np.array_equal(np.signbit(y[0]), np.arange(256) % 2 == 1)


def test_rmsnorm_rejects_bad_arguments():
    x = inputs.generate_small(0, 2, 64)
    for eps in (0.0, -1.0, float("inf")):
        with pytest.raises(ValueError):
            oracle.rmsnorm(x, None, eps)
    with pytest.raises(ValueError):
        oracle.rmsnorm_cast(x, None, 1e-6, 48)


@pytest.mark.parametrize("cols,group", [(7168, 32), (7168, 128), (2048, 16), (16384, 64)])
@pytest.mark.parametrize("dt", ["e4m3", "e2m1"])
def test_edge_rows_make_y_equal_x(cols, group, dt):
    """The rounding-edge rows (tests/norm_edges.py) do what their construction
    claims under the oracle: r = 2^-M exactly, so y equals x on every test
    column and 16 on the anchors; every group leads with its maximum D * 2^k."""
    import norm_edges
    x, w = norm_edges.edge_rows(cols, group, dt, ks=[-24, -9, 0, 1])
    y = oracle.rmsnorm(x, w, 1e-6, "f32")
    mask = norm_edges.edge_columns(cols, group)
    assert np.array_equal(y[:, mask].view(np.uint32), x[:, mask].astype(np.uint32) << 16)
    tail = y[:, ~mask]
    assert np.all((tail == 16.0) | (tail == 0.0)) and np.count_nonzero(tail == 16.0) == x.shape[0] * (cols // 256)
    d = 448.0 if dt == "e4m3" else 6.0
    lead = x[:, :int(mask.sum())].reshape(x.shape[0], -1, group)[:, :, 0]
    assert set(np.unique(lead).tolist()) <= {int(bf16([d * 2.0 ** k])[0]) for k in (-24, -9, 0, 1)}
    q, _ = oracle.rmsnorm_cast(x, w, 1e-6, group, dt, True, "f32")
    codes = np.unique(q) if dt == "e4m3" else np.unique(np.concatenate([q & 0xF, q >> 4]))
    assert codes.size == (254 if dt == "e4m3" else 16), "the rows do not reach every code"
