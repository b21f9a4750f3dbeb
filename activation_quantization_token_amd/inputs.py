"""Seeded synthetic inputs for the per-token cast, shared by tests, bench and smoke.

This module holds no step of the cast itself: it only draws numbers and rounds
them to bf16 bit patterns.  The pages measure on no public data set and print no
workload; the five workloads below are the cast's standard shapes (hidden size
7168, SwiGLU intermediate size 2 x 2048) with heavy-tailed value mixes that
exercise every scale range.

Recipe (per workload, one ``numpy.random.Generator(PCG64(seed))``), in this
draw order: (1) the base matrix in float64, (2) one log-uniform factor per row,
(3) the outlier positions as distinct flat indices drawn without replacement
(exactly round(p * rows * cols) of them), (4) the all-zero row (the last row).
The result is rounded float64 -> float32 -> bf16, both round-to-nearest-even.
"""
from __future__ import annotations

import dataclasses
import os
import pathlib

import numpy as np

RECIPE_VERSION = 1
CACHE_DIR = pathlib.Path(os.environ.get("TK_INPUT_CACHE",
                                        pathlib.Path(__file__).resolve().parent.parent / "build" / "inputs"))


@dataclasses.dataclass(frozen=True)
class Workload:
    index: int
    name: str
    rows: int
    cols: int                 # output channels (for SwiGLU: the intermediate size I)
    group: int
    out_dtype: str            # "e4m3" | "e2m1"
    round_pow2: bool
    scale_fmt: str            # "f32" | "ue8m0"
    swiglu: bool
    seed: int
    base: str                 # "normal" | "student_t3" | "swiglu"
    row_log10: tuple | None   # per-row factor 10^U(lo, hi)
    outlier_frac: float
    outlier_mul: float
    zero_last_row: bool

    @property
    def in_cols(self) -> int:
        return 2 * self.cols if self.swiglu else self.cols

    @property
    def code_cols(self) -> int:
        return self.cols if self.out_dtype == "e4m3" else self.cols // 2

    @property
    def scale_cols(self) -> int:
        n = self.cols // self.group
        return n if self.scale_fmt == "f32" else n // 4

    def algorithmic_bytes(self, rows: int | None = None) -> int:
        """bf16 input + code bytes + scale bytes (fp32, or packed UE8M0 bytes)."""
        r = self.rows if rows is None else rows
        return r * (2 * self.in_cols + self.code_cols + 4 * self.scale_cols)


WORKLOADS = [
    Workload(0, "e4m3 G128 fp32 scales, bf16 [128 x 7168]", 128, 7168, 128, "e4m3", False, "f32",
             False, 0, "normal", (-3.0, 2.0), 0.001, 100.0, True),
    Workload(1, "e4m3 G128 pow2 fp32 scales, bf16 [4096 x 7168]", 4096, 7168, 128, "e4m3", True,
             "f32", False, 1, "normal", (-3.0, 2.0), 0.01, 50.0, True),
    Workload(2, "e4m3 G32 UE8M0x4 scales, bf16 [16384 x 7168]", 16384, 7168, 32, "e4m3", True,
             "ue8m0", False, 2, "student_t3", (-2.0, 1.0), 0.0, 1.0, False),
    Workload(3, "SwiGLU + e4m3 G128 pow2 fp32 scales, bf16 [8192 x 2*2048]", 8192, 2048, 128,
             "e4m3", True, "f32", True, 3, "swiglu", None, 0.0, 1.0, False),
    Workload(4, "e2m1 G32 UE8M0x4 scales, bf16 [32768 x 7168]", 32768, 7168, 32, "e2m1", True,
             "ue8m0", False, 4, "normal", (-3.0, 2.0), 0.005, 20.0, False),
]


def f64_to_bf16_bits(x: np.ndarray, chunk_rows: int = 2048) -> np.ndarray:
    """float64 -> float32 -> bf16 bit patterns, both steps round-to-nearest-even.

    Inputs are finite and below the float32 range limit, so no NaN handling is
    needed."""
    x = np.asarray(x)
    out = np.empty(x.shape, dtype=np.uint16)
    flat_in = x.reshape(-1, x.shape[-1]) if x.ndim > 1 else x.reshape(1, -1)
    flat_out = out.reshape(flat_in.shape)
    for r0 in range(0, flat_in.shape[0], chunk_rows):
        b = flat_in[r0:r0 + chunk_rows].astype(np.float32).view(np.uint32)
        t = b >> 16
        t &= 1
        t += 0x7FFF
        t += b
        t >>= 16
        flat_out[r0:r0 + chunk_rows] = t
    return out


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def generate(w: Workload | int, rows: int | None = None, cache: bool = False) -> np.ndarray:
    """bf16 bit patterns [rows, in_cols] for workload ``w``.

    ``rows`` (default: the workload's) changes the matrix height; the outlier
    count and the zero row follow the recipe for that height.  With ``cache``
    the matrix is kept as a .npy file under CACHE_DIR for later calls."""
    if isinstance(w, int):
        w = WORKLOADS[w]
    R = w.rows if rows is None else rows
    if cache:
        path = CACHE_DIR / f"w{w.index}_r{R}_v{RECIPE_VERSION}.npy"
        if path.exists():
            return np.load(path)
        x = generate(w, R, cache=False)
        path.parent.mkdir(parents=True, exist_ok=True)
        tmp = path.with_suffix(f".tmp{os.getpid()}.npy")
        np.save(tmp, x)
        os.replace(tmp, path)
        return x
    rng = np.random.Generator(np.random.PCG64(w.seed))
    if w.base == "swiglu":
        gate = 2.0 * rng.standard_normal((R, w.cols))
        up = rng.standard_normal((R, w.cols))
        x = np.concatenate([gate, up], axis=1)
        del gate, up
    else:
        C = w.cols
        if w.base == "normal":
            x = rng.standard_normal((R, C))
        elif w.base == "student_t3":
            x = rng.standard_t(3.0, (R, C))
        else:
            raise ValueError(w.base)
        if w.row_log10 is not None:
            lo, hi = w.row_log10
            x *= (10.0 ** rng.uniform(lo, hi, size=R))[:, None]
        k = int(round(w.outlier_frac * R * C))
        if k:
            idx = rng.choice(R * C, k, replace=False)
            x.reshape(-1)[idx] *= w.outlier_mul
        if w.zero_last_row and R > 0:
            x[R - 1, :] = 0.0
    return f64_to_bf16_bits(x)


def generate_small(seed: int, rows: int, cols: int, kind: str = "normal") -> np.ndarray:
    """Small seeded bf16 matrices for parity sweeps: per-row log-uniform factors
    10^U(-4, 3), 1 % outliers x 64, a zero row when rows > 2, exact ties."""
    rng = np.random.Generator(np.random.PCG64(10_000 + seed))
    if kind == "normal":
        x = rng.standard_normal((rows, cols))
    elif kind == "student_t3":
        x = rng.standard_t(3.0, (rows, cols))
    else:
        raise ValueError(kind)
    x *= (10.0 ** rng.uniform(-4.0, 3.0, size=rows))[:, None]
    k = int(round(0.01 * rows * cols))
    if k:
        idx = rng.choice(rows * cols, k, replace=False)
        x.reshape(-1)[idx] *= 64.0
    if rows > 2:
        x[rows // 2, :] = 0.0
    return f64_to_bf16_bits(x)


def generate_small_f32(seed: int, rows: int, cols: int) -> np.ndarray:
    """Small seeded fp32 matrices (full 24-bit mantissas): per-row log-uniform
    factors 10^U(-4, 3), 1 % outliers x 64, a zero row when rows > 2."""
    rng = np.random.Generator(np.random.PCG64(20_000 + seed))
    x = rng.standard_normal((rows, cols)) * (10.0 ** rng.uniform(-4.0, 3.0, size=rows))[:, None]
    k = int(round(0.01 * rows * cols))
    if k:
        idx = rng.choice(rows * cols, k, replace=False)
        x.reshape(-1)[idx] *= 64.0
    if rows > 2:
        x[rows // 2, :] = 0.0
    return x.astype(np.float32)
