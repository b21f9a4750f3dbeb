"""Helpers for the GPU parity tests: device upload, canary-guarded outputs and a
row-parallel driver for the CPU oracle."""
from __future__ import annotations

import concurrent.futures
import os
import sys

import numpy as np
import torch

import oracle

CANARY = 0xA5


def log(msg: str):
    print(msg, flush=True)
    sys.stdout.flush()


def to_dev(bits: np.ndarray, ld: int | None = None) -> torch.Tensor:
    """bf16 bit patterns [rows, cols] -> a bf16 GPU tensor, optionally a view
    into a wider buffer with row stride `ld` (the extra columns hold NaN bits)."""
    bits = np.ascontiguousarray(bits, dtype=np.uint16)
    rows, cols = bits.shape
    host = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16)
    if ld is None or ld == cols:
        return host.to("cuda")
    buf = torch.full((rows, ld), float("nan"), dtype=torch.bfloat16, device="cuda")
    buf[:, :cols] = host.to("cuda")
    return buf[:, :cols]


class Guarded:
    """An output tensor view [rows, cols] of `dtype` inside a buffer whose other
    bytes hold CANARY, so writes outside the view can be detected."""

    def __init__(self, rows, cols, dtype, pad_cols, align_bytes=16):
        itemsize = torch.empty((), dtype=dtype).element_size()
        pad = max(pad_cols, 1)
        pad = -(-pad * itemsize // align_bytes) * align_bytes // itemsize   # keep the view aligned
        self.ld = cols + 2 * pad
        self.buf = torch.full((rows + 2, self.ld * itemsize), CANARY, dtype=torch.uint8, device="cuda")
        self.view = self.buf.view(dtype)[1:rows + 1, pad:pad + cols]
        self.rows, self.cols, self.pad, self.itemsize = rows, cols, pad, itemsize

    def canaries_intact(self) -> bool:
        b = self.buf.cpu().numpy().copy()
        lo, hi = self.pad * self.itemsize, (self.pad + self.cols) * self.itemsize
        b[1:self.rows + 1, lo:hi] = CANARY
        return bool((b == CANARY).all())


def oracle_cast(x_bits: np.ndarray, group, out_dtype, round_pow2, scale_fmt, swiglu=False,
                threads: int | None = None):
    """The oracle over row blocks on a thread pool (ctypes releases the GIL)."""
    fn = oracle.swiglu_per_token_cast if swiglu else oracle.per_token_cast
    rows = x_bits.shape[0]
    threads = threads or min(16, len(os.sched_getaffinity(0)))
    if rows < 64 or threads == 1:
        return fn(x_bits, group, out_dtype, round_pow2, scale_fmt)
    bounds = np.linspace(0, rows, threads + 1).astype(int)
    with concurrent.futures.ThreadPoolExecutor(threads) as ex:
        parts = list(ex.map(lambda i: fn(x_bits[bounds[i]:bounds[i + 1]], group, out_dtype,
                                         round_pow2, scale_fmt), range(threads)))
    return np.concatenate([p[0] for p in parts]), np.concatenate([p[1] for p in parts])


def first_mismatch(got: np.ndarray, want: np.ndarray) -> str:
    bad = np.argwhere(got != want)
    if bad.size == 0:
        return "none"
    r, c = bad[0]
    return f"{bad.shape[0]} mismatches; first at row {r} col {c}: got {got[r, c]!r} want {want[r, c]!r}"
