"""GPU parity of the per-block and per-channel casts against the CPU oracle
(codes and scales bit for bit)."""
from __future__ import annotations

import concurrent.futures
import os

import numpy as np
import pytest
import torch

import oracle
import activation_quantization_token_amd as tk
from activation_quantization_token_amd import inputs
from gpu_util import Guarded, first_mismatch, log, to_dev

pytestmark = pytest.mark.gpu

VARIANTS = [("e4m3", False, "f32"), ("e4m3", True, "f32"), ("e4m3", True, "ue8m0"),
            ("e2m1", False, "f32"), ("e2m1", True, "f32"), ("e2m1", True, "ue8m0")]
THREADS = min(16, len(os.sched_getaffinity(0)))


def oracle_block(x_bits, br, bc, dt, p2, sf):
    """The oracle split over whole block rows on a thread pool."""
    rows = x_bits.shape[0]
    nbr = -(-rows // br)
    if nbr < 8:
        return oracle.per_block_cast(x_bits, br, bc, dt, p2, sf)
    cuts = np.linspace(0, nbr, min(THREADS, nbr) + 1).astype(int) * br
    cuts[-1] = rows
    with concurrent.futures.ThreadPoolExecutor(THREADS) as ex:
        parts = list(ex.map(lambda i: oracle.per_block_cast(x_bits[cuts[i]:cuts[i + 1]], br, bc, dt, p2, sf),
                            range(len(cuts) - 1)))
    return np.concatenate([p[0] for p in parts]), np.concatenate([p[1] for p in parts])


def oracle_channel(x_bits, dt, p2, sf):
    """The oracle split over column ranges (multiples of 8 columns)."""
    cols = x_bits.shape[1]
    if x_bits.size < (1 << 20) or cols < 8 * THREADS:
        return oracle.per_channel_cast(x_bits, dt, p2, sf)
    cuts = (np.linspace(0, cols // 8, THREADS + 1).astype(int) * 8)
    with concurrent.futures.ThreadPoolExecutor(THREADS) as ex:
        parts = list(ex.map(lambda i: oracle.per_channel_cast(x_bits[:, cuts[i]:cuts[i + 1]], dt, p2, sf),
                            range(THREADS)))
    return np.concatenate([p[0] for p in parts], axis=1), np.concatenate([p[1] for p in parts])


def _host(t: torch.Tensor, like: np.ndarray) -> np.ndarray:
    return t.cpu().numpy().view(like.dtype)


def check_block(x_bits, br, bc, dt, p2, sf, x_ld=None, label=""):
    rows, cols = x_bits.shape
    log(f"[gpu] per-block {label} rows={rows} cols={cols} block={br}x{bc} {dt} pow2={p2} {sf} x_ld={x_ld}")
    want_q, want_s = oracle_block(x_bits, br, bc, dt, p2, sf)
    x = to_dev(x_bits, x_ld)
    gq = Guarded(rows, want_q.shape[1], torch.uint8, 16)
    gs = Guarded(want_s.shape[0], want_s.shape[1], torch.float32 if sf == "f32" else torch.int32, 4)
    tk.per_block_cast(x, br, bc, dt, p2, sf, out=(gq.view, gs.view))
    torch.cuda.synchronize()
    got_q, got_s = _host(gq.view, want_q), _host(gs.view, want_s)
    assert gq.canaries_intact() and gs.canaries_intact(), "write outside the outputs"
    assert np.array_equal(got_s.view(np.uint32), want_s.view(np.uint32)), first_mismatch(
        got_s.view(np.uint32), want_s.view(np.uint32))
    assert np.array_equal(got_q, want_q), first_mismatch(got_q, want_q)


def check_channel(x_bits, dt, p2, sf, x_ld=None, workspace=None, label=""):
    rows, cols = x_bits.shape
    log(f"[gpu] per-channel {label} rows={rows} cols={cols} {dt} pow2={p2} {sf} x_ld={x_ld}")
    want_q, want_s = oracle_channel(x_bits, dt, p2, sf)
    x = to_dev(x_bits, x_ld)
    gq = Guarded(rows, want_q.shape[1], torch.uint8, 16)
    gs = Guarded(1, want_s.shape[0], torch.float32 if sf == "f32" else torch.int32, 4)
    tk.per_channel_cast(x, dt, p2, sf, out=(gq.view, gs.view[0]), workspace=workspace)
    torch.cuda.synchronize()
    got_q, got_s = _host(gq.view, want_q), _host(gs.view[0], want_s)
    assert gq.canaries_intact() and gs.canaries_intact(), "write outside the outputs"
    assert np.array_equal(got_s.view(np.uint32), want_s.view(np.uint32)), first_mismatch(
        got_s.view(np.uint32)[None], want_s.view(np.uint32)[None])
    assert np.array_equal(got_q, want_q), first_mismatch(got_q, want_q)


# (rows, block_rows, extra columns beyond whole 512-column stripes in units of
# 4 blocks): partial last block rows, odd block heights, ragged last stripes.
BLOCK_SHAPES = [(1, 128, 0), (130, 128, 1), (40, 13, 1), (67, 8, 0), (33, 1, 1), (200, 64, 2), (300, 200, 1),
                (520, 256, 0)]


@pytest.mark.parametrize("dt,p2,sf", VARIANTS)
@pytest.mark.parametrize("bc", [16, 32, 64, 128])
@pytest.mark.parametrize("rows,br,extra", BLOCK_SHAPES)
def test_per_block_sweep(dt, p2, sf, bc, rows, br, extra):
    cols = 1024 + extra * 4 * bc
    x = inputs.generate_small(rows * 7 + bc + br, rows, cols, "student_t3" if rows % 2 else "normal")
    check_block(x, br, bc, dt, p2, sf, x_ld=cols + 8 * (rows % 3), label="sweep")


@pytest.mark.parametrize("dt,p2,sf", [("e4m3", False, "f32"), ("e4m3", True, "ue8m0"), ("e2m1", True, "ue8m0")])
@pytest.mark.parametrize("br,bc", [(128, 128), (32, 32)])
def test_per_block_full_size(dt, p2, sf, br, bc):
    w = inputs.WORKLOADS[1]
    x = inputs.generate(w, cache=True)
    check_block(x, br, bc, dt, p2, sf, label="4096x7168")


def test_per_block_largest_workload_128x128():
    """bf16 [32768, 7168]: enough tiles for the 16-rows-per-wave launch."""
    w = inputs.WORKLOADS[4]
    x = inputs.generate(w, cache=True)
    check_block(x, 128, 128, "e4m3", True, "ue8m0", label="32768x7168")


def test_per_block_of_one_row_equals_per_token():
    x = to_dev(inputs.generate_small(3, 96, 7168, "student_t3"))
    log("[gpu] per-block 1x32 vs per-token G32")
    a = tk.per_block_cast(x, 1, 32, "e2m1", True, "ue8m0")
    b = tk.per_token_cast(x, 32, "e2m1", True, "ue8m0")
    torch.cuda.synchronize()
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])


def test_per_block_zero_and_extreme_blocks():
    """All-zero blocks (scale from the 1e-4 floor, codes +-0), a block holding
    the largest bf16 values, and negative zeros."""
    rows, cols = 256, 1024
    x = inputs.generate_small(11, rows, cols, "normal")
    x[:128, :128] = 0
    x[:128, 128:256] = 0x8000                     # -0
    x[128:, :128] = 0x7F7F                        # largest finite bf16
    x[128:, 128] = 0xFF7F
    x[5, 700] = 0x0001                            # smallest subnormal
    for dt, p2, sf in VARIANTS:
        check_block(x, 128, 128, dt, p2, sf, label="zeros/extremes")


# Chunk counts from 1 to 32 (64-row chunks up to 2048 rows, 32 chunks above).
CHANNEL_SHAPES = [(1, 8), (3, 520), (64, 4096), (130, 7168), (1000, 776), (2049, 64), (4096, 1032), (4097, 520),
                  (5003, 1040)]


@pytest.mark.parametrize("dt,p2,sf", VARIANTS)
@pytest.mark.parametrize("rows,cols", CHANNEL_SHAPES)
def test_per_channel_sweep(dt, p2, sf, rows, cols):
    x = inputs.generate_small(rows + cols, rows, cols, "student_t3" if rows % 2 else "normal")
    check_channel(x, dt, p2, sf, x_ld=cols + 8 * (rows % 3), label="sweep")


@pytest.mark.parametrize("dt,p2,sf", [("e4m3", False, "f32"), ("e4m3", True, "ue8m0"), ("e2m1", True, "ue8m0")])
@pytest.mark.parametrize("w", [inputs.WORKLOADS[1], inputs.WORKLOADS[2]], ids=lambda w: f"{w.rows}x{w.cols}")
def test_per_channel_full_size(dt, p2, sf, w):
    x = inputs.generate(w, cache=True)
    check_channel(x, dt, p2, sf, label="full size")


@pytest.mark.parametrize("rows", [4681, 4682, 9362, 9363])
def test_per_channel_size_classes(rows):
    """Both sides of the per-channel cast's size boundaries at 7168 columns:
    x of at most 64 MiB (4681 rows; 2 rows in flight per wave), at most
    128 MiB (4682 and 9362 rows; ordinary second-pass loads), and above
    (9363 rows; non-temporal)."""
    x = inputs.generate_small(rows, rows, 7168, "student_t3")
    check_channel(x, "e4m3", True, "ue8m0", label="size classes")


@pytest.mark.parametrize("rows,cols,dt,p2,sf", [(4100, 8200, "e2m1", True, "f32"), (4100, 8200, "e4m3", False, "f32"),
                                                 (2100, 16392, "e4m3", True, "ue8m0")])
def test_per_channel_row_form_ragged(rows, cols, dt, p2, sf):
    """Above 64 MiB of x the codes come from the row-form pass: rows whose
    width is not a whole number of 1024-column runs, and rows of more runs
    than a workgroup has waves (16392 columns: 17 runs), with ragged row
    counts in the workgroup order."""
    assert rows * cols * 2 > 64 << 20
    x = inputs.generate_small(rows + cols, rows, cols, "student_t3")
    check_channel(x, dt, p2, sf, x_ld=cols + 8, label="row form")


def test_per_channel_zero_columns_and_reused_workspace():
    """Columns of zeros take the floored scale; one workspace serves a larger
    and then a smaller call (its contents on entry do not matter)."""
    rows, cols = 700, 1536
    x = inputs.generate_small(5, rows, cols, "student_t3")
    x[:, 8:24] = 0
    x[:, 40] = 0x8000
    ws = torch.full((tk.tk_per_channel_workspace_bytes(rows, cols),), 0x7F, dtype=torch.uint8, device="cuda")
    check_channel(x, "e4m3", True, "ue8m0", workspace=ws, label="zero columns")
    check_channel(x[:100, :512].copy(), "e2m1", False, "f32", workspace=ws, label="reused workspace")
