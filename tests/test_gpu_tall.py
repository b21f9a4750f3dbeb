"""Inputs taller than the launch grid: above 2^31 - 1 rows the row-form
kernels loop, each workgroup taking rows blockIdx.x, blockIdx.x + grid, ...
The per-token cast of 2^31 + 3 rows and the per-channel cast of 2^31 + 5 rows
(the row-form second pass) are checked against the CPU oracle on sampled
rows: the first and last rows, every row around the grid's size, and random
ones.  A per-channel result depends on a row and the column maxima only, so
the oracle's input is the sampled rows plus, for every column, a row holding
that column's maximum."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
import activation_quantization_token_amd as tk
from gpu_util import first_mismatch, log

pytestmark = pytest.mark.gpu

GRID = 2**31 - 1


def _need(nbytes: int):
    free, _ = torch.cuda.mem_get_info()
    if free < nbytes * 1.1:
        pytest.skip(f"needs {nbytes / 2**30:.0f} GiB of device memory, {free / 2**30:.0f} GiB free")


def _sample(rows: int, seed: int) -> np.ndarray:
    g = np.random.default_rng(seed)
    near = np.arange(GRID - 70, min(rows, GRID + 70))
    idx = np.concatenate([np.arange(64), near, np.arange(rows - 64, rows), g.integers(0, rows, 4096)])
    return np.unique(idx)


def _bits(t: torch.Tensor) -> np.ndarray:
    return t.cpu().view(torch.int16).numpy().view(np.uint16)


def _release():
    """Give the device memory back once the caller has dropped its tensors."""
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


def test_per_token_cast_taller_than_the_grid():
    rows, cols = GRID + 4, 16                      # 2^31 + 3 rows of one 16-column group
    _need(rows * cols * 3 + rows * 4)
    log(f"[gpu] tall per-token cast rows={rows} cols={cols} e4m3 G16 f32")
    torch.manual_seed(7)
    x = torch.empty((rows, cols), dtype=torch.bfloat16, device="cuda").normal_()
    idx = _sample(rows, 1)
    ti = torch.from_numpy(idx).cuda()
    x[ti[::7]] = 0                                 # some all-zero rows (floored scale) among the samples
    q, s = tk.per_token_cast(x, 16, "e4m3", False, "f32")
    torch.cuda.synchronize()
    xs, qs, ss = _bits(x[ti]), q[ti].cpu().numpy(), s[ti].cpu().numpy()
    del x, q, s
    _release()
    want_q, want_s = oracle.per_token_cast(xs, 16, "e4m3", False, "f32")
    assert np.array_equal(ss.view(np.uint32), want_s.view(np.uint32)), first_mismatch(ss.view(np.uint32),
                                                                                      want_s.view(np.uint32))
    assert np.array_equal(qs, want_q), first_mismatch(qs, want_q)


def test_per_channel_cast_taller_than_the_grid():
    rows, cols = GRID + 6, 8                       # 2^31 + 5 rows: the row-form pass loops
    _need(rows * cols * 3 + rows * 2)
    log(f"[gpu] tall per-channel cast rows={rows} cols={cols} e4m3 pow2 f32")
    torch.manual_seed(8)
    x = torch.empty((rows, cols), dtype=torch.bfloat16, device="cuda").normal_()
    x[GRID + 3, 5] = 1000.0                         # a column maximum in the rows past the grid
    q, s = tk.per_channel_cast(x, "e4m3", True, "f32")
    torch.cuda.synchronize()
    at_max = [int(x[:, j].abs().argmax()) for j in range(cols)]
    assert at_max[5] == GRID + 3
    idx = _sample(rows, 2)
    ti = torch.from_numpy(np.concatenate([idx, np.array(at_max)])).cuda()
    xs, qs, ss = _bits(x[ti]), q[ti].cpu().numpy(), s.cpu().numpy()
    del x, q, s
    _release()
    want_q, want_s = oracle.per_channel_cast(xs, "e4m3", True, "f32")
    assert np.array_equal(ss.view(np.uint32), want_s.view(np.uint32).reshape(-1))
    assert np.array_equal(qs, want_q), first_mismatch(qs, want_q)
