"""Every fp32 value the converters can meet, through the fp32-input cast.

After the scale and the clamp a code's input v lies in [-D, D] (D = 448 for
E4M3, 6 for E2M1).  Groups of 16 here hold 15 test values plus one anchor
whose magnitude makes the group's power-of-two scale exactly 1, so the kernel
converts the test values themselves: all 2 x 1.14e9 fp32 bit patterns with
|v| <= 448 for E4M3 and all 2 x 1.09e9 with |v| <= 6 for E2M1, signed zeros
and subnormals included, each compared with the oracle's encoder."""
from __future__ import annotations

import concurrent.futures
import os

import numpy as np
import pytest
import torch

import oracle
import activation_quantization_token_amd as tk
from gpu_util import log

pytestmark = pytest.mark.gpu

THREADS = min(16, len(os.sched_getaffinity(0)))
CHUNK = 1 << 26                       # positive bit patterns per chunk (x2 with the signs)
COLS = 1024                           # 64 groups of 16 per row


def _oracle_codes(values: np.ndarray, encode) -> np.ndarray:
    parts = np.array_split(values, THREADS)
    with concurrent.futures.ThreadPoolExecutor(THREADS) as ex:
        return np.concatenate(list(ex.map(encode, parts)))


@pytest.mark.parametrize("dt,limit,anchor", [("e4m3", 448.0, 300.0), ("e2m1", 6.0, 5.0)])
def test_converter_every_fp32_in_range(dt, limit, anchor):
    top = int(np.float32(limit).view(np.uint32))              # largest positive pattern with |v| <= D
    encode = oracle.encode_e4m3 if dt == "e4m3" else oracle.encode_e2m1
    for start in range(0, top + 1, CHUNK):
        stop = min(top + 1, start + CHUNK)
        log(f"[gpu] {dt} converter patterns {start:#010x}..{stop - 1:#010x} and their negatives")
        pos = np.arange(start, stop, dtype=np.uint32)
        bits = np.concatenate([pos, pos | np.uint32(0x80000000)])
        n = bits.size
        groups = -(-n // 15)
        pad = groups * 15 - n
        vals = np.concatenate([bits, np.zeros(pad, np.uint32)]).view(np.float32).reshape(groups, 15)
        rows = -(-groups // (COLS // 16))
        x = np.zeros((rows * (COLS // 16), 16), np.float32)
        x[:groups, :15] = vals
        x[:, 15] = np.float32(anchor)
        x = x.reshape(rows, COLS)
        q, s = tk.per_token_cast(torch.from_numpy(x).cuda(), 16, dt, True, "f32")
        torch.cuda.synchronize()
        assert torch.all(s == 1.0), "a group's scale is not 1"
        q = q.cpu().numpy()
        if dt == "e2m1":
            nib = np.empty((rows, COLS), np.uint8)
            nib[:, 0::2], nib[:, 1::2] = q & 0xF, q >> 4
            q = nib
        got = q.reshape(-1, 16)[:groups, :15].reshape(-1)[:n]
        want = _oracle_codes(bits.view(np.float32), encode)
        if not np.array_equal(got, want):
            i = int(np.argmax(got != want))
            raise AssertionError(f"{dt}: pattern {int(bits[i]):#010x} ({float(bits[i:i + 1].view(np.float32)[0])!r}) "
                                 f"-> {int(got[i]):#04x}, oracle {int(want[i]):#04x}; "
                                 f"{int(np.count_nonzero(got != want))} mismatches in the chunk")
