"""The per-channel cast's no-allocation entry point (tk_per_channel_cast_noalloc,
called through the C ABI) against the workspace entry point
(tk_per_channel_cast) and the oracle, bit for bit: several calls in a row on
the one static workspace, each smaller than the one before, with guarded
outputs; and the size limit."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
import activation_quantization_token_amd as tk
from activation_quantization_token_amd import binding, inputs, rawcall
from gpu_util import Guarded, first_mismatch, log, to_dev

pytestmark = pytest.mark.gpu

QD, SF = binding.QDTYPES, binding.SCALE_FMTS


def noalloc_call(x, dt, p2, sf):
    """The no-allocation cast of x into guarded outputs; returns (codes, scales, canaries intact)."""
    rows, cols = x.shape
    q = Guarded(rows, cols if dt == "e4m3" else cols // 2, torch.uint8, 24)
    s = Guarded(1, cols if sf == "f32" else cols // 4, torch.float32 if sf == "f32" else torch.int32, 4)
    stream = torch.cuda.current_stream().cuda_stream
    fn, args = rawcall.prepare(binding.load_library(), "tk_per_channel_cast_noalloc",
                               (x.data_ptr(), rows, cols, x.stride(0), q.view.data_ptr(), q.view.stride(0),
                                s.view.data_ptr(), QD[dt], int(p2), SF[sf], stream),
                               {"x": x, "q": q.view, "scales": s.view})
    st = fn(*args)
    assert st == 0, binding.tk_status_string(st)
    torch.cuda.synchronize()
    ok = q.canaries_intact() and s.canaries_intact()
    return q.view.cpu().numpy(), s.view.cpu().numpy().reshape(-1), ok


# (rows, cols, code format, pow2, scale format): each smaller than the one before
CALLS = [(32768, 7168, "e2m1", True, "ue8m0"),     # the largest workload's shape
         (4096, 7168, "e4m3", True, "f32"),
         (1031, 2048, "e4m3", False, "f32"),
         (67, 512, "e2m1", True, "ue8m0")]


def test_noalloc_matches_the_workspace_entry_point_call_after_call():
    for i, (rows, cols, dt, p2, sf) in enumerate(CALLS):
        log(f"[gpu] per-channel no-alloc call {i}: rows={rows} cols={cols} {dt} pow2={p2} {sf}")
        if rows == 32768:
            x_bits = inputs.generate(inputs.WORKLOADS[4], cache=True)
        else:
            x_bits = inputs.generate_small(rows + cols, rows, cols, "student_t3" if rows % 2 else "normal")
        x = to_dev(x_bits, cols + 8 if rows % 2 else None)
        got_q, got_s, ok = noalloc_call(x, dt, p2, sf)
        assert ok, "write outside the output views (canary overwritten)"
        want_q, want_s = tk.per_channel_cast(x, dt, p2, sf)        # the workspace entry point
        torch.cuda.synchronize()
        want_q, want_s = want_q.cpu().numpy(), want_s.cpu().numpy().reshape(-1)
        assert np.array_equal(got_q, want_q), first_mismatch(got_q, want_q)
        assert np.array_equal(got_s.view(np.uint32), want_s.view(np.uint32))
        if rows <= 4096:                                           # and the oracle where it is quick
            oq, os_ = oracle.per_channel_cast(x_bits, dt, p2, sf)
            assert np.array_equal(got_q, oq), first_mismatch(got_q, oq)
            assert np.array_equal(got_s.view(np.uint32), os_.reshape(-1).view(np.uint32))


def test_noalloc_size_limit():
    """A cast whose column maxima exceed the static workspace is refused
    before anything is launched; the largest that fits runs."""
    limit = binding.tk_per_channel_noalloc_max_workspace_bytes()
    assert limit == 1088 << 10
    rows, cols = 4096, 16384 + 8                 # 32 chunks x 16392 columns x 2 bytes + 4 per column > 1088 KiB
    assert tk.tk_per_channel_workspace_bytes(rows, cols) > limit
    log(f"[gpu] per-channel no-alloc refused at rows={rows} cols={cols}")
    x = torch.zeros((rows, cols), dtype=torch.bfloat16, device="cuda")
    q = torch.full((rows, cols), 0xA5, dtype=torch.uint8, device="cuda")
    s = torch.full((cols,), 7.0, dtype=torch.float32, device="cuda")
    st = binding.tk_per_channel_cast_noalloc(x.data_ptr(), rows, cols, cols, q.data_ptr(), cols, s.data_ptr(), 0, 1,
                                             0, torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    assert st == 2 and bool((q == 0xA5).all()) and bool((s == 7.0).all())
    cols = 16384                                  # exactly the limit
    assert tk.tk_per_channel_workspace_bytes(rows, cols) == limit
    x_bits = inputs.generate_small(11, rows, cols)
    got_q, got_s, ok = noalloc_call(to_dev(x_bits), "e4m3", True, "f32")
    assert ok
    want_q, want_s = tk.per_channel_cast(to_dev(x_bits), "e4m3", True, "f32")
    assert np.array_equal(got_q, want_q.cpu().numpy())
    assert np.array_equal(got_s.view(np.uint32), want_s.cpu().numpy().reshape(-1).view(np.uint32))
