"""The library's calls inside a captured HIP graph: several replays, with eager
work and synchronisations between them, each checked against the eager
results (no call records a memset or a host synchronisation once the
per-device table exists)."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import activation_quantization_token_amd as tk
from activation_quantization_token_amd import inputs
from gpu_util import log, to_dev

pytestmark = pytest.mark.gpu


def test_graph_replays_match_eager():
    tk.tk_prepare_device()                   # the SwiGLU table is built outside the capture
    x_bits = inputs.generate(inputs.WORKLOADS[1], rows=512)
    gu_bits = inputs.generate(inputs.WORKLOADS[3], rows=256)
    x, gu = to_dev(x_bits), to_dev(gu_bits)
    w = to_dev(inputs.generate_small(9, 1, x.shape[1], "normal"))[0].contiguous()
    rows, cols = x.shape

    def outputs():
        return {
            "cast": tk.empty_outputs(rows, cols, 32, "e2m1", "ue8m0", x.device),
            "swiglu": tk.empty_outputs(gu.shape[0], gu.shape[1] // 2, 128, "e4m3", "f32", x.device),
            "block": (torch.empty((rows, cols), dtype=torch.uint8, device="cuda"),
                      torch.empty((rows // 128, cols // 128), dtype=torch.float32, device="cuda")),
            "channel": (torch.empty((rows, cols), dtype=torch.uint8, device="cuda"),
                        torch.empty((cols,), dtype=torch.float32, device="cuda")),
            "norm": tk.empty_outputs(rows, cols, 128, "e4m3", "f32", x.device),
            "dequant": torch.empty((rows, cols), dtype=torch.bfloat16, device="cuda"),
        }

    ws = torch.empty((tk.tk_per_channel_workspace_bytes(rows, cols),), dtype=torch.uint8, device="cuda")

    def run(o):
        tk.per_token_cast(x, 32, "e2m1", True, "ue8m0", out=o["cast"])
        tk.swiglu_per_token_cast(gu, 128, "e4m3", True, "f32", out=o["swiglu"])
        tk.per_block_cast(x, 128, 128, "e4m3", False, "f32", out=o["block"])
        tk.per_channel_cast(x, "e4m3", True, "f32", out=o["channel"], workspace=ws)
        tk.rmsnorm_cast(x, w, 1e-6, 128, "e4m3", True, "f32", out=o["norm"])
        tk.per_token_dequant(o["cast"][0], o["cast"][1], cols, 32, "e2m1", "ue8m0", "bf16", out=o["dequant"])

    def flat(o):
        out = []
        for v in o.values():
            for t in (v if isinstance(v, tuple) else (v,)):
                out.append(t.view(torch.uint8).cpu().numpy().copy())
        return out

    eager = outputs()
    run(eager)
    torch.cuda.synchronize()
    want = flat(eager)

    graphed = outputs()
    for t in [t for v in graphed.values() for t in (v if isinstance(v, tuple) else (v,))]:
        t.view(torch.uint8).fill_(0xA5)
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        run(graphed)                          # warm the lazily built kernel tables
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        run(graphed)
    for rep in range(3):
        log(f"[gpu] graph replay {rep}")
        for t in [t for v in graphed.values() for t in (v if isinstance(v, tuple) else (v,))]:
            t.view(torch.uint8).fill_(0x5A)   # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = flat(graphed)
        for i, (a, b) in enumerate(zip(got, want)):
            assert np.array_equal(a, b), f"replay {rep}: output {i} differs from the eager run"


_CAPTURE_CHILD = r'''
import sys
import torch
sys.path.insert(0, sys.argv[1])
import activation_quantization_token_amd as tk
from activation_quantization_token_amd import rawcall
lib = tk.load_library()
rows, cols = 4, 128
gu = torch.ones((rows, 2 * cols), dtype=torch.bfloat16, device="cuda")
q, s = tk.empty_outputs(rows, cols, 128, "e4m3", "f32", gu.device)
side = torch.cuda.Stream()
torch.cuda.synchronize()
fn, args = rawcall.prepare(lib, "tk_swiglu_per_token_cast",
                           (gu.data_ptr(), rows, cols, 2 * cols, q.data_ptr(), cols, s.data_ptr(), 1, 128, 0, 1, 0,
                            side.cuda_stream), {"gate_up": gu, "q": q, "scales": s})
graph = torch.cuda.CUDAGraph()
with torch.cuda.stream(side):
    graph.capture_begin()
    during = fn(*args)                      # the table is not built yet: refused, nothing enqueued
    graph.capture_end()
print("during capture:", during, flush=True)
print("prepare:", lib.tk_prepare_device(), flush=True)
after = fn(*args)
torch.cuda.synchronize()
print("after:", after, flush=True)
'''


def test_table_build_refused_inside_a_capture(tmp_path):
    """A fresh process whose silu32 table is not built yet: a SwiGLU call on a
    stream being captured returns TK_ERROR_UNSUPPORTED and records nothing;
    after the capture, tk_prepare_device builds the table and the same call
    runs."""
    import os
    import subprocess
    import sys
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    log("[gpu] SwiGLU first call inside a graph capture (child process)")
    script = tmp_path / "capture_child.py"
    script.write_text(_CAPTURE_CHILD)
    r = subprocess.run([sys.executable, str(script), root], capture_output=True, text=True, timeout=100)
    assert r.returncode == 0, r.stdout + r.stderr[-3000:]
    lines = dict(l.split(":", 1) for l in r.stdout.splitlines() if ":" in l)
    assert lines["during capture"].strip() == "2", r.stdout           # TK_ERROR_UNSUPPORTED
    assert lines["prepare"].strip() == "0", r.stdout
    assert lines["after"].split()[0] == "0", r.stdout
