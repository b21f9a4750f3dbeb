"""First calls from many host threads at once, in a fresh process: the
per-device set-up (device properties, the silu32 table of the SwiGLU form) is
shared state that every entry point reaches on its first call.  Each thread
works on its own stream and inputs and checks its results against the oracle."""
from __future__ import annotations

import os
import subprocess
import sys
import textwrap

import pytest

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

CHILD = textwrap.dedent(r"""
    import sys, threading
    sys.path.insert(0, ROOT)
    sys.path.insert(0, ROOT + "/tests")
    import numpy as np, torch
    import oracle
    import activation_quantization_token_amd as tk
    from activation_quantization_token_amd import inputs

    N = 8
    barrier = threading.Barrier(N)
    results, errors = [None] * N, []

    def dev(bits):
        return torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).cuda()

    def work(i):
        try:
            x = inputs.generate_small(300 + i, 33 + i, 2 * 1024)
            w = inputs.generate_small(400 + i, 1, 1024)[0]
            with torch.cuda.device(0):
                stream = torch.cuda.Stream()
                xd, wd = dev(x), dev(w)
                torch.cuda.synchronize()
                barrier.wait()                          # every thread's first library call at once
                with torch.cuda.stream(stream):
                    sw = tk.swiglu_per_token_cast(xd, 64, "e4m3", True, "f32", stream=stream)
                    pt = tk.per_token_cast(xd, 32, "e2m1", True, "ue8m0", stream=stream)
                    nc = tk.rmsnorm_cast(xd[:, :1024], wd, 1e-6, 128, "e4m3", False, "f32", stream=stream)
                    pc = tk.per_channel_cast(xd, "e4m3", True, "ue8m0", stream=stream)
                stream.synchronize()
                results[i] = (x, w, [tuple(t.cpu().numpy() for t in r) for r in (sw, pt, nc, pc)])
        except Exception as e:                          # reported by the main thread
            errors.append(f"thread {i}: {e!r}")

    threads = [threading.Thread(target=work, args=(i,)) for i in range(N)]
    for t in threads: t.start()
    for t in threads: t.join()
    assert not errors, errors
    for i, (x, w, got) in enumerate(results):
        want = [oracle.swiglu_per_token_cast(x, 64, "e4m3", True, "f32"),
                oracle.per_token_cast(x, 32, "e2m1", True, "ue8m0"),
                oracle.rmsnorm_cast(np.ascontiguousarray(x[:, :1024]), w, 1e-6, 128, "e4m3", False, "f32"),
                oracle.per_channel_cast(x, "e4m3", True, "ue8m0")]
        for name, (gq, gs), (wq, ws) in zip(("swiglu", "per-token", "rmsnorm", "per-channel"), got, want):
            assert np.array_equal(gq, wq), f"thread {i} {name} codes"
            assert np.array_equal(gs.view(np.uint32), np.asarray(ws).view(np.uint32)), f"thread {i} {name} scales"
    print("ok", flush=True)
""")


def test_first_calls_from_many_threads():
    code = f"ROOT = {ROOT!r}\n" + CHILD
    print("[gpu] 8 threads, first calls of four entry points at once, fresh process", flush=True)
    r = subprocess.run([sys.executable, "-c", code], cwd=ROOT, capture_output=True, text=True, timeout=240)
    assert r.returncode == 0 and r.stdout.strip().endswith("ok"), (r.stdout[-2000:] + r.stderr[-4000:])
