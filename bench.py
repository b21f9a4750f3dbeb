#!/usr/bin/env python3
"""Benchmark of the per-token / per-group activation cast on one MI355X.

One step = one launch of the cast over the whole workload, inputs resident in
HBM.  Default workload: e2m1 codes, G = 32, UE8M0 x4 scales on bf16
[32768 x 7168], the largest of the cast's workloads (the other workloads are
selectable with --workload and are parity-test cases).  Prints ONE JSON line
on stdout; progress goes to stderr.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload I]
                    [--no-cpu-baseline]
"""
from __future__ import annotations

import argparse
import concurrent.futures
import hashlib
import json
import os
import pathlib
import sys
import time

ROOT = pathlib.Path(__file__).resolve().parent
sys.path.insert(0, str(ROOT))

HBM_PEAK_GBS = 8000.0            # MI355X HBM3E, AMD published peak
TRAFFIC_FILE = ROOT / "profiles" / "traffic.json"
KERNEL_SRC = ROOT / "activation_quantization_token_amd" / "csrc" / "tk_quant.hip"


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def kernel_source_hash() -> str:
    return hashlib.sha256(KERNEL_SRC.read_bytes()).hexdigest()[:16]


def measured_traffic(workload_index: int):
    """HBM bytes per launch from the committed rocprofv3 counter runs, or None
    when none exist for this workload or the kernel source changed since."""
    try:
        data = json.loads(TRAFFIC_FILE.read_text())
    except (OSError, ValueError):
        return None
    entry = data.get(f"workload{workload_index}")
    if not entry or entry.get("kernel_source_sha256_16") != kernel_source_hash():
        return None
    return entry.get("hbm_bytes_per_launch")


def cpu_baseline(w, x_bits, threads: int):
    """The CPU oracle over row blocks on `threads` host threads, timed on the
    whole workload (a sample of rows when the workload is large)."""
    import numpy as np
    import oracle
    fn = oracle.swiglu_per_token_cast if w.swiglu else oracle.per_token_cast
    rows = x_bits.shape[0]
    sample = min(rows, 32768)
    xs = x_bits[:sample]
    bounds = np.linspace(0, sample, threads + 1).astype(int)
    fn(xs[:8], w.group, w.out_dtype, w.round_pow2, w.scale_fmt)          # load the library
    t0 = time.perf_counter()
    with concurrent.futures.ThreadPoolExecutor(threads) as ex:
        list(ex.map(lambda i: fn(xs[bounds[i]:bounds[i + 1]], w.group, w.out_dtype, w.round_pow2,
                                 w.scale_fmt), range(threads)))
    dt = time.perf_counter() - t0
    return {
        "value": round(w.algorithmic_bytes(sample) / dt / 1e9, 3),
        "unit": "GB/s",
        "cores": threads,
        "kind": "oracle",
        "sample": f"rows 0..{sample - 1} of the workload ({sample} x {w.in_cols} bf16), "
                  f"{threads} threads over row blocks, {dt:.2f} s wall",
        "tokens_per_s": round(sample / dt, 1),
    }


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", type=int, default=4)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: the cast is row-parallel with no exchange between GPUs, "
              "and this build runs on a single GPU only (--gpus 1).", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch
    import activation_quantization_token_amd as tk
    from activation_quantization_token_amd import inputs

    w = inputs.WORKLOADS[args.workload]
    log(f"[bench] workload {w.index}: {w.name}; generating inputs")
    x_bits = inputs.generate(w, cache=True)
    dev = torch.device("cuda:0")
    x = torch.from_numpy(x_bits.view(np.int16)).view(torch.bfloat16).to(dev)
    q, s = tk.empty_outputs(w.rows, w.cols, w.group, w.out_dtype, w.scale_fmt, dev)
    fn = tk.swiglu_per_token_cast if w.swiglu else tk.per_token_cast
    if w.swiglu:
        tk.tk_prepare_device()

    def step():
        fn(x, w.group, w.out_dtype, w.round_pow2, w.scale_fmt, out=(q, s))

    log(f"[bench] warmup {args.warmup} steps")
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    # Timed region: K back-to-back launches on the current stream, with an
    # event pair around each launch for the per-launch kernel duration.
    stream = torch.cuda.current_stream(dev)
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(args.steps)]
    log(f"[bench] timing {args.steps} steps")
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for a, b in ev:
        a.record(stream)
        step()
        b.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    launch_ms = [a.elapsed_time(b) for a, b in ev]
    span_ms = ev[0][0].elapsed_time(ev[-1][1])

    nbytes = w.algorithmic_bytes()
    ms_per_step = span_ms / args.steps
    value = nbytes * args.steps / (span_ms / 1e3) / 1e9
    avg_launch_ms = float(np.mean(launch_ms))
    achieved = nbytes / (avg_launch_ms / 1e3) / 1e9
    traffic = measured_traffic(w.index)

    out = {
        "metric": "per-token cast GB/s (in+out bytes) and % of MI355X HBM peak; tokens/s",
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {
            "workload": w.name, "rows": w.rows, "cols": w.cols, "group": w.group,
            "out_dtype": w.out_dtype, "round_pow2": w.round_pow2, "scale_fmt": w.scale_fmt,
            "swiglu": w.swiglu, "seed": w.seed, "bytes_per_step": nbytes,
        },
        "pct_hbm_peak": round(100.0 * value / HBM_PEAK_GBS, 2),
        "tokens_per_s": round(w.rows * args.steps / (span_ms / 1e3), 1),
        "wall_s_timed_region": round(wall, 4),
        "roofline": {
            "bound": "hbm",
            "achieved": round(achieved, 2),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4),
            "traffic": traffic,
            "kernel_avg_us": round(avg_launch_ms * 1e3, 3),
            "kernel_min_us": round(float(np.min(launch_ms)) * 1e3, 3),
            "algorithmic_bytes_per_launch": nbytes,
        },
    }
    if not args.no_cpu_baseline:
        threads = min(16, len(os.sched_getaffinity(0)))
        log(f"[bench] CPU baseline: oracle on {threads} threads")
        out["cpu_baseline"] = cpu_baseline(w, x_bits, threads)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
