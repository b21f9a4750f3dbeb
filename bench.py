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
MALL_BYTES = 256 << 20           # MI355X Infinity Cache
TRAFFIC_FILE = ROOT / "profiles" / "traffic.json"
# the per-token cast kernels' sources: their hash keys the stored counter runs
KERNEL_SRCS = [ROOT / "activation_quantization_token_amd" / "csrc" / n for n in ("tk_quant.hip", "tk_device.h")]


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for src in KERNEL_SRCS:
        h.update(src.read_bytes())
    return h.hexdigest()[:16]


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


def _pmc_per_kernel(csv_path, counter):
    """{kernel name: [value per dispatch]} for one counter of a rocprofv3 --pmc CSV."""
    import csv
    vals = {}
    for r in csv.DictReader(open(csv_path)):
        if r["Counter_Name"] != counter:
            continue
        vals.setdefault(r["Kernel_Name"], {}).setdefault(r["Dispatch_Id"], 0.0)
        vals[r["Kernel_Name"]][r["Dispatch_Id"]] += float(r["Counter_Value"])
    return {k: list(v.values()) for k, v in vals.items()}


def summarize_pmc(workload_index, fetch_csv, write_csv, traffic_file=None):
    """HBM bytes per cast launch from FETCH_SIZE / WRITE_SIZE (KiB per dispatch),
    each scaled by what the same counter reads for the library's 1 GiB
    streaming copy in the same run (known size: 1 GiB read, 1 GiB written)."""
    import numpy as np
    from activation_quantization_token_amd import inputs
    w = inputs.WORKLOADS[workload_index]
    fetch, write = _pmc_per_kernel(fetch_csv, "FETCH_SIZE"), _pmc_per_kernel(write_csv, "WRITE_SIZE")
    copy_k = [k for k in fetch if "copy_stream_kernel" in k]
    cast_k = [k for k in fetch if "cast" in k and "copy_stream" not in k]
    if not copy_k or not cast_k:
        raise SystemExit("need both the cast kernel and the calibration copy in the counter runs")
    kib = float(1 << 20)
    f_scale = kib / float(np.median(fetch[copy_k[0]]))
    w_scale = kib / float(np.median(write[copy_k[0]]))
    f_kib, w_kib = float(np.median(fetch[cast_k[0]])), float(np.median(write[cast_k[0]]))
    hbm = (f_kib * f_scale + w_kib * w_scale) * 1024
    entry = {
        "kernel": cast_k[0],
        "kernel_source_sha256_16": kernel_source_hash(),
        "fetch_size_kib": f_kib, "write_size_kib": w_kib,
        "copy_fetch_scale": round(f_scale, 4), "copy_write_scale": round(w_scale, 4),
        "hbm_bytes_per_launch": int(round(hbm)),
        "algorithmic_bytes_per_launch": w.algorithmic_bytes(),
        "ratio_to_algorithmic": round(hbm / w.algorithmic_bytes(), 5),
    }
    out = pathlib.Path(traffic_file) if traffic_file is not None else TRAFFIC_FILE
    try:
        data = json.loads(out.read_text())
    except (OSError, ValueError):
        data = {}
    data[f"workload{workload_index}"] = entry
    out.parent.mkdir(exist_ok=True)
    out.write_text(json.dumps(data, indent=2) + "\n")
    print(json.dumps(entry, indent=2))
    return entry


# Raw TCC/EA request counters, the independent check of the calibrated
# FETCH_SIZE figure: FETCH_SIZE prices every read request that is neither a
# 32-byte one nor counted by TCC_BUBBLE at 64 bytes, and on this GPU the
# streaming reads are 128-byte requests that TCC_BUBBLE does not count.
EA_READ_COUNTERS = ("TCC_EA0_RDREQ_sum", "TCC_EA0_RDREQ_32B_sum", "TCC_BUBBLE_sum", "TCC_EA0_RDREQ_DRAM_sum")
EA_WRITE_COUNTERS = ("TCC_EA0_WRREQ_sum", "TCC_EA0_WRREQ_64B_sum", "TCC_EA0_WRREQ_DRAM_sum")


def summarize_ea(read_csv, write_csv, read_request_bytes=128):
    """Per kernel: the median request counts of two rocprofv3 --pmc runs
    (EA_READ_COUNTERS, EA_WRITE_COUNTERS) and the bytes they stand for: reads
    at 32 bytes for a 32-byte request and `read_request_bytes` for any other,
    writes at 64 bytes for a 64-byte request and 32 for any other.  The
    library's 1 GiB streaming copy, run in the same processes, checks the
    request size: its bytes must come out at 1 GiB each way."""
    import numpy as np
    out = {}
    for path, counters in ((read_csv, EA_READ_COUNTERS), (write_csv, EA_WRITE_COUNTERS)):
        for c in counters:
            for k, v in _pmc_per_kernel(path, c).items():
                out.setdefault(k, {})[c] = float(np.median(v))
    for k, d in out.items():
        if "TCC_EA0_RDREQ_sum" in d:
            r32 = d.get("TCC_EA0_RDREQ_32B_sum", 0.0)
            d["read_bytes"] = int(round(32 * r32 + read_request_bytes * (d["TCC_EA0_RDREQ_sum"] - r32)))
        if "TCC_EA0_WRREQ_sum" in d:
            w64 = d.get("TCC_EA0_WRREQ_64B_sum", 0.0)
            d["write_bytes"] = int(round(64 * w64 + 32 * (d["TCC_EA0_WRREQ_sum"] - w64)))
    for k, d in sorted(out.items()):
        print(f"{k[:100]:100s} " + " ".join(f"{c}={v:.0f}" for c, v in d.items()))
    return out


def _oracle_step(op: str, w, block, weight_bits):
    """(fn(rows of x) -> None, rows must be a multiple of, algorithmic bytes per row)
    for one operation's CPU oracle; the per-row byte count matches the bench's."""
    import numpy as np
    import oracle
    code_cols = w.code_cols
    if op == "cast":
        fn = oracle.swiglu_per_token_cast if w.swiglu else oracle.per_token_cast
        return (lambda xs: fn(xs, w.group, w.out_dtype, w.round_pow2, w.scale_fmt)), 1, w.algorithmic_bytes(1)
    if op == "cast_f32":
        def run(xs):
            xf = (xs.astype(np.uint32) << 16).view(np.float32)        # the bench's fp32 input: bf16 widened
            oracle.per_token_cast_f32(xf, w.group, w.out_dtype, w.round_pow2, w.scale_fmt)
        return run, 1, 4 * w.cols + code_cols + 4 * w.scale_cols
    if op == "dequant":
        def run(xs):
            q, s = oracle.per_token_cast(xs, w.group, w.out_dtype, w.round_pow2, w.scale_fmt)
            oracle.per_token_dequant(q, s, w.cols, w.group, w.out_dtype, w.scale_fmt, "bf16")
        # the cast that makes the codes runs inside the timed oracle step too: its bytes are counted
        return run, 1, w.algorithmic_bytes(1) + code_cols + 4 * w.scale_cols + 2 * w.cols
    if op == "cast_back":
        return (lambda xs: oracle.per_token_cast_back(xs, w.group, w.out_dtype, w.round_pow2)), 1, 4 * w.cols
    if op == "per_block":
        br, bc = block
        nbc = w.cols // bc
        sbytes = 4 * nbc if w.scale_fmt == "f32" else nbc
        return ((lambda xs: oracle.per_block_cast(xs, br, bc, w.out_dtype, w.round_pow2, w.scale_fmt)), br,
                2 * w.cols + code_cols + sbytes / br)
    if op == "per_channel":
        return ((lambda xs: oracle.per_channel_cast(xs, w.out_dtype, w.round_pow2, w.scale_fmt)), 1,
                2 * w.cols + code_cols)
    if op == "rmsnorm_cast":
        return ((lambda xs: oracle.rmsnorm_cast(xs, weight_bits, 1e-6, w.group, w.out_dtype, w.round_pow2,
                                                w.scale_fmt)), 1, w.algorithmic_bytes(1))
    if op == "rmsnorm":
        return (lambda xs: oracle.rmsnorm(xs, weight_bits, 1e-6, "bf16")), 1, 4 * w.cols
    raise ValueError(op)


def cpu_baseline(w, x_bits, threads: int, op: str = "cast", block=(128, 128), weight_bits=None,
                 min_wall_s: float = 1.0, max_passes: int = 20):
    """The operation's CPU oracle over row blocks on `threads` host threads:
    whole passes over the workload's first rows (at most 32768, rounded to the
    block height) until `min_wall_s` of wall time has elapsed, i.e. about
    threads * min_wall_s seconds of CPU work.  The per-channel oracle, whose
    column maxima span all rows, runs over column blocks instead."""
    import numpy as np
    fn, unit, bytes_per_row = _oracle_step(op, w, block, weight_bits)
    rows = x_bits.shape[0]
    sample = min(rows, 32768) // unit * unit
    xs = x_bits[:sample]
    if op == "per_channel":
        cuts = np.linspace(0, w.cols // 8, threads + 1).astype(int) * 8
        parts = [np.ascontiguousarray(xs[:, cuts[i]:cuts[i + 1]]) for i in range(threads)]
    else:
        cuts = (np.linspace(0, sample // unit, threads + 1).astype(int) * unit)
        parts = [xs[cuts[i]:cuts[i + 1]] for i in range(threads)]
    fn(parts[0][:unit] if op != "per_channel" else parts[0][:8])          # load the library
    passes = 0
    t0 = time.perf_counter()
    with concurrent.futures.ThreadPoolExecutor(threads) as ex:
        while passes < max_passes and (passes == 0 or time.perf_counter() - t0 < min_wall_s):
            list(ex.map(fn, parts))
            passes += 1
    dt = time.perf_counter() - t0
    nbytes = bytes_per_row * sample
    # one core: the first 1/threads of the sample, whole passes for >= 1 s
    one, t1, p1 = parts[0], time.perf_counter(), 0
    while p1 < max_passes and (p1 == 0 or time.perf_counter() - t1 < min_wall_s):
        fn(one)
        p1 += 1
    d1 = time.perf_counter() - t1
    one_bytes = bytes_per_row * (one.shape[0] if op != "per_channel" else sample) * \
        (1 if op != "per_channel" else one.shape[1] / w.cols)
    return {
        "value": round(passes * nbytes / dt / 1e9, 3),
        "unit": "GB/s",
        "cores": threads,
        "kind": "oracle",
        "sample": f"{passes} passes over rows 0..{sample - 1} of the workload ({sample} x {w.in_cols} bf16), "
                  f"{threads} threads over {'column' if op == 'per_channel' else 'row'} blocks, {dt:.2f} s wall",
        "tokens_per_s": round(passes * sample / dt, 1),
        "single_core": {"value": round(p1 * one_bytes / d1 / 1e9, 4), "unit": "GB/s",
                        "sample": f"{p1} passes over one thread's share, {d1:.2f} s"},
        **cpu_host(),
    }


def settle_clocks(step, stream, target_ms: float) -> dict:
    """Run `step` back to back for at least `target_ms` of GPU time (estimated
    from 3 timed launches, then measured): the MI355X memory clocks reach
    their steady state only after ~10-15 ms of sustained load, so a short
    warm-up alone leaves the first timed launches slower."""
    import math
    import torch
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record(stream)
    for _ in range(3):
        step()
    b.record(stream)
    b.synchronize()
    per_ms = max(a.elapsed_time(b) / 3, 1e-3)
    n = max(1, math.ceil(target_ms / per_ms))
    a.record(stream)
    for _ in range(n):
        step()
    b.record(stream)
    b.synchronize()
    return {"launches": n + 3, "ms": round(a.elapsed_time(b) + 3 * per_ms, 2), "target_ms": target_ms}


def cpu_host() -> dict:
    """What the host's /proc/cpuinfo says of its processor, and its core counts."""
    fields = {}
    try:
        for line in open("/proc/cpuinfo"):
            if ":" not in line:
                if fields:
                    break                       # the first processor's block is enough
                continue
            k, v = (t.strip() for t in line.split(":", 1))
            if k in ("model name", "cpu family", "model", "stepping") and k not in fields:
                fields[k] = v
    except OSError:
        pass
    name = fields.get("model name", "")
    ids = ", ".join(f"{k} {fields[k]}" for k in ("cpu family", "model", "stepping") if k in fields)
    return {"cpu_model": f"{name} ({ids})" if ids else name,
            "host_cores_affinity": len(os.sched_getaffinity(0)), "host_cpu_count": os.cpu_count()}


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=1000)
    ap.add_argument("--warmup", type=int, default=300, help="untimed steps before the timed ones")
    ap.add_argument("--settle-ms", type=float, default=30.0,
                    help="back-to-back launches of the same call, at least this long in GPU time, before "
                         "the warm-up: the memory clocks need ~10-15 ms of sustained load to settle")
    ap.add_argument("--workload", type=int, default=4)
    ap.add_argument("--op", choices=["cast", "cast_f32", "dequant", "cast_back", "per_block", "per_channel", "rmsnorm",
                                     "rmsnorm_cast"], default="cast",
                    help="cast (the workload's cast, fused SwiGLU for workload 3), the same cast of the "
                         "input widened to fp32, its dequantization, "
                         "the fused cast-and-cast-back, the per-block / per-channel cast of the "
                         "workload's input with its code and scale formats, RMSNorm forward (bf16 out) "
                         "or RMSNorm fused with the workload's per-token cast")
    ap.add_argument("--block", default="128x128", help="block rows x block columns for --op per_block")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--sets", type=int, default=0,
                    help="distinct input/output sets rotated over (default: at least 3, and enough that the sets "
                         "hold twice the 256 MB Infinity Cache)")
    ap.add_argument("--flushed", type=int, default=50,
                    help="extra launches timed one by one, each after a 512 MiB copy that flushes the caches")
    ap.add_argument("--vendor-copy", action="store_true",
                    help="also time the runtime's device-to-device copy and the library's streaming copy of "
                         "half the step's bytes each way")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="also run 3 device-to-device copies of 1 GiB (counter calibration)")
    ap.add_argument("--summarize-pmc", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="turn two rocprofv3 --pmc runs (FETCH_SIZE, WRITE_SIZE) into profiles/traffic.json")
    ap.add_argument("--summarize-ea", nargs=2, metavar=("READ_CSV", "WRITE_CSV"),
                    help="per-kernel TCC/EA request counts and bytes from two rocprofv3 --pmc runs")
    args = ap.parse_args()

    if args.summarize_pmc:
        summarize_pmc(args.workload, *args.summarize_pmc)
        return
    if args.summarize_ea:
        summarize_ea(*args.summarize_ea)
        return

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: the cast is row-parallel with no exchange between GPUs, "
              "and this benchmark runs on a single GPU only (--gpus 1).", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch
    import activation_quantization_token_amd as tk
    from activation_quantization_token_amd import inputs, rawcall

    w = inputs.WORKLOADS[args.workload]
    log(f"[bench] workload {w.index}: {w.name}; generating inputs")
    x_bits = inputs.generate(w, cache=True)
    dev = torch.device("cuda:0")
    x0 = torch.from_numpy(x_bits.view(np.int16)).view(torch.bfloat16).to(dev)
    # Rotate over distinct input/output sets so that no step can be served
    # from the 256 MB Infinity Cache with data an earlier step touched: the
    # sets together hold at least twice the cache (with three sets of a
    # ~89 MB workload, 267 MB, some of the oldest set's data was still cached:
    # 3 % faster than with eight).
    n_sets = args.sets if args.sets > 0 else max(3, -(-(2 * MALL_BYTES) // w.algorithmic_bytes()))
    sets = []
    for i in range(n_sets):
        xi = x0 if i == 0 else x0.clone()
        sets.append((xi, *tk.empty_outputs(w.rows, w.cols, w.group, w.out_dtype, w.scale_fmt, dev)))
    if args.op != "cast" and w.swiglu:
        raise SystemExit("dequant / cast_back benchmarks take a plain cast workload (not 3)")
    if args.op == "cast":
        fn = tk.swiglu_per_token_cast if w.swiglu else tk.per_token_cast
        if w.swiglu:
            tk.tk_prepare_device()

        def run(xi, qi, si, yi):
            fn(xi, w.group, w.out_dtype, w.round_pow2, w.scale_fmt, out=(qi, si))
        nbytes = w.algorithmic_bytes()
        read_bytes = w.rows * w.in_cols * 2
    elif args.op == "cast_f32":
        # the workload's input widened to fp32 (exact), cast with the fp32-input kernel
        sets = [(xi.float(), qi, si) for (xi, qi, si) in sets]

        def run(xi, qi, si, yi):
            tk.per_token_cast(xi, w.group, w.out_dtype, w.round_pow2, w.scale_fmt, out=(qi, si))
        nbytes = w.rows * (4 * w.cols + w.code_cols + 4 * w.scale_cols)
        read_bytes = w.rows * 4 * w.cols
    elif args.op == "dequant":
        # inputs: the workload's codes and scales (made by the cast); output bf16
        for i in range(len(sets)):
            tk.per_token_cast(sets[i][0], w.group, w.out_dtype, w.round_pow2, w.scale_fmt,
                              out=(sets[i][1], sets[i][2]))

        def run(xi, qi, si, yi):
            tk.per_token_dequant(qi, si, w.cols, w.group, w.out_dtype, w.scale_fmt, "bf16", out=yi)
        nbytes = w.rows * (w.code_cols + 4 * w.scale_cols + 2 * w.cols)
        read_bytes = w.rows * (w.code_cols + 4 * w.scale_cols)
    elif args.op == "cast_back":
        def run(xi, qi, si, yi):
            tk.per_token_cast_back(xi, w.group, w.out_dtype, w.round_pow2, out=yi)
        nbytes = w.rows * 4 * w.cols
        read_bytes = w.rows * 2 * w.cols
    elif args.op == "per_block":
        br, bc = (int(v) for v in args.block.split("x"))
        sets = [(xi, *tk.per_block_cast(xi, br, bc, w.out_dtype, w.round_pow2, w.scale_fmt)) for (xi, _, _) in sets]

        def run(xi, qi, si, yi):
            tk.per_block_cast(xi, br, bc, w.out_dtype, w.round_pow2, w.scale_fmt, out=(qi, si))
        s0 = sets[0][2]
        nbytes = w.rows * (2 * w.cols + w.code_cols) + s0.numel() * s0.element_size()
        read_bytes = w.rows * 2 * w.cols
    elif args.op == "rmsnorm":
        wt = (torch.randn(w.cols, generator=torch.Generator().manual_seed(5)) * 0.1 + 1).bfloat16().to(dev)

        def run(xi, qi, si, yi):
            tk.rmsnorm(xi, wt, 1e-6, "bf16", out=yi)
        nbytes = w.rows * 4 * w.cols
        read_bytes = w.rows * 2 * w.cols
    elif args.op == "rmsnorm_cast":
        wt = (torch.randn(w.cols, generator=torch.Generator().manual_seed(5)) * 0.1 + 1).bfloat16().to(dev)

        def run(xi, qi, si, yi):
            tk.rmsnorm_cast(xi, wt, 1e-6, w.group, w.out_dtype, w.round_pow2, w.scale_fmt, out=(qi, si))
        nbytes = w.algorithmic_bytes()
        read_bytes = w.rows * 2 * w.cols
    else:
        ws = torch.empty((tk.tk_per_channel_workspace_bytes(w.rows, w.cols),), dtype=torch.uint8, device=dev)
        sets = [(xi, *tk.per_channel_cast(xi, w.out_dtype, w.round_pow2, w.scale_fmt, workspace=ws))
                for (xi, _, _) in sets]

        def run(xi, qi, si, yi):
            tk.per_channel_cast(xi, w.out_dtype, w.round_pow2, w.scale_fmt, out=(qi, si), workspace=ws)
        s0 = sets[0][2]
        nbytes = w.rows * (2 * w.cols + w.code_cols) + s0.numel() * s0.element_size()
        read_bytes = w.rows * 2 * w.cols
    if args.op in ("dequant", "cast_back", "rmsnorm"):
        sets = [(xi, qi, si, torch.empty((w.rows, w.cols), dtype=torch.bfloat16, device=dev))
                for (xi, qi, si) in sets]
    else:
        sets = [(xi, qi, si, None) for (xi, qi, si) in sets]

    # The timed loops call the C ABI directly, with each buffer set's
    # arguments marshalled once: the tensor functions' checks cost about 8 us
    # of host time per call, more than the GPU needs for a 128-row cast.
    # Each raw call is checked first against the tensor function's output.
    lib = tk.load_library()
    sh = torch.cuda.current_stream(dev).cuda_stream
    qd, sf, p2 = {"e4m3": 0, "e2m1": 1}[w.out_dtype], {"f32": 0, "ue8m0": 1}[w.scale_fmt], int(w.round_pow2)

    def raw_call(xi, qi, si, yi):
        """(entry point, arguments, {pointer parameter: owning tensor}) of the step's call."""
        r, c = w.rows, w.cols
        if args.op in ("cast", "cast_f32"):
            name = ("tk_swiglu_per_token_cast" if w.swiglu else
                    "tk_per_token_cast_f32" if args.op == "cast_f32" else "tk_per_token_cast")
            return name, (xi.data_ptr(), r, c, xi.stride(0), qi.data_ptr(), qi.stride(0), si.data_ptr(),
                          si.stride(0), w.group, qd, p2, sf, sh), {"gate_up" if w.swiglu else "x": xi, "q": qi,
                                                                   "scales": si}
        if args.op == "dequant":
            return "tk_per_token_dequant", (qi.data_ptr(), r, c, qi.stride(0), si.data_ptr(), si.stride(0), w.group,
                                            qd, sf, yi.data_ptr(), yi.stride(0), 0, sh), {"q": qi, "scales": si,
                                                                                           "y": yi}
        if args.op == "cast_back":
            return "tk_per_token_cast_back", (xi.data_ptr(), r, c, xi.stride(0), yi.data_ptr(), yi.stride(0),
                                              w.group, qd, p2, sh), {"x": xi, "y": yi}
        if args.op == "per_block":
            return "tk_per_block_cast", (xi.data_ptr(), r, c, xi.stride(0), qi.data_ptr(), qi.stride(0),
                                         si.data_ptr(), si.stride(0), br, bc, qd, p2, sf, sh), {"x": xi, "q": qi,
                                                                                                "scales": si}
        if args.op == "rmsnorm":
            return "tk_rmsnorm", (xi.data_ptr(), r, c, xi.stride(0), wt.data_ptr(), 1e-6, yi.data_ptr(),
                                  yi.stride(0), 0, sh), {"x": xi, "weight": wt, "y": yi}
        if args.op == "rmsnorm_cast":
            return "tk_rmsnorm_cast", (xi.data_ptr(), r, c, xi.stride(0), wt.data_ptr(), 1e-6, qi.data_ptr(),
                                       qi.stride(0), si.data_ptr(), si.stride(0), w.group, qd, p2, sf, sh), \
                {"x": xi, "weight": wt, "q": qi, "scales": si}
        return "tk_per_channel_cast", (xi.data_ptr(), r, c, xi.stride(0), qi.data_ptr(), qi.stride(0), si.data_ptr(),
                                       ws.data_ptr(), ws.numel(), qd, p2, sf, sh), {"x": xi, "q": qi, "scales": si,
                                                                                    "workspace": ws}

    out_idx = (3,) if args.op in ("dequant", "cast_back", "rmsnorm") else (1, 2)
    calls = []
    for st in sets:
        run(*st)
        torch.cuda.synchronize()
        want = [st[i].clone() for i in out_idx]
        for i in out_idx:
            st[i].view(torch.uint8).fill_(0xA5)
        # every pointer's extent, from the call's own arguments, inside its tensor
        cfn, a = rawcall.prepare(lib, *raw_call(*st))
        if cfn(*a) != 0:
            raise SystemExit(f"raw {args.op} call failed")
        torch.cuda.synchronize()
        assert all(torch.equal(st[i].view(torch.uint8), v.view(torch.uint8)) for i, v in zip(out_idx, want)), \
            "raw call disagrees with the tensor function"
        calls.append((cfn, a))
    counter = [0]

    def step():
        cfn, a = calls[counter[0] % len(calls)]
        if cfn(*a) != 0:
            raise SystemExit(f"{args.op} launch failed")
        counter[0] += 1

    stream = torch.cuda.current_stream(dev)
    settle = settle_clocks(step, stream, args.settle_ms)
    log(f"[bench] clock settle: {settle['launches']} launches, {settle['ms']} ms")
    log(f"[bench] warmup {args.warmup} steps")
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    # Timed region: K back-to-back launches on the current stream between two
    # events; the per-launch kernel time is the span over K.
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    log(f"[bench] timing {args.steps} steps over {len(sets)} buffer sets")
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    start.record(stream)
    for _ in range(args.steps):
        step()
    end.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    span_ms = start.elapsed_time(end)

    # consistency check: every set holds the same inputs, so the last step's
    # outputs equal the first set's after re-running it
    if len(sets) > 1:
        last = sets[(counter[0] - 1) % len(sets)]
        run(*sets[0])
        torch.cuda.synchronize()
        assert all(torch.equal(last[i].view(torch.uint8), sets[0][i].view(torch.uint8)) for i in out_idx)

    # Per-launch durations with the 256 MB Infinity Cache flushed before each
    # launch (a 512 MiB streaming copy in between), event-timed one by one.
    flush_src = torch.empty(256 << 20, dtype=torch.uint8, device=dev)
    flush_dst = torch.empty_like(flush_src)
    per_launch = []
    for i in range(args.flushed):
        tk.copy_stream(flush_src, flush_dst)
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        cfn, cargs = calls[i % len(calls)]
        if cfn(*cargs) != 0:
            raise SystemExit(f"{args.op} launch failed")
        b.record(stream)
        b.synchronize()
        per_launch.append(a.elapsed_time(b) * 1e3)
    del flush_src, flush_dst
    flushed = None
    if per_launch:
        pl = np.sort(np.array(per_launch))
        med = float(np.median(pl))
        flushed = {"launches": len(pl), "median_us": round(med, 3), "p10_us": round(float(np.percentile(pl, 10)), 3),
                   "p90_us": round(float(np.percentile(pl, 90)), 3), "median_gbs": round(nbytes / med / 1e3, 2)}

    # Practical streaming ceiling for the same read and write volumes: the
    # library's stream diagnostic, timed exactly like the operation.
    rd, wr = read_bytes - read_bytes % 16, (nbytes - read_bytes) - (nbytes - read_bytes) % 16
    csrc = [torch.empty(rd, dtype=torch.uint8, device=dev) for _ in range(len(sets))]
    cdst = [torch.empty(wr, dtype=torch.uint8, device=dev) for _ in range(len(sets))]
    tk.stream_rw(csrc[0], rd, cdst[0], wr)          # argument checks, once
    rw_args = [rawcall.prepare(lib, "tk_stream_rw", (csrc[i].data_ptr(), rd, cdst[i].data_ptr(), wr, sh),
                               {"src": csrc[i], "dst": cdst[i]})[1] for i in range(len(sets))]
    rw_count = [0]

    def rw_step():
        lib.tk_stream_rw(*rw_args[rw_count[0] % len(sets)])
        rw_count[0] += 1
    settle_clocks(rw_step, stream, args.settle_ms)
    for i in range(args.warmup):
        rw_step()
    torch.cuda.synchronize()
    c0, c1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    c0.record(stream)
    for i in range(args.steps):
        lib.tk_stream_rw(*rw_args[i % len(sets)])
    c1.record(stream)
    torch.cuda.synchronize()
    ceil_us = c0.elapsed_time(c1) * 1e3 / args.steps
    del csrc, cdst

    # The runtime's own device-to-device copy (hipMemcpyAsync through
    # torch's copy_) against the library's streaming copy, each moving half
    # the step's bytes each way, settled and timed like the operation: a check
    # that the library's streams are no slower than the vendor's.
    vendor = None
    if args.vendor_copy:
        half = (nbytes // 2) - (nbytes // 2) % 16
        vsrc = [torch.ones(half, dtype=torch.uint8, device=dev) for _ in range(len(sets))]
        vdst = [torch.empty(half, dtype=torch.uint8, device=dev) for _ in range(len(sets))]
        cp_args = [rawcall.prepare(lib, "tk_copy_stream", (vsrc[i].data_ptr(), vdst[i].data_ptr(), half, sh),
                                   {"src": vsrc[i], "dst": vdst[i]})[1] for i in range(len(sets))]

        def timed(step_i):
            count = [0]

            def step():
                step_i(count[0] % len(sets))
                count[0] += 1
            settle_clocks(step, stream, args.settle_ms)
            for _ in range(args.warmup):
                step()
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            for _ in range(args.steps):
                step()
            e1.record(stream)
            torch.cuda.synchronize()
            return e0.elapsed_time(e1) * 1e3 / args.steps
        hip_us = timed(lambda i: vdst[i].copy_(vsrc[i]))
        own_us = timed(lambda i: lib.tk_copy_stream(*cp_args[i]))
        if not torch.equal(vdst[0], vsrc[0]):
            raise SystemExit("copy check failed")
        vendor = {"bytes_each_way": half, "hip_memcpy_us": round(hip_us, 3), "tk_copy_stream_us": round(own_us, 3),
                  "hip_memcpy_gbs": round(2 * half / hip_us / 1e3, 2),
                  "tk_copy_stream_gbs": round(2 * half / own_us / 1e3, 2)}
        del vsrc, vdst

    ms_per_step = span_ms / args.steps
    value = nbytes * args.steps / (span_ms / 1e3) / 1e9
    avg_launch_ms = ms_per_step
    achieved = nbytes / (avg_launch_ms / 1e3) / 1e9
    traffic = measured_traffic(w.index) if args.op == "cast" else None

    metric = "per-token cast GB/s (in+out bytes) and % of MI355X HBM peak; tokens/s"
    if args.op != "cast":
        metric = f"{args.op} GB/s (algorithmic in+out bytes) and % of MI355X HBM peak"
    out = {
        "metric": metric,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",                 # the arithmetic: amax, scale and x / s in fp32
        "settle": settle,
        "data": "synthetic",
        "config": {
            "workload": w.name, "rows": w.rows, "cols": w.cols, "group": w.group,
            "out_dtype": w.out_dtype, "round_pow2": w.round_pow2, "scale_fmt": w.scale_fmt,
            "swiglu": w.swiglu, "seed": w.seed, "bytes_per_step": nbytes, "op": args.op,
            "input_dtype": "f32" if args.op == "cast_f32" else "bf16",
            "code_format": "bf16" if args.op in ("cast_back", "rmsnorm") else w.out_dtype,
            **({"block": args.block} if args.op == "per_block" else {}),
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
            "algorithmic_bytes_per_launch": nbytes,
            "buffer_sets": len(sets),
        },
        "ceiling": {
            "kernel": "tk_stream_rw (the same read and write bytes, the cast's memory instructions)",
            "read_bytes": rd, "write_bytes": wr, "us": round(ceil_us, 3),
            "gbs": round(nbytes / ceil_us / 1e3, 2), "frac_of_peak": round(nbytes / ceil_us / 1e3 / HBM_PEAK_GBS, 4),
            "op_frac_of_ceiling": round(ceil_us / ms_per_step / 1e3, 4),
        },
        "flushed": flushed,
        **({"vendor_copy": vendor} if vendor is not None else {}),
    }
    if args.calibrate_copy:
        src = torch.ones(1 << 30, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            tk.copy_stream(src, dst)
        torch.cuda.synchronize()
    if not args.no_cpu_baseline:
        # at most 16 threads: a one-GPU machine's share of the host, whatever the
        # affinity mask shows (both counts are reported)
        threads = min(16, len(os.sched_getaffinity(0)))
        log(f"[bench] CPU baseline: oracle on {threads} threads")
        weight_bits = None
        if args.op in ("rmsnorm", "rmsnorm_cast"):
            weight_bits = wt.cpu().view(torch.int16).numpy().view(np.uint16)
        block = tuple(int(v) for v in args.block.split("x"))
        out["cpu_baseline"] = cpu_baseline(w, x_bits, threads, args.op, block, weight_bits)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
