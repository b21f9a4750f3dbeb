"""bench.py's command line on the CPU: it measures one GPU and refuses more."""
from __future__ import annotations

import csv
import os
import pathlib
import subprocess
import sys

ROOT = pathlib.Path(__file__).resolve().parent.parent


def test_more_than_one_gpu_is_refused():
    env = dict(os.environ, WORLD_SIZE="1")
    r = subprocess.run([sys.executable, str(ROOT / "bench.py"), "--gpus", "2", "--no-cpu-baseline"],
                       capture_output=True, text=True, env=env, timeout=120)
    assert r.returncode == 2
    assert "single GPU" in r.stderr and r.stdout == ""


def test_world_size_above_one_is_refused():
    env = dict(os.environ, WORLD_SIZE="4")
    r = subprocess.run([sys.executable, str(ROOT / "bench.py")], capture_output=True, text=True, env=env,
                       timeout=120)
    assert r.returncode == 2 and "single GPU" in r.stderr


def _pmc_csv(path, counter, rows):
    """A rocprofv3 --pmc counter CSV with the columns bench.py reads."""
    import csv
    with open(path, "w", newline="") as f:
        wr = csv.writer(f)
        wr.writerow(["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"])
        for dispatch, kernel, value in rows:
            wr.writerow([dispatch, kernel, counter, value])


def test_counter_summary_scales_by_the_calibration_copy(tmp_path):
    """HBM bytes = FETCH_SIZE and WRITE_SIZE of the cast (median over its
    dispatches, summed over a dispatch's rows) scaled by what the same
    counters read for the 1 GiB calibration copy."""
    sys.path.insert(0, str(ROOT))
    import bench
    from activation_quantization_token_amd import inputs
    copy = "(anonymous namespace)::copy_stream_kernel(...)"
    cast = "void (anonymous namespace)::cast_rows_kernel<32, 1, true, 1, 2>(...)"
    gib_kib = float(1 << 20)
    # the copy's reads counted at half their size, its writes in full; the
    # cast's counters split over two rows per dispatch (e.g. two channels)
    _pmc_csv(tmp_path / "f.csv", "FETCH_SIZE",
             [(1, copy, gib_kib / 2), (2, cast, 100.0), (2, cast, 50.0), (3, cast, 160.0), (4, cast, 149.0)])
    _pmc_csv(tmp_path / "w.csv", "WRITE_SIZE",
             [(1, copy, gib_kib), (2, cast, 30.0), (3, cast, 20.0), (3, cast, 12.0), (4, cast, 40.0)])
    entry = bench.summarize_pmc(4, tmp_path / "f.csv", tmp_path / "w.csv", traffic_file=tmp_path / "t.json")
    assert entry["copy_fetch_scale"] == 2.0 and entry["copy_write_scale"] == 1.0
    assert entry["fetch_size_kib"] == 150.0 and entry["write_size_kib"] == 32.0     # medians of 150/160/149, 30/32/40
    assert entry["hbm_bytes_per_launch"] == (2 * 150 + 32) * 1024
    assert entry["algorithmic_bytes_per_launch"] == inputs.WORKLOADS[4].algorithmic_bytes() == 594542592
    assert entry["kernel_source_sha256_16"] == bench.kernel_source_hash()
    import json
    assert json.loads((tmp_path / "t.json").read_text())["workload4"] == entry


def test_ea_request_summary(tmp_path):
    """Read bytes = 32 per 32-byte request + 128 per other request, write bytes
    = 64 per 64-byte request + 32 per other; medians over dispatches, a
    dispatch's rows summed."""
    sys.path.insert(0, str(ROOT))
    import bench
    copy = "(anonymous namespace)::copy_stream_kernel(...)"
    cast = "void (anonymous namespace)::cast_rows_kernel<32, 1, true, 1, 2>(...)"
    rd, wr = tmp_path / "rd.csv", tmp_path / "wr.csv"
    with open(rd, "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"])
        for d, k, c, v in [(1, copy, "TCC_EA0_RDREQ_sum", 1 << 23), (1, copy, "TCC_EA0_RDREQ_32B_sum", 0),
                           (2, cast, "TCC_EA0_RDREQ_sum", 60), (2, cast, "TCC_EA0_RDREQ_sum", 40),
                           (2, cast, "TCC_EA0_RDREQ_32B_sum", 10), (3, cast, "TCC_EA0_RDREQ_sum", 100),
                           (3, cast, "TCC_EA0_RDREQ_32B_sum", 10), (4, cast, "TCC_EA0_RDREQ_sum", 300),
                           (4, cast, "TCC_EA0_RDREQ_32B_sum", 10)]:
            w.writerow([d, k, c, v])
    with open(wr, "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"])
        for d, k, c, v in [(1, copy, "TCC_EA0_WRREQ_sum", 1 << 24), (1, copy, "TCC_EA0_WRREQ_64B_sum", 1 << 24),
                           (2, cast, "TCC_EA0_WRREQ_sum", 50), (2, cast, "TCC_EA0_WRREQ_64B_sum", 40)]:
            w.writerow([d, k, c, v])
    out = bench.summarize_ea(rd, wr)
    assert out[copy]["read_bytes"] == 1 << 30 and out[copy]["write_bytes"] == 1 << 30
    assert out[cast]["TCC_EA0_RDREQ_sum"] == 100                         # median of 100, 100, 300
    assert out[cast]["read_bytes"] == 32 * 10 + 128 * 90
    assert out[cast]["write_bytes"] == 64 * 40 + 32 * 10
