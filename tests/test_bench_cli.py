"""bench.py's command line on the CPU: it measures one GPU and refuses more."""
from __future__ import annotations

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
