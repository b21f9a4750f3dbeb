"""The C ABI driven from a plain C program (tests/c/c_abi_check.c): device
buffers from the HIP runtime's C API, the library's calls, and byte-for-byte
comparison with the CPU oracle inside the program."""
from __future__ import annotations

import importlib.util
import pathlib
import subprocess

import pytest

from gpu_util import log

pytestmark = pytest.mark.gpu

HERE = pathlib.Path(__file__).resolve().parent


def test_c_program_matches_oracle():
    spec = importlib.util.spec_from_file_location("c_abi_build", HERE / "c" / "build_check.py")
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    binary = mod.BIN if mod.BIN.exists() else mod.build()
    log(f"[gpu] running {binary.name}")
    res = subprocess.run([str(binary)], capture_output=True, text=True, timeout=100)
    print(res.stdout)
    assert res.returncode == 0, res.stdout + res.stderr
    assert "ALL PASSED" in res.stdout
