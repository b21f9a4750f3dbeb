"""Compile tests/c/c_abi_check.c (plain C against include/tk_quant.h, linked to
the HIP library and, for checking only, the CPU oracle).  Test infrastructure:
run it as ``python tests/c/build_check.py``; ``__graft_entry__.build()`` calls it."""
from __future__ import annotations

import pathlib
import subprocess

HERE = pathlib.Path(__file__).resolve().parent
ROOT = HERE.parent.parent
SRC = HERE / "c_abi_check.c"
BIN = HERE / "c_abi_check"


def build() -> pathlib.Path:
    pkg, orc = ROOT / "activation_quantization_token_amd", ROOT / "oracle"
    cmd = ["gcc", "-std=c11", "-O2", "-Wall", "-Wextra", "-Werror", f"-I{ROOT / 'include'}", "-I/opt/rocm/include",
           str(SRC), "-o", str(BIN), f"-L{pkg}", "-ltk_quant", f"-L{orc}", "-ltk_oracle", "-L/opt/rocm/lib",
           "-lamdhip64", "-Wl,-rpath,$ORIGIN/../../activation_quantization_token_amd:$ORIGIN/../../oracle:/opt/rocm/lib"]
    subprocess.check_call(cmd)
    return BIN


if __name__ == "__main__":
    print(build())
