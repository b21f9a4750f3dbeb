"""Build the gfx950 HIP library libtk_quant.so in place (hipcc, no JIT cache).

Run as ``python -m activation_quantization_token_amd.build``.  The library is
written next to this file, so it travels with the source tree.
"""
from __future__ import annotations

import os
import pathlib
import subprocess
import sys

PKG = pathlib.Path(__file__).resolve().parent
ROOT = PKG.parent
SRC = PKG / "csrc" / "tk_quant.hip"
INCLUDE = ROOT / "include"
LIB = PKG / "libtk_quant.so"
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
    "-Wall", "-Wextra", "-Werror",
    # no packed fp32 instructions (v_pk_*_f32) in any kernel
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


def build(verbose: bool = False) -> pathlib.Path:
    tmp = LIB.with_suffix(".so.tmp%d" % os.getpid())
    cmd = [HIPCC, *FLAGS, f"-I{INCLUDE}", str(SRC), "-o", str(tmp)]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    # hipcc's host pass reports the device-only feature flag as unknown
    noise = "'-packed-fp32-ops' is not a recognized feature for this target (ignoring feature)"
    err = "\n".join(l for l in res.stderr.splitlines() if noise not in l)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}):\n{err}")
    if err.strip() and verbose:
        print(err, file=sys.stderr)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
