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
SOURCES = [PKG / "csrc" / "tk_quant.hip", PKG / "csrc" / "tk_block.hip", PKG / "csrc" / "tk_norm.hip",
           PKG / "csrc" / "tk_diag.hip"]
INCLUDE = ROOT / "include"
LIB = PKG / "libtk_quant.so"
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    "-Wall", "-Wextra", "-Werror",
    # no packed fp32 instructions (v_pk_*_f32) in any kernel
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


def _clean(stderr: str) -> str:
    # hipcc's host pass reports the device-only feature flag as unknown
    noise = "'-packed-fp32-ops' is not a recognized feature for this target (ignoring feature)"
    return "\n".join(l for l in stderr.splitlines() if noise not in l)


def build(verbose: bool = False) -> pathlib.Path:
    """Compile every source to an object (in parallel), then link the library."""
    tag = "tmp%d" % os.getpid()
    objs = [LIB.parent / f"{src.stem}.{tag}.o" for src in SOURCES]
    cmds = [[HIPCC, *FLAGS, f"-I{INCLUDE}", "-c", str(src), "-o", str(obj)] for src, obj in zip(SOURCES, objs)]
    tmp = LIB.with_suffix(".so." + tag)
    try:
        procs = []
        for cmd in cmds:
            if verbose:
                print(" ".join(cmd), flush=True)
            procs.append(subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.PIPE, text=True))
        for proc in procs:
            _, err = proc.communicate()
            err = _clean(err)
            if proc.returncode != 0:
                raise RuntimeError(f"hipcc failed ({proc.returncode}):\n{err}")
            if err.strip() and verbose:
                print(err, file=sys.stderr)
        link = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *map(str, objs), "-o", str(tmp)]
        res = subprocess.run(link, capture_output=True, text=True)
        if res.returncode != 0:
            raise RuntimeError(f"link failed ({res.returncode}):\n{_clean(res.stderr)}")
        os.replace(tmp, LIB)
    finally:
        for f in [*objs, tmp]:
            if f.exists():
                f.unlink()
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
