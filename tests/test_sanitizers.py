"""The CPU oracle and the library's host-side argument checks under
AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

Each part is rebuilt with both sanitizers, aborting on the first report, and
an existing CPU suite is run against that build in a child process with the
sanitizer runtime preloaded:
  * the oracle (gcc -fsanitize=address,undefined) under every oracle pin;
  * the HIP library with sanitized host code (hipcc, sanitizer flags on the
    host pass only) under the ABI tests, which drive every entry point's
    argument checks with fake device pointers and never reach a kernel.
"""
from __future__ import annotations

import glob
import os
import pathlib
import subprocess
import sys

import pytest

ROOT = pathlib.Path(__file__).resolve().parent.parent
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
SAN_ENV = {"ASAN_OPTIONS": "detect_leaks=0:halt_on_error=1:abort_on_error=0:exitcode=66",
           "UBSAN_OPTIONS": "halt_on_error=1:print_stacktrace=1"}
PINS = ["tests/test_oracle_pins.py", "tests/test_oracle_block_pins.py", "tests/test_oracle_rmsnorm_pins.py",
        "tests/test_oracle_dequant_pins.py"]


def _run_suite(files, env_extra, timeout):
    env = dict(os.environ, **SAN_ENV, **env_extra)
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider", "-m", "not gpu", *files],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=timeout)
    report = r.stdout[-4000:] + r.stderr[-4000:]
    assert r.returncode == 0, report
    assert "AddressSanitizer" not in r.stderr and "runtime error:" not in r.stderr, report
    assert " passed" in r.stdout, report
    return r


def test_oracle_pins_under_asan_ubsan(tmp_path):
    lib = tmp_path / "libtk_oracle_san.so"
    subprocess.check_call(["gcc", "-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
                           "-fno-sanitize-recover=all", "-ffp-contract=off", "-fno-fast-math", "-std=c11", "-fPIC",
                           "-shared", "-Wall", "-Wextra", "-Werror", "-o", str(lib), str(ROOT / "oracle" / "tk_oracle.c"),
                           "-lm"])
    asan = subprocess.run(["gcc", "-print-file-name=libasan.so"], capture_output=True, text=True).stdout.strip()
    assert os.path.isabs(asan), "gcc has no AddressSanitizer runtime"
    _run_suite(PINS, {"LD_PRELOAD": asan, "TK_ORACLE_LIBRARY": str(lib)}, timeout=900)


def test_abi_checks_under_asan_ubsan(tmp_path):
    runtimes = glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so")
    if not runtimes:
        pytest.skip("no clang AddressSanitizer runtime under /opt/rocm/llvm")
    srcs = ["tk_quant", "tk_block", "tk_norm", "tk_diag"]
    objs = [tmp_path / f"{s}.o" for s in srcs]
    # the sanitizers apply to the host pass only (-Xarch_host before each flag)
    host_san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                "-Xarch_host", "-fno-sanitize-recover=all"]
    procs = [subprocess.Popen([HIPCC, "--offload-arch=gfx950", "-O1", "-g", "-std=c++17", "-fPIC",
                               "-fno-omit-frame-pointer", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
                               *host_san, f"-I{ROOT / 'include'}", "-c",
                               str(ROOT / "activation_quantization_token_amd" / "csrc" / f"{s}.hip"), "-o", str(o)],
                              stdout=subprocess.PIPE, stderr=subprocess.PIPE, text=True)
             for s, o in zip(srcs, objs)]
    for p in procs:
        _, err = p.communicate(timeout=600)
        assert p.returncode == 0, err[-3000:]
    lib = tmp_path / "libtk_quant_san.so"
    subprocess.check_call([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-Xarch_host", "-fsanitize=address",
                           "-Xarch_host", "-fsanitize=undefined", *map(str, objs), "-o", str(lib)])
    _run_suite(["tests/test_abi.py"], {"LD_PRELOAD": sorted(runtimes)[-1], "TK_QUANT_LIBRARY": str(lib)},
               timeout=600)


@pytest.mark.parametrize("body,arg,report", [
    # use after free: AddressSanitizer (exit code 66 from ASAN_OPTIONS)
    ("char *p = malloc(8); p[0] = 1; free(p); return p[n & 7];", 3, "heap-use-after-free"),
    # signed overflow: UndefinedBehaviorSanitizer
    ("int big = 0x7FFFFFF0; return big + n;", 100, "signed integer overflow"),
])
def test_the_setup_reports_planted_mistakes(tmp_path, body, arg, report):
    """The same flags, runtime preload and options turn a planted mistake in
    a loaded library into a failing child process that names it."""
    src = tmp_path / "planted.c"
    src.write_text("#include <stdlib.h>\nint poke(int n) { " + body + " }\n")
    lib = tmp_path / "libplanted.so"
    subprocess.check_call(["gcc", "-O0", "-g", "-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fPIC",
                           "-shared", "-o", str(lib), str(src)])
    asan = subprocess.run(["gcc", "-print-file-name=libasan.so"], capture_output=True, text=True).stdout.strip()
    code = f"import ctypes; ctypes.CDLL({str(lib)!r}).poke({arg})"
    r = subprocess.run([sys.executable, "-c", code], env=dict(os.environ, **SAN_ENV, LD_PRELOAD=asan),
                       capture_output=True, text=True, timeout=120)
    assert r.returncode != 0 and report in r.stderr, r.stderr[-2000:]
