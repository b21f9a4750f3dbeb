"""Checks on the machine code of the built library (gfx950 code objects taken
from its offload bundles; llvm-objdump and llvm-readelf from ROCm).

- No 12- or 16-byte buffer store takes a register in its scalar-offset field:
  for such stores the compiler inserts no wait state before a VALU write of
  the stored registers, and on gfx950 a write right after the store was seen
  to change the stored data.  The kernels give these stores a zero scalar
  offset, which the compiler's hazard handling covers.
- No kernel spills registers or uses private (scratch) memory.
- The one-wave-per-row RMSNorm kernels fit 4 waves per SIMD (<= 128 VGPRs),
  which their launch assumes.
"""
from __future__ import annotations

import pathlib
import re
import struct
import subprocess
import tempfile

import pytest
import yaml

ROOT = pathlib.Path(__file__).resolve().parent.parent
LIB = ROOT / "activation_quantization_token_amd" / "libtk_quant.so"
LLVM = pathlib.Path("/opt/rocm/llvm/bin")
MAGIC = b"__CLANG_OFFLOAD_BUNDLE__"

pytestmark = pytest.mark.skipif(not LIB.exists() or not (LLVM / "llvm-objdump").exists(),
                                reason="library or ROCm LLVM tools missing")


def _code_objects() -> list[bytes]:
    """gfx950 code objects of every offload bundle in the library's .hip_fatbin."""
    with tempfile.TemporaryDirectory() as d:
        fb = pathlib.Path(d) / "fatbin"
        subprocess.run([str(LLVM / "llvm-objcopy"), "--dump-section", f".hip_fatbin={fb}", str(LIB),
                        str(pathlib.Path(d) / "copy.so")], check=True, capture_output=True)
        data = fb.read_bytes()
    out, pos = [], 0
    while (i := data.find(MAGIC, pos)) >= 0:
        n, = struct.unpack_from("<Q", data, i + len(MAGIC))
        p = i + len(MAGIC) + 8
        for _ in range(n):
            off, size, tl = struct.unpack_from("<QQQ", data, p)
            p += 24
            triple = data[p:p + tl].decode()
            p += tl
            if triple.endswith("gfx950"):
                out.append(data[i + off:i + off + size])
        pos = i + 1
    return out


@pytest.fixture(scope="module")
def objects(tmp_path_factory):
    d = tmp_path_factory.mktemp("co")
    paths = []
    for k, co in enumerate(_code_objects()):
        path = d / f"module{k}.o"
        path.write_bytes(co)
        paths.append(path)
    assert len(paths) == 4, "one code object per HIP source expected"
    return paths


def test_no_wide_buffer_store_takes_a_register_soffset(objects):
    pat = re.compile(r"buffer_store_dword(?:x3|x4)\s[^\n]*,\s*s\d+\s+(?:offen|idxen)")
    for path in objects:
        asm = subprocess.run([str(LLVM / "llvm-objdump"), "-d", str(path)], check=True, capture_output=True,
                             text=True).stdout
        assert "buffer_store" in asm, "disassembly looks empty"
        bad = pat.findall(asm)
        assert not bad, f"{path.name}: {len(bad)} wide stores with a register scalar offset, e.g. {bad[0]}"


def _kernels(path):
    notes = subprocess.run([str(LLVM / "llvm-readelf"), "--notes", str(path)], check=True, capture_output=True,
                           text=True).stdout
    doc = notes[notes.index("---"):]
    doc = doc[:doc.index("\n...") if "\n..." in doc else len(doc)]
    return yaml.safe_load(doc)["amdhsa.kernels"]


def test_no_kernel_spills_or_uses_scratch(objects):
    n = 0
    for path in objects:
        for k in _kernels(path):
            n += 1
            assert k[".private_segment_fixed_size"] == 0, k[".name"]
            assert k[".vgpr_spill_count"] == 0 and k[".sgpr_spill_count"] == 0, k[".name"]
    assert n > 300


def test_wave_rmsnorm_kernels_fit_four_waves_per_simd(objects):
    wave = [k for path in objects for k in _kernels(path) if "rmsnorm_wave_kernel" in k[".name"]]
    assert wave
    for k in wave:
        assert k[".vgpr_count"] <= 128, (k[".name"], k[".vgpr_count"])
