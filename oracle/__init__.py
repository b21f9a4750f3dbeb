"""CPU oracle for the per-token / per-group activation cast (numpy front end).

TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
benchmark's CPU-baseline leg may import this package.  The product path (the
HIP library and its binding) never imports it, and the two share no code.

The arithmetic lives in ``tk_oracle.c`` (plain scalar C, one IEEE binary32
operation per step); this module builds it with gcc, loads it with ctypes and
offers numpy-array wrappers.  The definition it follows, step by step, is
written out at the top of ``tk_oracle.c`` with its sources on the pages:
"Tile Kernels" (PyPI, v2.0.0) Features; "TileKernels" (aiwiki.ai) sections
Quantization and Version 2.0.0; "TileKernels, TileLang kernels for MoE routing
and low-precision quantization" (hysenlabs.com) section "Seven kernel
families".  Besides the per-token cast it covers the fused SwiGLU form,
dequantization, cast-and-cast-back, fp32 input, the per-block and per-channel
casts, and RMSNorm forward with the optional fused cast.
"""
from __future__ import annotations

import ctypes
import os
import pathlib
import subprocess
import threading

import numpy as np

_DIR = pathlib.Path(__file__).resolve().parent
_SRC = _DIR / "tk_oracle.c"
_LIB = _DIR / "libtk_oracle.so"

E4M3, E2M1 = 0, 1
SCALE_F32, SCALE_UE8M0_X4 = 0, 1
_QDTYPES = {"e4m3": E4M3, "e2m1": E2M1}
_SCALE_FMTS = {"f32": SCALE_F32, "ue8m0": SCALE_UE8M0_X4}

_lock = threading.Lock()
_handle = None


def compile_source(src, out) -> pathlib.Path:
    """gcc -O2 without FP contraction or fast-math: one IEEE op per C operator."""
    out = pathlib.Path(out)
    tmp = out.with_suffix(".so.tmp%d" % os.getpid())
    subprocess.check_call([
        "gcc", "-O2", "-ffp-contract=off", "-fno-fast-math", "-std=c11", "-fPIC", "-shared",
        "-Wall", "-Wextra", "-Werror", "-o", str(tmp), str(src), "-lm",
    ])
    os.replace(tmp, out)
    return out


def build() -> pathlib.Path:
    """Compile tk_oracle.c into libtk_oracle.so next to it."""
    return compile_source(_SRC, _LIB)


def _open(path) -> ctypes.CDLL:
    lib = ctypes.CDLL(str(path))
    p, i64, i32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32
    for name in ("oracle_per_token_cast", "oracle_swiglu_per_token_cast", "oracle_per_token_cast_f32"):
        fn = getattr(lib, name)
        fn.argtypes = [p, i64, i64, i64, p, i64, p, i64, i32, i32, i32, i32, p]
        fn.restype = ctypes.c_int
    for name in ("oracle_encode_e4m3_n", "oracle_encode_e2m1_n", "oracle_silu32_n"):
        fn = getattr(lib, name)
        fn.argtypes = [p, p, i64]
        fn.restype = None
    lib.oracle_group_scale_n.argtypes = [p, p, p, i64, i32, i32]
    lib.oracle_group_scale_n.restype = None
    lib.oracle_div_n.argtypes = [p, p, p, i64]
    lib.oracle_div_n.restype = None
    lib.oracle_per_token_dequant.argtypes = [p, i64, i64, i64, p, i64, i32, i32, i32, p, i64, i32]
    lib.oracle_per_token_dequant.restype = ctypes.c_int
    lib.oracle_per_token_cast_back.argtypes = [p, i64, i64, i64, p, i64, i32, i32, i32, p, p, p]
    lib.oracle_per_token_cast_back.restype = ctypes.c_int
    lib.oracle_per_block_cast.argtypes = [p, i64, i64, i64, p, i64, p, i64, i64, i64, i32, i32, i32]
    lib.oracle_per_block_cast.restype = ctypes.c_int
    lib.oracle_rmsnorm.argtypes = [p, i64, i64, i64, p, ctypes.c_float, p, i64, i32, p]
    lib.oracle_rmsnorm.restype = ctypes.c_int
    lib.oracle_rmsnorm_cast.argtypes = [p, i64, i64, i64, p, ctypes.c_float, p, i64, p, i64, i32, i32, i32, i32, p]
    lib.oracle_rmsnorm_cast.restype = ctypes.c_int
    lib.oracle_sum_squares_rows.argtypes = [p, i64, i64, i64, p]
    lib.oracle_sum_squares_rows.restype = None
    lib.oracle_code_value_n.argtypes = [p, p, i64, i32]
    lib.oracle_code_value_n.restype = None
    lib.oracle_f32_to_bf16_n.argtypes = [p, p, i64]
    lib.oracle_f32_to_bf16_n.restype = None
    return lib


def _lib():
    """The oracle library: TK_ORACLE_LIBRARY names another build of tk_oracle.c
    (the sanitizer test's), else libtk_oracle.so, rebuilt when older than the
    source."""
    global _handle
    with _lock:
        if _handle is None:
            other = os.environ.get("TK_ORACLE_LIBRARY")
            if other:
                _handle = _open(other)
                return _handle
            if not _LIB.exists() or _LIB.stat().st_mtime < _SRC.stat().st_mtime:
                build()
            _handle = _open(_LIB)
        return _handle


class using:
    """Context manager that points this module at another build of the oracle
    source (the tests use it to check that planted mistakes are caught)."""

    def __init__(self, path):
        self._path = path

    def __enter__(self):
        global _handle
        self._saved = _lib()
        with _lock:
            _handle = _open(self._path)
        return self

    def __exit__(self, *exc):
        global _handle
        with _lock:
            _handle = self._saved
        return False


def _ptr(a: np.ndarray) -> int:
    return a.ctypes.data


def _check_2d(x: np.ndarray):
    if x.dtype != np.uint16 or x.ndim != 2:
        raise TypeError("bf16 input must be a 2-D uint16 array of bf16 bit patterns")
    if x.strides[1] != 2 or x.strides[0] % 2 != 0:
        raise ValueError("rows must be contiguous")


def _outputs(rows, cols, group, out_dtype, scale_fmt):
    qcols = cols if out_dtype == "e4m3" else cols // 2
    q = np.zeros((rows, qcols), dtype=np.uint8)
    if scale_fmt == "f32":
        s = np.zeros((rows, cols // group), dtype=np.float32)
    else:
        s = np.zeros((rows, cols // group // 4), dtype=np.int32)
    return q, s


def per_token_cast(x: np.ndarray, group: int = 128, out_dtype: str = "e4m3",
                   round_pow2: bool = False, scale_fmt: str = "f32"):
    """Oracle cast of bf16 bits ``x`` [rows, cols] -> (codes, scales).

    codes: uint8 [rows, cols] (e4m3) or [rows, cols/2] (e2m1, element 2i in
    the low nibble).  scales: float32 [rows, cols/group], or int32
    [rows, cols/group/4] holding UE8M0 bytes little-endian (scale_fmt="ue8m0").
    """
    _check_2d(x)
    rows, cols = x.shape
    q, s = _outputs(rows, cols, group, out_dtype, scale_fmt)
    work = np.empty(cols, dtype=np.float32)
    rc = _lib().oracle_per_token_cast(
        _ptr(x), rows, cols, x.strides[0] // 2, _ptr(q), q.shape[1], _ptr(s), s.shape[1],
        group, _QDTYPES[out_dtype], int(bool(round_pow2)), _SCALE_FMTS[scale_fmt], _ptr(work))
    if rc != 0:
        raise ValueError("oracle rejected the cast arguments")
    return q, s


def per_token_cast_f32(x: np.ndarray, group: int = 128, out_dtype: str = "e4m3",
                       round_pow2: bool = False, scale_fmt: str = "f32"):
    """Oracle cast of fp32 activations x [rows, cols] -> (codes, scales)."""
    if x.dtype != np.float32 or x.ndim != 2 or x.strides[1] != 4:
        raise TypeError("x must be a 2-D float32 array with contiguous rows")
    rows, cols = x.shape
    q, s = _outputs(rows, cols, group, out_dtype, scale_fmt)
    work = np.empty(cols, dtype=np.float32)
    rc = _lib().oracle_per_token_cast_f32(
        _ptr(x), rows, cols, x.strides[0] // 4, _ptr(q), q.shape[1], _ptr(s), s.shape[1],
        group, _QDTYPES[out_dtype], int(bool(round_pow2)), _SCALE_FMTS[scale_fmt], _ptr(work))
    if rc != 0:
        raise ValueError("oracle rejected the cast arguments")
    return q, s


def swiglu_per_token_cast(gate_up: np.ndarray, group: int = 128, out_dtype: str = "e4m3",
                          round_pow2: bool = False, scale_fmt: str = "f32"):
    """Oracle of the fused form: gate_up bf16 bits [rows, 2*I]; gate = first I
    columns, up = last I; casts h = fl32(silu32(gate) * up) -> (codes, scales)."""
    _check_2d(gate_up)
    rows, cols2 = gate_up.shape
    if cols2 % 2:
        raise ValueError("gate_up must have an even number of columns")
    cols = cols2 // 2
    q, s = _outputs(rows, cols, group, out_dtype, scale_fmt)
    work = np.empty(cols, dtype=np.float32)
    rc = _lib().oracle_swiglu_per_token_cast(
        _ptr(gate_up), rows, cols, gate_up.strides[0] // 2, _ptr(q), q.shape[1], _ptr(s),
        s.shape[1], group, _QDTYPES[out_dtype], int(bool(round_pow2)), _SCALE_FMTS[scale_fmt],
        _ptr(work))
    if rc != 0:
        raise ValueError("oracle rejected the cast arguments")
    return q, s


def encode_e4m3(v) -> np.ndarray:
    """Saturating RNE fp32 -> OCP e4m3fn byte, elementwise."""
    v = np.ascontiguousarray(v, dtype=np.float32)
    out = np.empty(v.shape, dtype=np.uint8)
    _lib().oracle_encode_e4m3_n(_ptr(v), _ptr(out), v.size)
    return out


def encode_e2m1(v) -> np.ndarray:
    """Saturating RNE fp32 -> e2m1 nibble (0..15), elementwise."""
    v = np.ascontiguousarray(v, dtype=np.float32)
    out = np.empty(v.shape, dtype=np.uint8)
    _lib().oracle_encode_e2m1_n(_ptr(v), _ptr(out), v.size)
    return out


def silu32(g) -> np.ndarray:
    """fp32 nearest to g / (1 + e^-g), elementwise over fp32 inputs."""
    g = np.ascontiguousarray(g, dtype=np.float32)
    out = np.empty(g.shape, dtype=np.float32)
    _lib().oracle_silu32_n(_ptr(g), _ptr(out), g.size)
    return out


def group_scale(amax, out_dtype: str = "e4m3", round_pow2: bool = False):
    """Scale from group amax (floor, divide, optional pow2) -> (fp32 s, exponent byte)."""
    a = np.ascontiguousarray(amax, dtype=np.float32)
    s = np.empty(a.shape, dtype=np.float32)
    e8 = np.empty(a.shape, dtype=np.uint8)
    _lib().oracle_group_scale_n(_ptr(a), _ptr(s), _ptr(e8), a.size, _QDTYPES[out_dtype],
                                int(bool(round_pow2)))
    return s, e8


def divide(x, s) -> np.ndarray:
    """The cast's fp32 division x / s, elementwise."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    s = np.ascontiguousarray(np.broadcast_to(s, x.shape), dtype=np.float32)
    out = np.empty(x.shape, dtype=np.float32)
    _lib().oracle_div_n(_ptr(x), _ptr(s), _ptr(out), x.size)
    return out


def per_token_dequant(q: np.ndarray, scales: np.ndarray, cols: int, group: int = 128,
                      in_dtype: str = "e4m3", scale_fmt: str = "f32", out: str = "bf16"):
    """Oracle dequantization: codes + scales -> y = fl32(value(code) * s) as
    fp32 (out="f32") or bf16 bit patterns (out="bf16"), [rows, cols]."""
    q = np.ascontiguousarray(q, dtype=np.uint8)
    rows = q.shape[0]
    sc = np.ascontiguousarray(scales)
    y = np.zeros((rows, cols), dtype=np.float32 if out == "f32" else np.uint16)
    rc = _lib().oracle_per_token_dequant(
        _ptr(q), rows, cols, q.shape[1], _ptr(sc), sc.shape[1], group, _QDTYPES[in_dtype],
        _SCALE_FMTS[scale_fmt], _ptr(y), cols, int(out == "f32"))
    if rc != 0:
        raise ValueError("oracle rejected the dequantization arguments")
    return y


def per_token_cast_back(x: np.ndarray, group: int = 128, out_dtype: str = "e4m3",
                        round_pow2: bool = False):
    """Oracle cast-and-cast-back: bf16 bits [rows, cols] -> bf16 bits of the
    dequantized cast (fp32 scales; UE8M0 packing does not change values)."""
    _check_2d(x)
    rows, cols = x.shape
    y = np.zeros((rows, cols), dtype=np.uint16)
    work = np.empty(cols, dtype=np.float32)
    qwork = np.zeros(cols, dtype=np.uint8)
    swork = np.empty(max(cols // group, 1), dtype=np.float32)
    rc = _lib().oracle_per_token_cast_back(
        _ptr(x), rows, cols, x.strides[0] // 2, _ptr(y), cols, group, _QDTYPES[out_dtype],
        int(bool(round_pow2)), _ptr(work), _ptr(qwork), _ptr(swork))
    if rc != 0:
        raise ValueError("oracle rejected the cast-back arguments")
    return y


def code_value(codes, in_dtype: str = "e4m3") -> np.ndarray:
    """fp32 value of E4M3 bytes or E2M1 nibbles, elementwise."""
    c = np.ascontiguousarray(codes, dtype=np.uint8)
    out = np.empty(c.shape, dtype=np.float32)
    _lib().oracle_code_value_n(_ptr(c), _ptr(out), c.size, _QDTYPES[in_dtype])
    return out


def f32_to_bf16(v) -> np.ndarray:
    """fp32 -> bf16 bit patterns, nearest with ties to even, elementwise."""
    v = np.ascontiguousarray(v, dtype=np.float32)
    out = np.empty(v.shape, dtype=np.uint16)
    _lib().oracle_f32_to_bf16_n(_ptr(v), _ptr(out), v.size)
    return out


def per_block_cast(x: np.ndarray, block_rows: int = 128, block_cols: int = 128, out_dtype: str = "e4m3",
                   round_pow2: bool = False, scale_fmt: str = "f32"):
    """Oracle per-block cast of bf16 bits x [rows, cols] -> (codes, scales);
    scales [ceil(rows/block_rows), cols/block_cols] fp32 or [.., cols/block_cols/4] int32."""
    _check_2d(x)
    rows, cols = x.shape
    if block_rows <= 0 or block_cols <= 0:
        raise ValueError("block sizes must be positive")
    qcols = cols if out_dtype == "e4m3" else cols // 2
    q = np.zeros((rows, qcols), dtype=np.uint8)
    nbr, nbc = -(-rows // block_rows), cols // block_cols
    s = np.zeros((nbr, nbc), np.float32) if scale_fmt == "f32" else np.zeros((nbr, max(nbc // 4, 1)), np.int32)
    rc = _lib().oracle_per_block_cast(_ptr(x), rows, cols, x.strides[0] // 2, _ptr(q), qcols, _ptr(s),
                                      s.shape[1], block_rows, block_cols, _QDTYPES[out_dtype],
                                      int(bool(round_pow2)), _SCALE_FMTS[scale_fmt])
    if rc != 0:
        raise ValueError("oracle rejected the per-block cast arguments")
    return q, s


def per_channel_cast(x: np.ndarray, out_dtype: str = "e4m3", round_pow2: bool = False,
                     scale_fmt: str = "f32"):
    """Oracle per-channel cast: one scale per column over all rows -> (codes,
    scales [cols] fp32 or [cols/4] int32)."""
    rows = x.shape[0]
    q, s = per_block_cast(x, max(rows, 1), 1, out_dtype, round_pow2, scale_fmt)
    return q, s.reshape(-1)


def sum_squares(x: np.ndarray) -> np.ndarray:
    """Per row of bf16 bits x: the exact sum of squares rounded to fp32."""
    _check_2d(x)
    out = np.empty(x.shape[0], dtype=np.float32)
    _lib().oracle_sum_squares_rows(_ptr(x), x.shape[0], x.shape[1], x.strides[0] // 2, _ptr(out))
    return out


def _weight_ptr(weight, cols):
    if weight is None:
        return None, None
    w = np.ascontiguousarray(weight, dtype=np.uint16)
    if w.shape != (cols,):
        raise ValueError("weight must be bf16 bits of shape [cols]")
    return w, _ptr(w)


def rmsnorm(x: np.ndarray, weight: np.ndarray | None = None, eps: float = 1e-6, out: str = "bf16") -> np.ndarray:
    """Oracle RMSNorm forward of bf16 bits x [rows, cols] with bf16 weight bits
    [cols] (or none) -> bf16 bits (uint16) or fp32 [rows, cols]."""
    _check_2d(x)
    rows, cols = x.shape
    w, wp = _weight_ptr(weight, cols)
    y = np.empty((rows, cols), dtype=np.uint16 if out == "bf16" else np.float32)
    work = np.empty(cols, dtype=np.float32)
    rc = _lib().oracle_rmsnorm(_ptr(x), rows, cols, x.strides[0] // 2, wp, eps, _ptr(y), cols,
                               0 if out == "bf16" else 1, _ptr(work))
    if rc != 0:
        raise ValueError("oracle rejected the RMSNorm arguments")
    return y


def rmsnorm_cast(x: np.ndarray, weight: np.ndarray | None = None, eps: float = 1e-6, group: int = 128,
                 out_dtype: str = "e4m3", round_pow2: bool = False, scale_fmt: str = "f32"):
    """Oracle RMSNorm forward followed by the per-token cast of its fp32
    output -> (codes, scales) as per_token_cast returns them."""
    _check_2d(x)
    rows, cols = x.shape
    w, wp = _weight_ptr(weight, cols)
    q, s = _outputs(rows, cols, group, out_dtype, scale_fmt)
    work = np.empty(cols, dtype=np.float32)
    rc = _lib().oracle_rmsnorm_cast(_ptr(x), rows, cols, x.strides[0] // 2, wp, eps, _ptr(q), q.shape[1],
                                    _ptr(s), s.shape[1], group, _QDTYPES[out_dtype], int(bool(round_pow2)),
                                    _SCALE_FMTS[scale_fmt], _ptr(work))
    if rc != 0:
        raise ValueError("oracle rejected the RMSNorm-cast arguments")
    return q, s
