"""Thin Python binding over libtk_quant.so (argument marshalling only).

PyTorch supplies device memory and the current stream; every step of the cast
runs in the library's HIP kernels.  The functions named like the C ABI
(``tk_per_token_cast`` ...) take tensors that the caller allocated; the
convenience forms (``per_token_cast`` ...) allocate the outputs.

There is no fallback: if the library is missing or fails to load, every call
raises.
"""
from __future__ import annotations

import ctypes
import os
import pathlib
import threading

import torch  # imported first so the library binds to torch's HIP runtime

_PKG = pathlib.Path(__file__).resolve().parent
LIB_PATH = _PKG / "libtk_quant.so"

TK_SUCCESS = 0
QDTYPES = {"e4m3": 0, "e2m1": 1}
SCALE_FMTS = {"f32": 0, "ue8m0": 1}
OUT_DTYPES = {"bf16": 0, "f32": 1}
GROUPS = (16, 32, 64, 128)

_lock = threading.Lock()
_lib_handle = None


class TkError(RuntimeError):
    """A tk_* call returned a status other than TK_SUCCESS."""

    def __init__(self, status: int, message: str):
        super().__init__(message)
        self.status = status


def load_library(path: pathlib.Path | str | None = None) -> ctypes.CDLL:
    """Load (once) and return the HIP library; raises if it is not built.
    Without `path`, TK_QUANT_LIBRARY names another build of the same sources
    (e.g. one with sanitized host code), else libtk_quant.so next to this file."""
    global _lib_handle
    with _lock:
        if _lib_handle is not None and path is None:
            return _lib_handle
        if path is not None:
            p = pathlib.Path(path)
        else:
            p = pathlib.Path(os.environ.get("TK_QUANT_LIBRARY") or LIB_PATH)
        if not p.exists():
            raise RuntimeError(
                f"{p} is not built; run `python -m activation_quantization_token_amd.build`")
        lib = ctypes.CDLL(str(p))
        vp, i64, i32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32
        for name in ("tk_per_token_cast", "tk_swiglu_per_token_cast", "tk_per_token_cast_f32"):
            fn = getattr(lib, name)
            fn.argtypes = [vp, i64, i64, i64, vp, i64, vp, i64, i32, i32, i32, i32, vp]
            fn.restype = ctypes.c_int
        lib.tk_per_token_dequant.argtypes = [vp, i64, i64, i64, vp, i64, i32, i32, i32, vp, i64, i32, vp]
        lib.tk_per_token_dequant.restype = ctypes.c_int
        lib.tk_per_token_cast_back.argtypes = [vp, i64, i64, i64, vp, i64, i32, i32, i32, vp]
        lib.tk_per_token_cast_back.restype = ctypes.c_int
        lib.tk_per_block_cast.argtypes = [vp, i64, i64, i64, vp, i64, vp, i64, i64, i64, i32, i32, i32, vp]
        lib.tk_per_block_cast.restype = ctypes.c_int
        lib.tk_per_channel_workspace_bytes.argtypes = [i64, i64]
        lib.tk_per_channel_workspace_bytes.restype = i64
        lib.tk_per_channel_cast.argtypes = [vp, i64, i64, i64, vp, i64, vp, vp, i64, i32, i32, i32, vp]
        lib.tk_per_channel_cast.restype = ctypes.c_int
        lib.tk_per_channel_cast_noalloc.argtypes = [vp, i64, i64, i64, vp, i64, vp, i32, i32, i32, vp]
        lib.tk_per_channel_cast_noalloc.restype = ctypes.c_int
        lib.tk_per_channel_noalloc_max_workspace_bytes.argtypes = []
        lib.tk_per_channel_noalloc_max_workspace_bytes.restype = i64
        f32 = ctypes.c_float
        lib.tk_rmsnorm.argtypes = [vp, i64, i64, i64, vp, f32, vp, i64, i32, vp]
        lib.tk_rmsnorm.restype = ctypes.c_int
        lib.tk_rmsnorm_cast.argtypes = [vp, i64, i64, i64, vp, f32, vp, i64, vp, i64, i32, i32, i32, i32, vp]
        lib.tk_rmsnorm_cast.restype = ctypes.c_int
        lib.tk_silu32_bf16.argtypes = [vp, vp, i64, vp]
        lib.tk_silu32_bf16.restype = ctypes.c_int
        lib.tk_copy_stream.argtypes = [vp, vp, i64, vp]
        lib.tk_copy_stream.restype = ctypes.c_int
        lib.tk_stream_rw.argtypes = [vp, i64, vp, i64, vp]
        lib.tk_stream_rw.restype = ctypes.c_int
        lib.tk_prepare_device.argtypes = []
        lib.tk_prepare_device.restype = ctypes.c_int
        lib.tk_status_string.argtypes = [i32]
        lib.tk_status_string.restype = ctypes.c_char_p
        lib.tk_abi_version.argtypes = []
        lib.tk_abi_version.restype = ctypes.c_int32
        if path is None:
            _lib_handle = lib
        return lib


def tk_status_string(status: int) -> str:
    return load_library().tk_status_string(int(status)).decode()


def tk_abi_version() -> int:
    return int(load_library().tk_abi_version())


def _check(status: int):
    if status != TK_SUCCESS:
        raise TkError(status, tk_status_string(status))


def _stream_handle(stream, device) -> int:
    if stream is None:
        stream = torch.cuda.current_stream(device)
    if isinstance(stream, torch.cuda.Stream):
        return stream.cuda_stream
    return int(stream)


def tk_prepare_device() -> None:
    _check(load_library().tk_prepare_device())


def tk_silu32_bf16(g: int, out: int, n: int, stream: int) -> int:
    """Raw C call: out[i] = silu32(g[i]) for bf16 gates; returns the tk_status code."""
    return load_library().tk_silu32_bf16(g, out, n, stream)


def silu32_bf16(g: torch.Tensor, stream=None) -> torch.Tensor:
    """Diagnostic: the fused kernel's silu32 applied to a 1-D bf16 tensor."""
    if g.dtype != torch.bfloat16 or g.dim() != 1 or not g.is_cuda or g.stride(0) != 1:
        raise TypeError("g must be a contiguous 1-D torch.bfloat16 GPU tensor")
    out = torch.empty(g.shape, dtype=torch.float32, device=g.device)
    _check(tk_silu32_bf16(g.data_ptr(), out.data_ptr(), g.numel(), _stream_handle(stream, g.device)))
    return out


def tk_copy_stream(src: int, dst: int, nbytes: int, stream: int) -> int:
    """Raw C call: streaming copy of nbytes (diagnostic); returns the tk_status code."""
    return load_library().tk_copy_stream(src, dst, nbytes, stream)


def copy_stream(src: torch.Tensor, dst: torch.Tensor, stream=None) -> None:
    """Diagnostic: byte copy src -> dst with the cast's streaming memory instructions."""
    for t in (src, dst):
        if not t.is_cuda or not t.is_contiguous():
            raise TypeError("src and dst must be contiguous GPU tensors")
    n = src.numel() * src.element_size()
    if dst.numel() * dst.element_size() < n:
        raise ValueError("dst is smaller than src")
    _check(tk_copy_stream(src.data_ptr(), dst.data_ptr(), n, _stream_handle(stream, src.device)))


def tk_stream_rw(src: int, read_bytes: int, dst: int, write_bytes: int, stream: int) -> int:
    """Raw C call: streaming-ceiling diagnostic; returns the tk_status code."""
    return load_library().tk_stream_rw(src, read_bytes, dst, write_bytes, stream)


def stream_rw(src: torch.Tensor, read_bytes: int, dst: torch.Tensor, write_bytes: int, stream=None) -> None:
    """Diagnostic: read `read_bytes` of src and write `write_bytes` of dst (the
    cast's memory instructions; practical streaming ceiling)."""
    for t, n in ((src, read_bytes), (dst, write_bytes)):
        if not t.is_cuda or not t.is_contiguous() or t.numel() * t.element_size() < n:
            raise ValueError("src and dst must be contiguous GPU tensors holding the byte counts")
    _check(tk_stream_rw(src.data_ptr(), read_bytes, dst.data_ptr(), write_bytes, _stream_handle(stream, src.device)))


def tk_per_token_cast(x: int, rows: int, cols: int, x_ld: int, q: int, q_ld: int, scales: int,
                      s_ld: int, group: int, out_dtype: int, round_pow2: int, scale_fmt: int,
                      stream: int) -> int:
    """Raw C call with integer pointers; returns the tk_status code."""
    return load_library().tk_per_token_cast(x, rows, cols, x_ld, q, q_ld, scales, s_ld, group,
                                            out_dtype, round_pow2, scale_fmt, stream)


def tk_per_token_cast_f32(x: int, rows: int, cols: int, x_ld: int, q: int, q_ld: int, scales: int,
                          s_ld: int, group: int, out_dtype: int, round_pow2: int, scale_fmt: int,
                          stream: int) -> int:
    """Raw C call (fp32 input) with integer pointers; returns the tk_status code."""
    return load_library().tk_per_token_cast_f32(x, rows, cols, x_ld, q, q_ld, scales, s_ld, group,
                                                out_dtype, round_pow2, scale_fmt, stream)


def tk_swiglu_per_token_cast(gate_up: int, rows: int, cols: int, x_ld: int, q: int, q_ld: int,
                             scales: int, s_ld: int, group: int, out_dtype: int, round_pow2: int,
                             scale_fmt: int, stream: int) -> int:
    """Raw C call with integer pointers; returns the tk_status code."""
    return load_library().tk_swiglu_per_token_cast(gate_up, rows, cols, x_ld, q, q_ld, scales,
                                                   s_ld, group, out_dtype, round_pow2, scale_fmt,
                                                   stream)


def _check_input(x: torch.Tensor, what: str, dtype=torch.bfloat16):
    if not isinstance(x, torch.Tensor) or x.dtype != dtype or x.dim() != 2:
        raise TypeError(f"{what} must be a 2-D {dtype} tensor")
    if not x.is_cuda:
        raise TypeError(f"{what} must be on a GPU device")
    if x.stride(1) != 1:
        raise ValueError(f"{what} must have contiguous rows (stride(1) == 1)")


def empty_outputs(rows: int, cols: int, group: int, out_dtype: str, scale_fmt: str, device):
    """Allocate (codes, scales) for a cast of `cols` output channels."""
    q_cols = cols if out_dtype == "e4m3" else cols // 2
    q = torch.empty((rows, q_cols), dtype=torch.uint8, device=device)
    if scale_fmt == "f32":
        s = torch.empty((rows, cols // group), dtype=torch.float32, device=device)
    else:
        s = torch.empty((rows, cols // group // 4), dtype=torch.int32, device=device)
    return q, s


def _check_out_shapes(q, s, q_cols, s_cols, scale_fmt):
    """Caller-given outputs: dtypes, and room for every column the call writes."""
    if q.dtype != torch.uint8:
        raise TypeError("codes must be uint8")
    want = torch.float32 if scale_fmt == "f32" else torch.int32
    if s.dtype != want:
        raise TypeError(f"scales must be {want} for scale_fmt {scale_fmt!r}")
    if q.shape[-1] < q_cols or s.shape[-1] < s_cols:
        raise ValueError(f"outputs too narrow: codes need {q_cols} columns, scales {s_cols}")


def _run(fn, x, cols, group, out_dtype, round_pow2, scale_fmt, out, stream):
    if group not in GROUPS:
        raise ValueError(f"group must be one of {GROUPS}")
    if out_dtype not in QDTYPES or scale_fmt not in SCALE_FMTS:
        raise ValueError("out_dtype must be 'e4m3'|'e2m1' and scale_fmt 'f32'|'ue8m0'")
    rows = x.shape[0]
    if out is None:
        if cols % group or (scale_fmt == "ue8m0" and (cols // group) % 4):
            raise ValueError("cols must be a multiple of group (of 4*group for ue8m0 scales)")
        q, s = empty_outputs(rows, cols, group, out_dtype, scale_fmt, x.device)
    else:
        q, s = out
    for t in (q, s):
        if t.device != x.device or t.dim() != 2 or t.stride(1) != 1 or t.shape[0] != rows:
            raise ValueError("outputs must be 2-D, row-contiguous, on the input's device")
    _check_out_shapes(q, s, cols if out_dtype == "e4m3" else cols // 2,
                      cols // group if scale_fmt == "f32" else cols // group // 4, scale_fmt)
    st = fn(x.data_ptr(), rows, cols, x.stride(0), q.data_ptr(), q.stride(0), s.data_ptr(),
            s.stride(0), group, QDTYPES[out_dtype], int(bool(round_pow2)), SCALE_FMTS[scale_fmt],
            _stream_handle(stream, x.device))
    _check(st)
    return q, s


def per_token_cast(x: torch.Tensor, group: int = 128, out_dtype: str = "e4m3",
                   round_pow2: bool = False, scale_fmt: str = "f32", out=None, stream=None):
    """bf16 or fp32 x [rows, cols] -> (codes uint8, scales float32 | int32), see include/tk_quant.h."""
    if isinstance(x, torch.Tensor) and x.dtype == torch.float32:
        _check_input(x, "x", torch.float32)
        return _run(tk_per_token_cast_f32, x, x.shape[1], group, out_dtype, round_pow2, scale_fmt, out,
                    stream)
    _check_input(x, "x")
    return _run(tk_per_token_cast, x, x.shape[1], group, out_dtype, round_pow2, scale_fmt, out,
                stream)


def swiglu_per_token_cast(gate_up: torch.Tensor, group: int = 128, out_dtype: str = "e4m3",
                          round_pow2: bool = False, scale_fmt: str = "f32", out=None,
                          stream=None):
    """bf16 gate_up [rows, 2*I] -> cast of silu(gate) * up, (codes, scales)."""
    _check_input(gate_up, "gate_up")
    if gate_up.shape[1] % 2:
        raise ValueError("gate_up must have an even number of columns")
    return _run(tk_swiglu_per_token_cast, gate_up, gate_up.shape[1] // 2, group, out_dtype,
                round_pow2, scale_fmt, out, stream)


def tk_per_token_dequant(q: int, rows: int, cols: int, q_ld: int, scales: int, s_ld: int, group: int,
                         in_dtype: int, scale_fmt: int, y: int, y_ld: int, y_dtype: int,
                         stream: int) -> int:
    """Raw C call with integer pointers; returns the tk_status code."""
    return load_library().tk_per_token_dequant(q, rows, cols, q_ld, scales, s_ld, group, in_dtype,
                                               scale_fmt, y, y_ld, y_dtype, stream)


def tk_per_token_cast_back(x: int, rows: int, cols: int, x_ld: int, y: int, y_ld: int, group: int,
                           out_dtype: int, round_pow2: int, stream: int) -> int:
    """Raw C call with integer pointers; returns the tk_status code."""
    return load_library().tk_per_token_cast_back(x, rows, cols, x_ld, y, y_ld, group, out_dtype,
                                                 round_pow2, stream)


def per_token_dequant(q: torch.Tensor, scales: torch.Tensor, cols: int, group: int = 128,
                      in_dtype: str = "e4m3", scale_fmt: str = "f32", out_dtype: str = "bf16",
                      out=None, stream=None) -> torch.Tensor:
    """Codes + scales (as per_token_cast returns them) -> y [rows, cols] in
    bf16 or fp32, y = value(code) * s."""
    for t, what in ((q, "q"), (scales, "scales")):
        if not isinstance(t, torch.Tensor) or not t.is_cuda or t.dim() != 2 or t.stride(1) != 1:
            raise TypeError(f"{what} must be a 2-D row-contiguous GPU tensor")
    _check_formats(in_dtype, scale_fmt)
    if out_dtype not in OUT_DTYPES:
        raise ValueError("out_dtype must be 'bf16'|'f32'")
    if group not in GROUPS or cols <= 0 or cols % group or (scale_fmt == "ue8m0" and (cols // group) % 4):
        raise ValueError("cols must be a positive multiple of group (of 4*group for ue8m0 scales)")
    rows = q.shape[0]
    if scales.shape[0] != rows or scales.device != q.device:
        raise ValueError("scales must have q's rows, on q's device")
    _check_out_shapes(q, scales, cols if in_dtype == "e4m3" else cols // 2,
                      cols // group if scale_fmt == "f32" else cols // group // 4, scale_fmt)
    ydt = torch.bfloat16 if out_dtype == "bf16" else torch.float32
    y = torch.empty((rows, cols), dtype=ydt, device=q.device) if out is None else out
    if (y.dtype != ydt or y.dim() != 2 or y.stride(1) != 1 or tuple(y.shape) != (rows, cols)
            or y.device != q.device):
        raise ValueError("out must be a row-contiguous [rows, cols] tensor of the output dtype on q's device")
    _check(tk_per_token_dequant(q.data_ptr(), rows, cols, q.stride(0), scales.data_ptr(), scales.stride(0),
                                group, QDTYPES[in_dtype], SCALE_FMTS[scale_fmt], y.data_ptr(), y.stride(0),
                                OUT_DTYPES[out_dtype], _stream_handle(stream, q.device)))
    return y


def per_token_cast_back(x: torch.Tensor, group: int = 128, out_dtype: str = "e4m3",
                        round_pow2: bool = False, out=None, stream=None) -> torch.Tensor:
    """bf16 x -> bf16 dequantized per-token cast of x, fused (no codes written)."""
    _check_input(x, "x")
    rows, cols = x.shape
    y = torch.empty((rows, cols), dtype=torch.bfloat16, device=x.device) if out is None else out
    if (y.dtype != torch.bfloat16 or y.dim() != 2 or y.stride(1) != 1 or tuple(y.shape) != (rows, cols)
            or y.device != x.device):
        raise ValueError("out must be a row-contiguous bf16 tensor of x's shape on x's device")
    if out_dtype not in QDTYPES:
        raise ValueError("out_dtype must be 'e4m3'|'e2m1'")
    _check(tk_per_token_cast_back(x.data_ptr(), rows, cols, x.stride(0), y.data_ptr(), y.stride(0), group,
                                  QDTYPES[out_dtype], int(bool(round_pow2)), _stream_handle(stream, x.device)))
    return y


def tk_per_block_cast(x: int, rows: int, cols: int, x_ld: int, q: int, q_ld: int, scales: int, s_ld: int,
                      block_rows: int, block_cols: int, out_dtype: int, round_pow2: int, scale_fmt: int,
                      stream: int) -> int:
    """Raw C call with integer pointers; returns the tk_status code."""
    return load_library().tk_per_block_cast(x, rows, cols, x_ld, q, q_ld, scales, s_ld, block_rows, block_cols,
                                            out_dtype, round_pow2, scale_fmt, stream)


def tk_per_channel_workspace_bytes(rows: int, cols: int) -> int:
    return int(load_library().tk_per_channel_workspace_bytes(rows, cols))


def tk_per_channel_cast(x: int, rows: int, cols: int, x_ld: int, q: int, q_ld: int, scales: int, workspace: int,
                        workspace_bytes: int, out_dtype: int, round_pow2: int, scale_fmt: int, stream: int) -> int:
    """Raw C call with integer pointers; returns the tk_status code."""
    return load_library().tk_per_channel_cast(x, rows, cols, x_ld, q, q_ld, scales, workspace, workspace_bytes,
                                              out_dtype, round_pow2, scale_fmt, stream)


def tk_per_channel_cast_noalloc(x: int, rows: int, cols: int, x_ld: int, q: int, q_ld: int, scales: int,
                                out_dtype: int, round_pow2: int, scale_fmt: int, stream: int) -> int:
    """Raw C call with integer pointers (the library's static workspace); returns the tk_status code."""
    return load_library().tk_per_channel_cast_noalloc(x, rows, cols, x_ld, q, q_ld, scales, out_dtype, round_pow2,
                                                      scale_fmt, stream)


def tk_per_channel_noalloc_max_workspace_bytes() -> int:
    return int(load_library().tk_per_channel_noalloc_max_workspace_bytes())


def _check_formats(out_dtype: str, scale_fmt: str):
    if out_dtype not in QDTYPES or scale_fmt not in SCALE_FMTS:
        raise ValueError("out_dtype must be 'e4m3'|'e2m1' and scale_fmt 'f32'|'ue8m0'")


def per_block_cast(x: torch.Tensor, block_rows: int = 128, block_cols: int = 128, out_dtype: str = "e4m3",
                   round_pow2: bool = False, scale_fmt: str = "f32", out=None, stream=None):
    """bf16 x [rows, cols] -> (codes, scales) with one scale per block_rows x
    block_cols block; scales [ceil(rows/block_rows), cols/block_cols] float32
    or [.., cols/block_cols/4] int32 (UE8M0)."""
    _check_input(x, "x")
    _check_formats(out_dtype, scale_fmt)
    rows, cols = x.shape
    if block_rows <= 0 or block_cols not in GROUPS or cols % block_cols:
        raise ValueError("block_rows must be positive and block_cols one of 16/32/64/128 dividing cols")
    nbr, nbc = -(-rows // block_rows), cols // block_cols
    if out is None:
        if scale_fmt == "ue8m0" and nbc % 4:
            raise ValueError("ue8m0 scales need a multiple of 4 column blocks")
        q = torch.empty((rows, cols if out_dtype == "e4m3" else cols // 2), dtype=torch.uint8, device=x.device)
        s = (torch.empty((nbr, nbc), dtype=torch.float32, device=x.device) if scale_fmt == "f32"
             else torch.empty((nbr, nbc // 4), dtype=torch.int32, device=x.device))
    else:
        q, s = out
    for t in (q, s):
        if t.device != x.device or t.dim() != 2 or t.stride(1) != 1:
            raise ValueError("outputs must be 2-D, row-contiguous, on the input's device")
    if q.shape[0] != rows or s.shape[0] != nbr:
        raise ValueError("outputs have the wrong number of rows")
    _check_out_shapes(q, s, cols if out_dtype == "e4m3" else cols // 2, nbc if scale_fmt == "f32" else nbc // 4,
                      scale_fmt)
    _check(tk_per_block_cast(x.data_ptr(), rows, cols, x.stride(0), q.data_ptr(), q.stride(0), s.data_ptr(),
                             s.stride(0), block_rows, block_cols, QDTYPES[out_dtype], int(bool(round_pow2)),
                             SCALE_FMTS[scale_fmt], _stream_handle(stream, x.device)))
    return q, s


def per_channel_cast(x: torch.Tensor, out_dtype: str = "e4m3", round_pow2: bool = False, scale_fmt: str = "f32",
                     out=None, workspace: torch.Tensor | None = None, stream=None):
    """bf16 x [rows, cols] -> (codes, scales) with one scale per column;
    scales [cols] float32 or [cols/4] int32 (UE8M0).  `workspace` (a GPU
    tensor of at least tk_per_channel_workspace_bytes(rows, cols) bytes) is
    allocated when not given."""
    _check_input(x, "x")
    _check_formats(out_dtype, scale_fmt)
    rows, cols = x.shape
    if out is None:
        if cols % 8:
            raise ValueError("cols must be a multiple of 8")
        q = torch.empty((rows, cols if out_dtype == "e4m3" else cols // 2), dtype=torch.uint8, device=x.device)
        s = (torch.empty((cols,), dtype=torch.float32, device=x.device) if scale_fmt == "f32"
             else torch.empty((cols // 4,), dtype=torch.int32, device=x.device))
    else:
        q, s = out
    if q.device != x.device or q.dim() != 2 or q.stride(1) != 1 or q.shape[0] != rows:
        raise ValueError("codes must be 2-D, row-contiguous, on the input's device")
    if s.device != x.device or not s.is_contiguous():
        raise ValueError("scales must be contiguous on the input's device")
    _check_out_shapes(q, s, cols if out_dtype == "e4m3" else cols // 2, cols if scale_fmt == "f32" else cols // 4,
                      scale_fmt)
    need = tk_per_channel_workspace_bytes(rows, cols)
    if workspace is None:
        workspace = torch.empty((max(need, 16),), dtype=torch.uint8, device=x.device)
    ws_bytes = workspace.numel() * workspace.element_size()
    if not workspace.is_cuda or not workspace.is_contiguous():
        raise ValueError("workspace must be a contiguous GPU tensor")
    _check(tk_per_channel_cast(x.data_ptr(), rows, cols, x.stride(0), q.data_ptr(), q.stride(0), s.data_ptr(),
                               workspace.data_ptr(), ws_bytes, QDTYPES[out_dtype], int(bool(round_pow2)),
                               SCALE_FMTS[scale_fmt], _stream_handle(stream, x.device)))
    return q, s


def tk_rmsnorm(x: int, rows: int, cols: int, x_ld: int, weight: int | None, eps: float, y: int, y_ld: int,
               y_dtype: int, stream: int) -> int:
    """Raw C call with integer pointers; returns the tk_status code."""
    return load_library().tk_rmsnorm(x, rows, cols, x_ld, weight, eps, y, y_ld, y_dtype, stream)


def tk_rmsnorm_cast(x: int, rows: int, cols: int, x_ld: int, weight: int | None, eps: float, q: int, q_ld: int,
                    scales: int, s_ld: int, group: int, out_dtype: int, round_pow2: int, scale_fmt: int,
                    stream: int) -> int:
    """Raw C call with integer pointers; returns the tk_status code."""
    return load_library().tk_rmsnorm_cast(x, rows, cols, x_ld, weight, eps, q, q_ld, scales, s_ld, group, out_dtype,
                                          round_pow2, scale_fmt, stream)


def _weight(weight, x):
    if weight is None:
        return None
    if (not isinstance(weight, torch.Tensor) or weight.dtype != torch.bfloat16 or weight.dim() != 1
            or weight.shape[0] != x.shape[1] or not weight.is_contiguous() or weight.device != x.device):
        raise TypeError("weight must be a contiguous 1-D bf16 tensor of x.shape[1] on x's device")
    return weight.data_ptr()


def rmsnorm(x: torch.Tensor, weight: torch.Tensor | None = None, eps: float = 1e-6, out_dtype: str = "bf16",
            out=None, stream=None) -> torch.Tensor:
    """RMSNorm forward of bf16 x [rows, cols] -> y in bf16 or fp32."""
    _check_input(x, "x")
    rows, cols = x.shape
    ydt = torch.bfloat16 if out_dtype == "bf16" else torch.float32
    y = torch.empty((rows, cols), dtype=ydt, device=x.device) if out is None else out
    if y.dtype != ydt or y.dim() != 2 or y.stride(1) != 1 or tuple(y.shape) != (rows, cols) or y.device != x.device:
        raise ValueError("out must be a row-contiguous tensor of x's shape and the output dtype")
    _check(tk_rmsnorm(x.data_ptr(), rows, cols, x.stride(0), _weight(weight, x), float(eps), y.data_ptr(),
                      y.stride(0), OUT_DTYPES[out_dtype], _stream_handle(stream, x.device)))
    return y


def rmsnorm_cast(x: torch.Tensor, weight: torch.Tensor | None = None, eps: float = 1e-6, group: int = 128,
                 out_dtype: str = "e4m3", round_pow2: bool = False, scale_fmt: str = "f32", out=None, stream=None):
    """RMSNorm forward fused with the per-token cast -> (codes, scales)."""
    _check_input(x, "x")
    wp = _weight(weight, x)

    def fn(xp, rows, cols, x_ld, q, q_ld, s, s_ld, g, dt, p2, sf, st):
        return tk_rmsnorm_cast(xp, rows, cols, x_ld, wp, float(eps), q, q_ld, s, s_ld, g, dt, p2, sf, st)
    return _run(fn, x, x.shape[1], group, out_dtype, round_pow2, scale_fmt, out, stream)
