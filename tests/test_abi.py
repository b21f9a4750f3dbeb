"""The C-ABI library loads, exports every declared entry point, and validates
arguments on the host (CPU only: nothing here reaches the GPU runtime)."""
from __future__ import annotations

import ctypes
import os
import re

import pytest

import activation_quantization_token_amd as tk
from activation_quantization_token_amd import binding

HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include", "tk_quant.h")

INVALID, UNSUPPORTED, MISALIGNED = 1, 2, 3


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(tk_[a-z0-9_]+)\s*\(", text)))


def test_header_declares_the_entry_points():
    names = declared_functions()
    for n in ("tk_per_token_cast", "tk_swiglu_per_token_cast", "tk_status_string", "tk_abi_version",
              "tk_prepare_device", "tk_silu32_bf16", "tk_copy_stream", "tk_per_token_dequant",
              "tk_per_token_cast_back", "tk_per_token_cast_f32", "tk_per_block_cast", "tk_per_channel_cast",
              "tk_per_channel_workspace_bytes", "tk_rmsnorm", "tk_rmsnorm_cast", "tk_stream_rw"):
        assert n in names


def test_library_exports_every_declared_symbol():
    lib = tk.load_library()
    for name in declared_functions():
        assert hasattr(lib, name), f"{name} declared in tk_quant.h but not exported"
    # exported with C linkage, i.e. unmangled
    raw = ctypes.CDLL(str(binding.LIB_PATH))
    for name in declared_functions():
        ctypes.cast(getattr(raw, name), ctypes.c_void_p)


def test_abi_version_and_status_strings():
    assert tk.tk_abi_version() == 1
    assert tk.tk_status_string(0) == "TK_SUCCESS"
    for st in range(1, 6):
        assert tk.tk_status_string(st).startswith("TK_ERROR_")
    assert tk.tk_status_string(99) == "TK_ERROR_UNKNOWN"


# Fake, suitably aligned device addresses: validation must reject before any
# pointer is used, and a successful rows == 0 call must not touch them.
X, Q, S = 0x10000, 0x20000, 0x30000


def call(fn=tk.tk_per_token_cast, x=X, rows=4, cols=256, x_ld=None, q=Q, q_ld=None, s=S, s_ld=None,
         group=32, out_dtype=0, round_pow2=1, scale_fmt=0, swiglu=False):
    in_cols = 2 * cols if swiglu else cols
    x_ld = in_cols if x_ld is None else x_ld
    q_ld = (cols if out_dtype == 0 else cols // 2) if q_ld is None else q_ld
    if s_ld is None:
        g = group if group > 0 else 32
        s_ld = max(cols // g, 1) if scale_fmt == 0 else max(cols // g // 4, 1)
    return fn(x, rows, cols, x_ld, q, q_ld, s, s_ld, group, out_dtype, round_pow2, scale_fmt, 0)


@pytest.mark.parametrize("fn,swiglu", [(tk.tk_per_token_cast, False), (tk.tk_swiglu_per_token_cast, True)])
@pytest.mark.parametrize("kw,want", [
    (dict(group=48), INVALID),
    (dict(group=0), INVALID),
    (dict(group=256), INVALID),
    (dict(cols=200), INVALID),                       # not a multiple of the group
    (dict(cols=0), INVALID),
    (dict(cols=-32), INVALID),
    (dict(rows=-1), INVALID),
    (dict(out_dtype=2), INVALID),
    (dict(scale_fmt=2), INVALID),
    (dict(scale_fmt=1, round_pow2=0), INVALID),      # UE8M0 holds powers of two only
    (dict(scale_fmt=1, cols=96), INVALID),           # 3 groups: not a multiple of 4
    (dict(x_ld=100), INVALID),                       # row stride below the row length
    (dict(q_ld=100), INVALID),
    (dict(s_ld=1), INVALID),
    (dict(x=0), INVALID),
    (dict(q=0), INVALID),
    (dict(s=0), INVALID),
    (dict(x=X + 8), MISALIGNED),
    (dict(q=Q + 4), MISALIGNED),
    (dict(q=Q + 2, out_dtype=1), MISALIGNED),
    (dict(s=S + 2), MISALIGNED),
    (dict(x_ld=260, cols=256), MISALIGNED),          # 520-byte rows: not 16-byte multiples
    (dict(q_ld=260), MISALIGNED),
    (dict(rows=1 << 62), INVALID),                   # spans beyond 2^52 bytes
    (dict(rows=1 << 45), INVALID),
    (dict(x_ld=1 << 61), INVALID),
    (dict(q_ld=1 << 60), INVALID),
    (dict(s_ld=1 << 60), INVALID),
])
def test_validation_errors(fn, swiglu, kw, want):
    if swiglu and "x_ld" in kw:
        kw = dict(kw, x_ld=kw["x_ld"] * 2 if want == INVALID else 2 * 256 + 4)
    assert call(fn, swiglu=swiglu, **kw) == want


@pytest.mark.parametrize("fn,swiglu", [(tk.tk_per_token_cast, False), (tk.tk_swiglu_per_token_cast, True)])
def test_zero_rows_is_a_no_op(fn, swiglu):
    # rows == 0 succeeds without touching (null) pointers or the device
    assert call(fn, rows=0, x=0, q=0, s=0, swiglu=swiglu) == 0
    assert call(fn, rows=0, x=0, q=0, s=0, x_ld=1 << 62, q_ld=1 << 62, s_ld=1 << 62, swiglu=swiglu) == 0


def test_silu_diagnostic_validation():
    assert tk.tk_silu32_bf16(X, Q, -1, 0) == INVALID
    assert tk.tk_silu32_bf16(X, Q, 0, 0) == 0
    assert tk.tk_silu32_bf16(0, Q, 5, 0) == INVALID
    assert tk.tk_silu32_bf16(X + 1, Q, 5, 0) == MISALIGNED
    assert tk.tk_silu32_bf16(X, Q + 2, 5, 0) == MISALIGNED
    assert tk.tk_silu32_bf16(X, Q, 1 << 62, 0) == INVALID
    assert tk.tk_silu32_bf16(X, Q, (1 << 63) - 1, 0) == INVALID


Y = 0x40000


@pytest.mark.parametrize("kw,want", [
    (dict(group=48), INVALID), (dict(in_dtype=2), INVALID), (dict(scale_fmt=2), INVALID),
    (dict(y_dtype=2), INVALID), (dict(cols=200), INVALID), (dict(rows=-1), INVALID),
    (dict(scale_fmt=1, cols=96), INVALID), (dict(q_ld=100), INVALID), (dict(s_ld=1), INVALID),
    (dict(y_ld=100), INVALID), (dict(q=0), INVALID), (dict(y=0), INVALID), (dict(s=0), INVALID),
    (dict(q=Q + 4), MISALIGNED), (dict(y=Y + 8), MISALIGNED), (dict(s=S + 2), MISALIGNED),
    (dict(y_ld=260), MISALIGNED), (dict(rows=0, q=0, s=0, y=0), 0),
    (dict(rows=1 << 62), INVALID), (dict(q_ld=1 << 60), INVALID), (dict(s_ld=1 << 60), INVALID),
    (dict(y_ld=1 << 60), INVALID), (dict(rows=0, q=0, s=0, y=0, q_ld=1 << 62, y_ld=1 << 62), 0),
])
def test_dequant_validation(kw, want):
    a = dict(q=Q, rows=4, cols=256, q_ld=None, s=S, s_ld=None, group=32, in_dtype=0, scale_fmt=0, y=Y,
             y_ld=None, y_dtype=0)
    a.update(kw)
    q_ld = a["q_ld"] if a["q_ld"] is not None else (a["cols"] if a["in_dtype"] != 1 else a["cols"] // 2)
    s_ld = a["s_ld"] if a["s_ld"] is not None else max(a["cols"] // 32 // (4 if a["scale_fmt"] == 1 else 1), 1)
    y_ld = a["y_ld"] if a["y_ld"] is not None else a["cols"]
    assert tk.tk_per_token_dequant(a["q"], a["rows"], a["cols"], q_ld, a["s"], s_ld, a["group"], a["in_dtype"],
                                   a["scale_fmt"], a["y"], y_ld, a["y_dtype"], 0) == want


@pytest.mark.parametrize("kw,want", [
    (dict(group=48), INVALID), (dict(out_dtype=2), INVALID), (dict(cols=200), INVALID),
    (dict(x_ld=100), INVALID), (dict(y_ld=100), INVALID), (dict(x=0), INVALID), (dict(y=0), INVALID),
    (dict(x=X + 8), MISALIGNED), (dict(y=Y + 8), MISALIGNED), (dict(y_ld=260), MISALIGNED),
    (dict(rows=0, x=0, y=0), 0),
    (dict(rows=1 << 62), INVALID), (dict(x_ld=1 << 61), INVALID), (dict(y_ld=1 << 61), INVALID),
])
def test_cast_back_validation(kw, want):
    a = dict(x=X, rows=4, cols=256, x_ld=256, y=Y, y_ld=256, group=32, out_dtype=0, round_pow2=1)
    a.update(kw)
    assert tk.tk_per_token_cast_back(a["x"], a["rows"], a["cols"], a["x_ld"], a["y"], a["y_ld"], a["group"],
                                     a["out_dtype"], a["round_pow2"], 0) == want


@pytest.mark.parametrize("kw,want", [
    (dict(group=48), INVALID), (dict(cols=200), INVALID), (dict(x_ld=100), INVALID), (dict(x=0), INVALID),
    (dict(scale_fmt=1, round_pow2=0), INVALID), (dict(x=X + 8), MISALIGNED), (dict(x_ld=258), MISALIGNED),
    (dict(q=Q + 4), MISALIGNED), (dict(rows=0, x=0, q=0, s=0), 0),
    (dict(group=16, cols=16 * 8200, x_ld=16 * 8200, q_ld=16 * 8200, s_ld=8200), UNSUPPORTED),
    (dict(rows=1 << 62), INVALID), (dict(x_ld=1 << 61), INVALID), (dict(x_ld=1 << 50), INVALID),   # 2^52 B rows
    (dict(q_ld=1 << 60), INVALID), (dict(s_ld=1 << 60), INVALID),
])
def test_cast_f32_validation(kw, want):
    a = dict(x=X, rows=4, cols=256, x_ld=256, q=Q, q_ld=256, s=S, s_ld=8, group=32, out_dtype=0, round_pow2=1,
             scale_fmt=0)
    a.update(kw)
    assert tk.tk_per_token_cast_f32(a["x"], a["rows"], a["cols"], a["x_ld"], a["q"], a["q_ld"], a["s"], a["s_ld"],
                                    a["group"], a["out_dtype"], a["round_pow2"], a["scale_fmt"], 0) == want


@pytest.mark.parametrize("kw,want", [
    (dict(block_cols=48), INVALID), (dict(block_cols=1), INVALID), (dict(block_rows=0), INVALID),
    (dict(cols=200), INVALID), (dict(out_dtype=2), INVALID), (dict(scale_fmt=2), INVALID),
    (dict(scale_fmt=1, round_pow2=0), INVALID), (dict(scale_fmt=1, cols=96), INVALID),
    (dict(x_ld=100), INVALID), (dict(q_ld=100), INVALID), (dict(s_ld=1), INVALID), (dict(rows=-1), INVALID),
    (dict(x=0), INVALID), (dict(q=0), INVALID), (dict(s=0), INVALID),
    (dict(x=X + 8), MISALIGNED), (dict(x_ld=260), MISALIGNED), (dict(q=Q + 4), MISALIGNED),
    (dict(s=S + 2), MISALIGNED), (dict(block_rows=257), UNSUPPORTED), (dict(rows=0, x=0, q=0, s=0), 0),
    (dict(rows=1 << 62), INVALID), (dict(x_ld=1 << 61), INVALID), (dict(q_ld=1 << 61), INVALID),
    (dict(s_ld=1 << 60, rows=512), INVALID),
])
def test_per_block_validation(kw, want):
    a = dict(x=X, rows=4, cols=256, x_ld=256, q=Q, q_ld=256, s=S, s_ld=8, block_rows=128, block_cols=32,
             out_dtype=0, round_pow2=1, scale_fmt=0)
    a.update(kw)
    assert tk.tk_per_block_cast(a["x"], a["rows"], a["cols"], a["x_ld"], a["q"], a["q_ld"], a["s"], a["s_ld"],
                                a["block_rows"], a["block_cols"], a["out_dtype"], a["round_pow2"], a["scale_fmt"],
                                0) == want


W = 0x50000


@pytest.mark.parametrize("kw,want", [
    (dict(cols=100), INVALID), (dict(cols=0), INVALID), (dict(rows=-1), INVALID), (dict(out_dtype=2), INVALID),
    (dict(scale_fmt=1, round_pow2=0), INVALID), (dict(x_ld=100), INVALID), (dict(q_ld=100), INVALID),
    (dict(x=0), INVALID), (dict(q=0), INVALID), (dict(s=0), INVALID), (dict(ws=0), INVALID),
    (dict(ws_bytes=16), INVALID), (dict(x=X + 8), MISALIGNED), (dict(q=Q + 4), MISALIGNED),
    (dict(s=S + 8), MISALIGNED), (dict(ws=W + 8), MISALIGNED),
    (dict(rows=0, x=0, q=0, s=0, ws=0, ws_bytes=0), 0),
    (dict(rows=1 << 62, ws_bytes=1 << 40), INVALID), (dict(x_ld=1 << 61), INVALID), (dict(q_ld=1 << 61), INVALID),
])
def test_per_channel_validation(kw, want):
    a = dict(x=X, rows=4, cols=256, x_ld=256, q=Q, q_ld=256, s=S, ws=W, ws_bytes=None, out_dtype=0, round_pow2=1,
             scale_fmt=0)
    a.update(kw)
    ws_bytes = tk.tk_per_channel_workspace_bytes(a["rows"], a["cols"]) if a["ws_bytes"] is None else a["ws_bytes"]
    assert tk.tk_per_channel_cast(a["x"], a["rows"], a["cols"], a["x_ld"], a["q"], a["q_ld"], a["s"], a["ws"],
                                  ws_bytes, a["out_dtype"], a["round_pow2"], a["scale_fmt"], 0) == want


@pytest.mark.parametrize("kw,want", [
    (dict(cols=12), INVALID), (dict(cols=0), INVALID), (dict(rows=-1), INVALID), (dict(out_dtype=2), INVALID),
    (dict(scale_fmt=1, round_pow2=0), INVALID), (dict(x_ld=100), INVALID), (dict(x=0), INVALID), (dict(s=0), INVALID),
    (dict(x=X + 8), MISALIGNED), (dict(s=S + 8), MISALIGNED),
    (dict(rows=4096, cols=16392, x_ld=16392, q_ld=16392), UNSUPPORTED),    # workspace above 1088 KiB
    (dict(rows=0, x=0, q=0, s=0), 0),
    (dict(rows=1 << 62), INVALID), (dict(x_ld=1 << 61), INVALID),
])
def test_per_channel_noalloc_validation(kw, want):
    """Checks before anything is launched (the valid calls here stop at the
    missing GPU, TK_ERROR_DEVICE, before the static workspace is looked up)."""
    a = dict(x=X, rows=4, cols=256, x_ld=256, q=Q, q_ld=256, s=S, out_dtype=0, round_pow2=1, scale_fmt=0)
    a.update(kw)
    assert binding.tk_per_channel_cast_noalloc(a["x"], a["rows"], a["cols"], a["x_ld"], a["q"], a["q_ld"], a["s"],
                                               a["out_dtype"], a["round_pow2"], a["scale_fmt"], 0) == want
    assert binding.tk_per_channel_noalloc_max_workspace_bytes() == 1088 << 10


def _ws(chunks, cols):
    """Chunk maxima (2 bytes per column and chunk) padded to 256 bytes, then
    4 bytes of scale per column."""
    return (chunks * cols * 2 + 255) // 256 * 256 + cols * 4


def test_per_channel_workspace_size():
    assert tk.tk_per_channel_workspace_bytes(0, 256) == 0
    assert tk.tk_per_channel_workspace_bytes(1, 256) == _ws(1, 256)
    # at most 32 chunks of at least 64 rows
    assert tk.tk_per_channel_workspace_bytes(64, 256) == _ws(1, 256)
    assert tk.tk_per_channel_workspace_bytes(65, 256) == _ws(2, 256)
    assert tk.tk_per_channel_workspace_bytes(4096, 7168) == _ws(32, 7168)
    assert tk.tk_per_channel_workspace_bytes(70, 8) == 256 + 32            # the maxima padded to 256 bytes
    assert tk.tk_per_channel_workspace_bytes(10**6, 16) <= _ws(32, 16)
    # the largest input the allocation-free entry point takes: 32 chunks of 16384 columns
    assert tk.tk_per_channel_workspace_bytes(4096, 16384) == binding.tk_per_channel_noalloc_max_workspace_bytes()
    # sizes the cast refuses whatever the strides: no size, and no overflow
    assert tk.tk_per_channel_workspace_bytes(1 << 52, 8) == _ws(32, 8)
    assert tk.tk_per_channel_workspace_bytes((1 << 52) + 1, 8) == 0
    assert tk.tk_per_channel_workspace_bytes((1 << 63) - 1, 8) == 0
    assert tk.tk_per_channel_workspace_bytes(64, 1 << 29) == 0
    assert tk.tk_per_channel_workspace_bytes((1 << 63) - 1, (1 << 63) - 1) == 0


@pytest.mark.parametrize("kw,want", [
    (dict(cols=100), INVALID), (dict(cols=0), INVALID), (dict(rows=-1), INVALID), (dict(x_ld=100), INVALID),
    (dict(y_ld=100), INVALID), (dict(eps=0.0), INVALID), (dict(eps=-1e-6), INVALID), (dict(eps=float("inf")), INVALID),
    (dict(eps=float("nan")), INVALID), (dict(y_dtype=2), INVALID), (dict(x=0), INVALID), (dict(y=0), INVALID),
    (dict(x=X + 8), MISALIGNED), (dict(y=Y + 8), MISALIGNED), (dict(w=W + 8), MISALIGNED), (dict(x_ld=260), MISALIGNED),
    (dict(cols=16392, x_ld=16392, y_ld=16392), UNSUPPORTED), (dict(rows=0, x=0, y=0), 0),
    (dict(rows=1 << 62), INVALID), (dict(x_ld=1 << 61), INVALID), (dict(y_ld=1 << 61), INVALID),
    (dict(y_ld=1 << 50, y_dtype=1), INVALID), (dict(rows=0, x=0, y=0, x_ld=1 << 62, y_ld=1 << 62), 0),
])
def test_rmsnorm_validation(kw, want):
    a = dict(x=X, rows=4, cols=256, x_ld=256, w=W, eps=1e-6, y=Y, y_ld=256, y_dtype=0)
    a.update(kw)
    assert tk.tk_rmsnorm(a["x"], a["rows"], a["cols"], a["x_ld"], a["w"], a["eps"], a["y"], a["y_ld"], a["y_dtype"],
                         0) == want


@pytest.mark.parametrize("kw,want", [
    (dict(group=48), INVALID), (dict(cols=200), INVALID), (dict(out_dtype=2), INVALID), (dict(scale_fmt=2), INVALID),
    (dict(scale_fmt=1, round_pow2=0), INVALID), (dict(scale_fmt=1, cols=96), INVALID), (dict(q_ld=100), INVALID),
    (dict(s_ld=1), INVALID), (dict(eps=0.0), INVALID), (dict(x=0), INVALID), (dict(q=0), INVALID),
    (dict(s=0), INVALID), (dict(x=X + 8), MISALIGNED), (dict(q=Q + 4), MISALIGNED), (dict(s=S + 2), MISALIGNED),
    (dict(w=W + 8), MISALIGNED), (dict(cols=16384 + 128, x_ld=16512, q_ld=16512, s_ld=516), UNSUPPORTED),
    (dict(rows=0, x=0, q=0, s=0), 0),
    (dict(rows=1 << 62), INVALID), (dict(x_ld=1 << 61), INVALID), (dict(q_ld=1 << 61), INVALID),
    (dict(s_ld=1 << 60), INVALID),
])
def test_rmsnorm_cast_validation(kw, want):
    a = dict(x=X, rows=4, cols=256, x_ld=256, w=W, eps=1e-6, q=Q, q_ld=256, s=S, s_ld=8, group=32, out_dtype=0,
             round_pow2=1, scale_fmt=0)
    a.update(kw)
    assert tk.tk_rmsnorm_cast(a["x"], a["rows"], a["cols"], a["x_ld"], a["w"], a["eps"], a["q"], a["q_ld"], a["s"],
                              a["s_ld"], a["group"], a["out_dtype"], a["round_pow2"], a["scale_fmt"], 0) == want


def test_copy_stream_validation():
    assert tk.tk_copy_stream(X, Q, -16, 0) == INVALID
    assert tk.tk_copy_stream(X, Q, 24, 0) == INVALID
    assert tk.tk_copy_stream(X, Q, 0, 0) == 0
    assert tk.tk_copy_stream(0, Q, 32, 0) == INVALID
    assert tk.tk_copy_stream(X + 8, Q, 32, 0) == MISALIGNED


def test_stream_rw_validation():
    assert tk.tk_stream_rw(X, -16, Q, 0, 0) == INVALID
    assert tk.tk_stream_rw(X, 24, Q, 0, 0) == INVALID
    assert tk.tk_stream_rw(X, 32, Q, 0, 0) == INVALID           # one stream empty
    assert tk.tk_stream_rw(X, 0, Q, 0, 0) == 0
    assert tk.tk_stream_rw(0, 32, Q, 16, 0) == INVALID
    assert tk.tk_stream_rw(X + 8, 32, Q, 16, 0) == MISALIGNED
    assert tk.tk_stream_rw(X, 1 << 35, Q, 16, 0) == UNSUPPORTED


def test_binding_rejects_cpu_tensors():
    import torch
    x = torch.zeros(2, 64, dtype=torch.bfloat16)
    with pytest.raises(TypeError):
        tk.per_token_cast(x, 32)
    with pytest.raises(TypeError):
        tk.per_token_cast(x.float(), 32)


def test_header_is_plain_c_and_links():
    """include/tk_quant.h compiles as C11 and every call the C driver makes
    links against the built library (the driver runs in the GPU tests)."""
    import importlib.util
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "c", "build_check.py")
    spec = importlib.util.spec_from_file_location("c_abi_build", path)
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    assert mod.build().exists()


def test_missing_library_fails_loudly(tmp_path):
    with pytest.raises(RuntimeError, match="not built"):
        binding.load_library(tmp_path / "libtk_quant.so")
