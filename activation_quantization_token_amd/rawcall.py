"""Extent checks for raw calls of the C ABI.

The C ABI takes bare device pointers, so a call cannot see how large the
buffers behind them are.  A kernel reaches its memory only through row
descriptors built from the call's own arguments (base + r * ld, one row's
bytes), so every byte it can touch lies in the ranges that `extents` returns:
for each pointer argument of an entry point, the bytes from that pointer that
the call reads or writes, computed from the other arguments and the layouts
written out in include/tk_quant.h.

`prepare` checks those ranges against the tensors that own the memory (each
range must lie inside its tensor's storage) and returns the function and the
argument tuple to call it with, so that timing loops can make the call again
and again without re-checking.  Callers that marshal raw calls themselves (the
benchmark, experiments) go through `prepare`; the tensor functions of the
binding check shapes instead.
"""
from __future__ import annotations

import torch

# Parameter names of each entry point, in order (include/tk_quant.h).
_CAST = ("x", "rows", "cols", "x_ld", "q", "q_ld", "scales", "s_ld", "group", "out_dtype", "round_pow2",
         "scale_fmt", "stream")
SIGNATURES = {
    "tk_per_token_cast": _CAST,
    "tk_swiglu_per_token_cast": ("gate_up",) + _CAST[1:],
    "tk_per_token_cast_f32": _CAST,
    "tk_per_token_dequant": ("q", "rows", "cols", "q_ld", "scales", "s_ld", "group", "in_dtype", "scale_fmt", "y",
                             "y_ld", "y_dtype", "stream"),
    "tk_per_token_cast_back": ("x", "rows", "cols", "x_ld", "y", "y_ld", "group", "out_dtype", "round_pow2",
                               "stream"),
    "tk_per_block_cast": ("x", "rows", "cols", "x_ld", "q", "q_ld", "scales", "s_ld", "block_rows", "block_cols",
                          "out_dtype", "round_pow2", "scale_fmt", "stream"),
    "tk_per_channel_cast": ("x", "rows", "cols", "x_ld", "q", "q_ld", "scales", "workspace", "workspace_bytes",
                            "out_dtype", "round_pow2", "scale_fmt", "stream"),
    "tk_per_channel_cast_noalloc": ("x", "rows", "cols", "x_ld", "q", "q_ld", "scales", "out_dtype", "round_pow2",
                                    "scale_fmt", "stream"),
    "tk_rmsnorm": ("x", "rows", "cols", "x_ld", "weight", "eps", "y", "y_ld", "y_dtype", "stream"),
    "tk_rmsnorm_cast": ("x", "rows", "cols", "x_ld", "weight", "eps", "q", "q_ld", "scales", "s_ld", "group",
                        "out_dtype", "round_pow2", "scale_fmt", "stream"),
    "tk_silu32_bf16": ("g", "out", "n", "stream"),
    "tk_copy_stream": ("src", "dst", "bytes", "stream"),
    "tk_stream_rw": ("src", "read_bytes", "dst", "write_bytes", "stream"),
}

E4M3, E2M1 = 0, 1
SCALE_F32 = 0
OUT_F32 = 1


def _rows_span(rows, ld, row_bytes, elt):
    """Bytes from the base pointer of a row-major matrix: rows - 1 strides of
    ld elements of `elt` bytes, then one row of `row_bytes`; 0 for no rows."""
    return 0 if rows <= 0 else (rows - 1) * ld * elt + row_bytes


def _code_bytes(cols, qd):
    return cols if qd == E4M3 else cols // 2


def _scale_words(ncols_of_scales, scale_fmt):
    """fp32 words per scale row, or int32 words of four UE8M0 bytes."""
    return ncols_of_scales if scale_fmt == SCALE_F32 else ncols_of_scales // 4


def extents(name: str, args) -> dict:
    """{pointer parameter: bytes the call covers from it} for entry point `name`
    called with `args` (positional, as the C function takes them)."""
    sig = SIGNATURES[name]
    if len(args) != len(sig):
        raise TypeError(f"{name} takes {len(sig)} arguments, got {len(args)}")
    a = dict(zip(sig, args))
    rows, cols = a.get("rows", 0), a.get("cols", 0)
    if name in ("tk_per_token_cast", "tk_swiglu_per_token_cast", "tk_per_token_cast_f32", "tk_rmsnorm_cast"):
        x = "gate_up" if name == "tk_swiglu_per_token_cast" else "x"
        in_cols = 2 * cols if x == "gate_up" else cols
        elt = 4 if name == "tk_per_token_cast_f32" else 2
        out = {x: _rows_span(rows, a["x_ld"], in_cols * elt, elt),
               "q": _rows_span(rows, a["q_ld"], _code_bytes(cols, a["out_dtype"]), 1),
               "scales": _rows_span(rows, a["s_ld"], 4 * _scale_words(cols // a["group"], a["scale_fmt"]), 4)}
        if name == "tk_rmsnorm_cast":
            out["weight"] = 2 * cols if a["weight"] else 0
        return out
    if name == "tk_per_token_dequant":
        ysize = 4 if a["y_dtype"] == OUT_F32 else 2
        return {"q": _rows_span(rows, a["q_ld"], _code_bytes(cols, a["in_dtype"]), 1),
                "scales": _rows_span(rows, a["s_ld"], 4 * _scale_words(cols // a["group"], a["scale_fmt"]), 4),
                "y": _rows_span(rows, a["y_ld"], cols * ysize, ysize)}
    if name == "tk_per_token_cast_back":
        return {"x": _rows_span(rows, a["x_ld"], 2 * cols, 2), "y": _rows_span(rows, a["y_ld"], 2 * cols, 2)}
    if name == "tk_per_block_cast":
        nbr = -(-rows // a["block_rows"]) if a["block_rows"] > 0 else 0
        return {"x": _rows_span(rows, a["x_ld"], 2 * cols, 2),
                "q": _rows_span(rows, a["q_ld"], _code_bytes(cols, a["out_dtype"]), 1),
                "scales": _rows_span(nbr, a["s_ld"], 4 * _scale_words(cols // a["block_cols"], a["scale_fmt"]), 4)}
    if name in ("tk_per_channel_cast", "tk_per_channel_cast_noalloc"):
        out = {"x": _rows_span(rows, a["x_ld"], 2 * cols, 2),
               "q": _rows_span(rows, a["q_ld"], _code_bytes(cols, a["out_dtype"]), 1),
               "scales": 0 if rows <= 0 else 4 * _scale_words(cols, a["scale_fmt"])}
        if name == "tk_per_channel_cast":
            out["workspace"] = a["workspace_bytes"]
        return out
    if name == "tk_rmsnorm":
        ysize = 4 if a["y_dtype"] == OUT_F32 else 2
        return {"x": _rows_span(rows, a["x_ld"], 2 * cols, 2), "weight": 2 * cols if a["weight"] else 0,
                "y": _rows_span(rows, a["y_ld"], cols * ysize, ysize)}
    if name == "tk_silu32_bf16":
        return {"g": 2 * a["n"], "out": 4 * a["n"]}
    if name == "tk_copy_stream":
        return {"src": a["bytes"], "dst": a["bytes"]}
    if name == "tk_stream_rw":
        return {"src": a["read_bytes"], "dst": a["write_bytes"]}
    raise KeyError(name)


def check(name: str, args, buffers: dict) -> None:
    """Raise ValueError unless every pointer argument that covers any bytes is
    owned by the tensor given for it in `buffers` (by parameter name) and the
    covered range lies inside that tensor's storage."""
    sig = SIGNATURES[name]
    a = dict(zip(sig, args))
    for param, nbytes in extents(name, args).items():
        if nbytes <= 0:
            continue
        if param not in buffers:
            raise ValueError(f"{name}: no tensor given for pointer argument {param!r} ({nbytes} bytes)")
        t = buffers[param]
        if not isinstance(t, torch.Tensor):
            raise TypeError(f"{name}: buffer for {param!r} must be a tensor")
        st = t.untyped_storage()
        lo, hi = st.data_ptr(), st.data_ptr() + st.nbytes()
        p = int(a[param] or 0)
        if not lo <= p <= hi:
            raise ValueError(f"{name}: {param!r} = {p:#x} is not inside its tensor's storage [{lo:#x}, {hi:#x})")
        if p + nbytes > hi:
            raise ValueError(f"{name}: {param!r} covers {nbytes} bytes from {p:#x}, {p + nbytes - hi} past the end "
                             f"of its tensor's storage ({st.nbytes()} bytes)")


def prepare(lib, name: str, args, buffers: dict):
    """check() the call, then return (C function, argument tuple)."""
    args = tuple(args)
    check(name, args, buffers)
    return getattr(lib, name), args
