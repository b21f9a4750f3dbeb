"""The Python binding refuses caller-given tensors that cannot hold what a call
reads or writes (the C ABI sees only pointers and strides, so extents are
checked here); nothing is launched for a refused call."""
from __future__ import annotations

import pytest
import torch

import activation_quantization_token_amd as tk

pytestmark = pytest.mark.gpu

ROWS, COLS = 8, 256


def _x():
    return torch.zeros((ROWS, COLS), dtype=torch.bfloat16, device="cuda")


def _u8(r, c):
    return torch.zeros((r, c), dtype=torch.uint8, device="cuda")


@pytest.mark.parametrize("q,s,err", [
    (lambda: _u8(ROWS, COLS - 16), lambda: torch.zeros((ROWS, 2), device="cuda"), ValueError),      # narrow codes
    (lambda: _u8(ROWS, COLS), lambda: torch.zeros((ROWS, 1), device="cuda"), ValueError),           # narrow scales
    (lambda: _u8(ROWS, COLS), lambda: torch.zeros((ROWS, 2), dtype=torch.int32, device="cuda"), TypeError),
    (lambda: torch.zeros((ROWS, COLS), dtype=torch.int8, device="cuda"),
     lambda: torch.zeros((ROWS, 2), device="cuda"), TypeError),
    (lambda: _u8(ROWS - 1, COLS), lambda: torch.zeros((ROWS, 2), device="cuda"), ValueError),
])
def test_per_token_cast_rejects_bad_outputs(q, s, err):
    with pytest.raises(err):
        tk.per_token_cast(_x(), 128, "e4m3", False, "f32", out=(q(), s()))


def test_per_token_cast_rejects_narrow_ue8m0_scales():
    q = _u8(ROWS, COLS // 2)
    s = torch.zeros((ROWS, 1), dtype=torch.int32, device="cuda")        # 256/32/4 = 2 words needed
    with pytest.raises(ValueError):
        tk.per_token_cast(_x(), 32, "e2m1", True, "ue8m0", out=(q, s))


def test_per_block_and_channel_reject_bad_outputs():
    x = _x()
    with pytest.raises(ValueError):
        tk.per_block_cast(x, 4, 128, "e4m3", False, "f32",
                          out=(_u8(ROWS, COLS), torch.zeros((ROWS // 4, 1), device="cuda")))
    with pytest.raises(TypeError):
        tk.per_block_cast(x, 4, 128, "e4m3", True, "ue8m0",
                          out=(_u8(ROWS, COLS), torch.zeros((ROWS // 4, 2), device="cuda")))
    with pytest.raises(ValueError):
        tk.per_channel_cast(x, "e4m3", False, "f32", out=(_u8(ROWS, COLS), torch.zeros((COLS - 8,), device="cuda")))
    with pytest.raises(ValueError):
        tk.per_channel_cast(x, "e2m1", False, "f32", out=(_u8(ROWS, COLS // 2 - 4), torch.zeros((COLS,), device="cuda")))


def test_dequant_rejects_bad_operands():
    q, s = tk.per_token_cast(_x(), 32, "e4m3", False, "f32")
    with pytest.raises(ValueError):                                   # codes narrower than cols
        tk.per_token_dequant(q[:, :COLS - 32], s, COLS, 32, "e4m3", "f32")
    with pytest.raises(ValueError):                                   # scales narrower than cols / group
        tk.per_token_dequant(q, s[:, :4], COLS, 32, "e4m3", "f32")
    with pytest.raises(ValueError):                                   # scales with other rows
        tk.per_token_dequant(q, s[:ROWS - 1], COLS, 32, "e4m3", "f32")
    with pytest.raises(TypeError):                                    # int32 scales under scale_fmt f32
        tk.per_token_dequant(q, s.view(torch.int32), COLS, 32, "e4m3", "f32")
    with pytest.raises(ValueError):                                   # output narrower than cols
        tk.per_token_dequant(q, s, COLS, 32, "e4m3", "f32",
                             out=torch.empty((ROWS, COLS - 32), dtype=torch.bfloat16, device="cuda"))
    with pytest.raises(ValueError):
        tk.per_token_dequant(q, s, COLS, 32, "e5m2", "f32")


def test_cast_back_rejects_bad_output():
    with pytest.raises(ValueError):
        tk.per_token_cast_back(_x(), 32, "e4m3", True, out=torch.empty((ROWS, COLS), dtype=torch.float32,
                                                                          device="cuda"))
    with pytest.raises(ValueError):
        tk.per_token_cast_back(_x(), 32, "e5m2", True)
