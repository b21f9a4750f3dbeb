"""GPU parity of dequantization and the fused cast-and-cast-back against the
CPU oracle (bit for bit)."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
import activation_quantization_token_amd as tk
from activation_quantization_token_amd import inputs
from gpu_util import Guarded, first_mismatch, log, oracle_cast, to_dev

pytestmark = pytest.mark.gpu


def _dev_bytes(a: np.ndarray, dtype) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a)).view(dtype).to("cuda")


def check_dequant(x_bits, group, dt, p2, sf, out, label=""):
    rows, cols = x_bits.shape
    log(f"[gpu] dequant {label} rows={rows} cols={cols} G={group} {dt} pow2={p2} {sf} -> {out}")
    q, s = oracle_cast(x_bits, group, dt, p2, sf)
    want = oracle.per_token_dequant(q, s, cols, group, dt, sf, out)
    qd = _dev_bytes(q, torch.uint8)
    sd = _dev_bytes(s, torch.float32 if sf == "f32" else torch.int32)
    ydt = torch.bfloat16 if out == "bf16" else torch.float32
    g = Guarded(rows, cols, ydt, 8)
    tk.per_token_dequant(qd, sd, cols, group, dt, sf, out, out=g.view)
    torch.cuda.synchronize()
    got = g.view.cpu()
    got = got.view(torch.int16).numpy().view(np.uint16) if out == "bf16" else got.numpy().view(np.uint32)
    assert g.canaries_intact(), "write outside the output view"
    assert np.array_equal(got, want.view(np.uint16 if out == "bf16" else np.uint32)), first_mismatch(
        got, want.view(got.dtype))


def check_cast_back(x_bits, group, dt, p2, x_ld=None, guard=True, label=""):
    rows, cols = x_bits.shape
    log(f"[gpu] cast-back {label} rows={rows} cols={cols} G={group} {dt} pow2={p2} x_ld={x_ld}")
    want = oracle.per_token_cast_back(x_bits, group, dt, p2) if rows < 64 else _oracle_cast_back_parallel(
        x_bits, group, dt, p2)
    x = to_dev(x_bits, x_ld)
    if guard:
        g = Guarded(rows, cols, torch.bfloat16, 8)
        tk.per_token_cast_back(x, group, dt, p2, out=g.view)
        y = g.view
    else:
        y = tk.per_token_cast_back(x, group, dt, p2)
    torch.cuda.synchronize()
    got = y.cpu().view(torch.int16).numpy().view(np.uint16)
    if guard:
        assert g.canaries_intact(), "write outside the output view"
    assert np.array_equal(got, want), first_mismatch(got, want)


def _oracle_cast_back_parallel(x_bits, group, dt, p2):
    import concurrent.futures
    import os
    threads = min(16, len(os.sched_getaffinity(0)))
    bounds = np.linspace(0, x_bits.shape[0], threads + 1).astype(int)
    with concurrent.futures.ThreadPoolExecutor(threads) as ex:
        parts = list(ex.map(lambda i: oracle.per_token_cast_back(x_bits[bounds[i]:bounds[i + 1]], group, dt, p2),
                            range(threads)))
    return np.concatenate(parts)


CASES = [(g, dt, p2, sf) for g in (16, 32, 64, 128) for dt in ("e4m3", "e2m1")
         for p2, sf in ((False, "f32"), (True, "f32"), (True, "ue8m0"))]


@pytest.mark.parametrize("group,dt,p2,sf", CASES)
@pytest.mark.parametrize("out", ["bf16", "f32"])
@pytest.mark.parametrize("rows,extra", [(3, None), (129, 512), (2, 3584)])
def test_dequant_sweep(group, dt, p2, sf, out, rows, extra):
    ncols = 7168 if extra is None else extra + 4 * group      # ragged tails, whole UE8M0 words
    x = inputs.generate_small(rows + ncols + group, rows, ncols, "student_t3")
    check_dequant(x, group, dt, p2, sf, out, label="sweep")


@pytest.mark.parametrize("group,dt", [(g, dt) for g in (16, 32, 64, 128) for dt in ("e4m3", "e2m1")])
@pytest.mark.parametrize("p2", [False, True])
@pytest.mark.parametrize("rows,cols", [(1, 512), (5, 7168), (129, 1024 + 128)])
def test_cast_back_sweep(group, dt, p2, rows, cols):
    x = inputs.generate_small(rows * 3 + cols + group, rows, cols, "normal" if rows % 2 else "student_t3")
    check_cast_back(x, group, dt, p2, x_ld=cols + 8 * (1 + rows % 2), label="sweep")


@pytest.mark.parametrize("w", [inputs.WORKLOADS[i] for i in (0, 1, 2, 4)], ids=lambda w: f"workload{w.index}")
def test_cast_back_workload_full_size(w):
    x = inputs.generate(w, cache=True)
    check_cast_back(x, w.group, w.out_dtype, w.round_pow2, guard=False, label=f"workload{w.index}")


@pytest.mark.parametrize("dt", ["e4m3", "e2m1"])
def test_dequant_every_code_and_extreme_scales(dt):
    """Every code value under extreme scales (largest and smallest the cast
    produces), through the UE8M0 and fp32 paths."""
    rows, cols = 64, 512
    if dt == "e4m3":
        codes = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], dtype=np.uint8)
        q = np.resize(codes, rows * cols).reshape(rows, cols)
    else:
        q = np.resize(np.arange(256, dtype=np.uint8), rows * cols // 2).reshape(rows, cols // 2)
    group = 32
    ng = cols // group
    lo, hi = (105, 247) if dt == "e4m3" else (112, 253)
    e8 = np.linspace(lo, hi, rows * ng).round().astype(np.uint8).reshape(rows, ng)
    s_u = np.ascontiguousarray(e8).view(np.int32).reshape(rows, ng // 4)
    s_f = (e8.astype(np.uint32) << 23).view(np.float32)
    for sf, s in (("ue8m0", s_u), ("f32", s_f)):
        for out in ("bf16", "f32"):
            log(f"[gpu] dequant codes {dt} {sf} -> {out}")
            want = oracle.per_token_dequant(q, s, cols, group, dt, sf, out)
            y = tk.per_token_dequant(_dev_bytes(q, torch.uint8),
                                     _dev_bytes(s, torch.int32 if sf == "ue8m0" else torch.float32),
                                     cols, group, dt, sf, out)
            torch.cuda.synchronize()
            got = y.cpu()
            got = got.view(torch.int16).numpy().view(np.uint16) if out == "bf16" else got.numpy().view(np.uint32)
            assert np.array_equal(got, want.view(got.dtype)), first_mismatch(got, want.view(got.dtype))


def test_cast_back_equals_cast_then_dequant_on_gpu():
    w = inputs.WORKLOADS[4]
    x_bits = inputs.generate(w, rows=512)
    x = to_dev(x_bits)
    log("[gpu] cast-back vs cast + dequant")
    q, s = tk.per_token_cast(x, w.group, w.out_dtype, w.round_pow2, w.scale_fmt)
    y1 = tk.per_token_dequant(q, s, w.cols, w.group, w.out_dtype, w.scale_fmt, "bf16")
    y2 = tk.per_token_cast_back(x, w.group, w.out_dtype, w.round_pow2)
    torch.cuda.synchronize()
    assert torch.equal(y1.view(torch.int16), y2.view(torch.int16))
