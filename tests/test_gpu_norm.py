"""GPU parity of RMSNorm forward and RMSNorm + per-token cast against the CPU
oracle (y bit for bit in fp32 and bf16; codes and scales bit for bit)."""
from __future__ import annotations

import concurrent.futures
import os

import numpy as np
import pytest
import torch

import oracle
import activation_quantization_token_amd as tk
from activation_quantization_token_amd import inputs
from gpu_util import Guarded, first_mismatch, log, to_dev

pytestmark = pytest.mark.gpu

THREADS = min(16, len(os.sched_getaffinity(0)))
VARIANTS = [("e4m3", False, "f32"), ("e4m3", True, "f32"), ("e4m3", True, "ue8m0"),
            ("e2m1", False, "f32"), ("e2m1", True, "f32"), ("e2m1", True, "ue8m0")]


def _rows_parallel(fn, x_bits):
    rows = x_bits.shape[0]
    if rows < 64:
        return fn(x_bits)
    cuts = np.linspace(0, rows, THREADS + 1).astype(int)
    with concurrent.futures.ThreadPoolExecutor(THREADS) as ex:
        parts = list(ex.map(lambda i: fn(x_bits[cuts[i]:cuts[i + 1]]), range(THREADS)))
    if isinstance(parts[0], tuple):
        return tuple(np.concatenate([p[k] for p in parts]) for k in range(len(parts[0])))
    return np.concatenate(parts)


def _weight(seed, cols):
    return inputs.generate_small(seed, 1, cols, "normal")[0]


def _wdev(w_bits):
    if w_bits is None:
        return None
    return torch.from_numpy(w_bits.view(np.int16)).view(torch.bfloat16).cuda()


def check_norm(x_bits, w_bits, eps, out, x_ld=None, label=""):
    rows, cols = x_bits.shape
    log(f"[gpu] rmsnorm {label} rows={rows} cols={cols} weight={w_bits is not None} eps={eps} out={out} x_ld={x_ld}")
    want = _rows_parallel(lambda xb: oracle.rmsnorm(xb, w_bits, eps, out), x_bits)
    ydt = torch.bfloat16 if out == "bf16" else torch.float32
    g = Guarded(rows, cols, ydt, 8)
    tk.rmsnorm(to_dev(x_bits, x_ld), _wdev(w_bits), eps, out, out=g.view)
    torch.cuda.synchronize()
    got = g.view.cpu()
    got = got.view(torch.int16).numpy().view(np.uint16) if out == "bf16" else got.numpy().view(np.uint32)
    assert g.canaries_intact(), "write outside the output view"
    assert np.array_equal(got, want.view(got.dtype)), first_mismatch(got, want.view(got.dtype))


def check_norm_cast(x_bits, w_bits, eps, group, dt, p2, sf, x_ld=None, label=""):
    rows, cols = x_bits.shape
    log(f"[gpu] rmsnorm-cast {label} rows={rows} cols={cols} G={group} {dt} pow2={p2} {sf} "
        f"weight={w_bits is not None} x_ld={x_ld}")
    want_q, want_s = _rows_parallel(lambda xb: oracle.rmsnorm_cast(xb, w_bits, eps, group, dt, p2, sf), x_bits)
    gq = Guarded(rows, want_q.shape[1], torch.uint8, 16)
    gs = Guarded(rows, want_s.shape[1], torch.float32 if sf == "f32" else torch.int32, 4)
    tk.rmsnorm_cast(to_dev(x_bits, x_ld), _wdev(w_bits), eps, group, dt, p2, sf, out=(gq.view, gs.view))
    torch.cuda.synchronize()
    got_q = gq.view.cpu().numpy()
    got_s = gs.view.cpu().numpy().view(np.uint32)
    assert gq.canaries_intact() and gs.canaries_intact(), "write outside the outputs"
    assert np.array_equal(got_s, want_s.view(np.uint32)), first_mismatch(got_s, want_s.view(np.uint32))
    assert np.array_equal(got_q, want_q), first_mismatch(got_q, want_q)


@pytest.mark.parametrize("out", ["f32", "bf16"])
@pytest.mark.parametrize("weighted", [False, True])
@pytest.mark.parametrize("rows,cols", [(1, 8), (3, 520), (67, 1024), (4, 2048), (3, 2056), (5, 4096), (2, 4104),
                                       (5, 7168), (9, 7176), (2, 16384)])
def test_rmsnorm_sweep(out, weighted, rows, cols):
    x = inputs.generate_small(rows + cols, rows, cols, "student_t3" if rows % 2 else "normal")
    w = _weight(cols, cols) if weighted else None
    check_norm(x, w, 1e-6, out, x_ld=cols + 8 * (rows % 3), label="sweep")


@pytest.mark.parametrize("dt,p2,sf", VARIANTS)
@pytest.mark.parametrize("group", [16, 32, 64, 128])
@pytest.mark.parametrize("rows,extra", [(3, 0), (40, 1)])
def test_rmsnorm_cast_sweep(dt, p2, sf, group, rows, extra):
    cols = 7168 if extra == 0 else 1024 + 4 * group
    x = inputs.generate_small(rows + group, rows, cols, "student_t3")
    check_norm_cast(x, _weight(group, cols), 1e-6, group, dt, p2, sf, x_ld=cols + 16, label="sweep")


def _ambiguous_rows(cols: int) -> list:
    """Rows whose fp64 sum of squares cannot be certified (exact path)."""
    def row(entries):
        r = np.zeros(cols, dtype=np.float32)
        for c, v in entries:
            r[c % cols] = v
        return r
    return [
        row([(cols - 3, 1.0), (17, 2.0 ** -12)]),                              # exact tie -> even
        row([(cols // 2, 1.0), (5, 2.0 ** -12), (cols - 1, 2.0 ** -40)]),      # just past the tie
        row([(0, 2.0 ** -75), (cols - 9, 2.0 ** -100)]),                       # subnormal, past the tie
        row([(1, 2.0 ** -75)]),                                                # subnormal tie -> 0
        row([(3, 1.0 + 2.0 ** -7), (cols - 2, 2.0 ** -12)]),
        row([(c, 2.0 ** 63) for c in (0, 9, 700, cols - 1)]),                  # overflow to inf
        row([(2, 2.0 ** 63), (cols - 5, 2.0 ** 63)]),                          # 2^127, finite
        row([(4, 1.5 * 2.0 ** 63), (cols - 7, 2.0 ** 20)]),                    # in [2^127, 2^128)
        row([(6, 2.0 ** -64), (cols - 1, 2.0 ** -70)]),                        # below 2^-126
    ]


@pytest.mark.parametrize("cols", [1024, 7168, 16384])
def test_rmsnorm_exact_path_rows(cols):
    """Rows built on and next to rounding midpoints of the sum of squares,
    interleaved with ordinary rows."""
    special = np.stack(_ambiguous_rows(cols))
    bits = (special.view(np.uint32) >> 16).astype(np.uint16)
    ordinary = inputs.generate_small(cols, 30, cols, "student_t3")
    x = np.concatenate([ordinary[:10], bits, ordinary[10:], bits[::-1]])
    for out in ("f32", "bf16"):
        check_norm(x, _weight(1, cols), 1e-6, out, label="exact path")
    check_norm_cast(x, None, 1e-6, 128, "e4m3", True, "ue8m0", label="exact path")


def _wave_rows():
    """A row count to place test rows around (16 waves per compute unit)."""
    return torch.cuda.get_device_properties(0).multi_processor_count * 16


def _looped_input(cols, seed, n=None):
    """A tall input (2 n + 7 rows; n = 4096 on 256 CUs, the row count of 16
    waves per CU, by default) with exact-path rows placed at its start, middle
    and end and around multiples of n."""
    n = _wave_rows() if n is None else n
    rows = 2 * n + 7
    x = inputs.generate_small(seed, rows, cols, "student_t3")
    special = (np.stack(_ambiguous_rows(cols)).view(np.uint32) >> 16).astype(np.uint16)
    at = [1, n - 1, n, n + 2, 2 * n - 1, 2 * n, 2 * n + 3, 2 * n + 6, n // 2]
    for i, r in enumerate(at):
        x[r] = special[i % len(special)]
    return x


@pytest.mark.parametrize("dt,p2,sf", VARIANTS)
@pytest.mark.parametrize("group", [16, 32, 64, 128])
def test_rmsnorm_cast_tall_inputs(dt, p2, sf, group):
    """Tall inputs (thousands of workgroups, rows of 1088 to 1536 channels)
    with exact-path rows among them."""
    cols = 1024 + 4 * group
    x = _looped_input(cols, 11 + group)
    check_norm_cast(x, _weight(group, cols), 1e-6, group, dt, p2, sf, x_ld=cols + 8, label="tall")


@pytest.mark.parametrize("cols,group,dt,p2,sf", [(7168, 128, "e4m3", True, "f32"), (7168, 32, "e2m1", True, "ue8m0"),
                                                 (4096, 64, "e4m3", True, "ue8m0"), (3584, 16, "e2m1", False, "f32")])
def test_rmsnorm_cast_tall_inputs_wide(cols, group, dt, p2, sf):
    x = _looped_input(cols, 5)
    check_norm_cast(x, _weight(1, cols), 1e-6, group, dt, p2, sf, label="tall")


@pytest.mark.parametrize("cols", [9216, 16384])
def test_rmsnorm_workgroup_kernel_loops_over_rows(cols):
    """Rows wider than 7168 channels take the persistent workgroup-per-row
    kernel, whose grid holds 32 waves per CU (cols / 1024 waves a workgroup)
    and whose workgroups prefetch their next row: twice its grid of rows and
    7 more, with exact-path rows at the grid's multiples."""
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    grid = cus * max(1, 32 // (cols // 1024))
    x = _looped_input(cols, 13, n=grid)
    check_norm_cast(x, _weight(3, cols), 1e-6, 64, "e2m1", True, "ue8m0", label="workgroup kernel, tall")
    check_norm(x, _weight(3, cols), 1e-6, "bf16", label="workgroup kernel, tall")


def _one_round_rows():
    """Row counts around the band where rows of 4097..7168 channels run in
    8-wave workgroups: more than three and at most four of the 16 wave slots
    of every CU (3072 < rows <= 4096 on 256 CUs), plus both edges."""
    slots = torch.cuda.get_device_properties(0).multi_processor_count * 16
    return [3 * slots // 4, 3 * slots // 4 + 1, slots - 3, slots, slots + 1]


@pytest.mark.parametrize("cols", [7168, 4224])
@pytest.mark.parametrize("at", range(5))
def test_rmsnorm_one_round_workgroup_sizes(cols, at):
    """Both workgroup sizes of the one-wave-per-row kernel, on either side of
    the band's edges (ragged last workgroups included), fused cast and plain
    forward, with a strided input."""
    rows = _one_round_rows()[at]
    x = inputs.generate_small(40 + at, rows, cols, "student_t3")
    w = _weight(7, cols)
    if cols == 7168:
        check_norm_cast(x, w, 1e-6, 128, "e4m3", True, "f32", label=f"one round, {rows} rows")
        check_norm(x, w, 1e-6, "bf16", x_ld=cols + 8, label=f"one round, {rows} rows")
    else:
        check_norm_cast(x, w, 1e-5, 32, "e2m1", True, "ue8m0", x_ld=cols + 8, label=f"one round, {rows} rows")
        check_norm(x, None, 1e-6, "f32", label=f"one round, {rows} rows")


@pytest.mark.parametrize("out", ["f32", "bf16"])
@pytest.mark.parametrize("cols", [1024, 3584, 7168])
def test_rmsnorm_tall_inputs(out, cols):
    x = _looped_input(cols, 3)
    check_norm(x, _weight(2, cols), 1e-6, out, x_ld=cols + 8, label="tall")


@pytest.mark.parametrize("wi", [2, 4])
def test_rmsnorm_cast_full_size_sampled(wi):
    """Full-size workloads (16384 and 32768 rows), as the benchmark launches
    them; the oracle checks a sample of rows (each row is independent): the
    first and last rows, those around multiples of 4096, and every 97th."""
    w = inputs.WORKLOADS[wi]
    x = inputs.generate(w, cache=True)
    wt = _weight(7, w.cols)
    log(f"[gpu] rmsnorm-cast full size {w.rows}x{w.cols} G={w.group} {w.out_dtype} {w.scale_fmt}")
    q, s = tk.rmsnorm_cast(to_dev(x), _wdev(wt), 1e-6, w.group, w.out_dtype, w.round_pow2, w.scale_fmt)
    torch.cuda.synchronize()
    n = _wave_rows()
    pick = set(range(8)) | set(range(w.rows - 8, w.rows)) | set(range(0, w.rows, 97))
    for k in range(1, w.rows // n + 1):
        pick |= {r for r in range(k * n - 3, k * n + 3) if 0 <= r < w.rows}
    idx = np.array(sorted(pick))
    want_q, want_s = _rows_parallel(
        lambda xb: oracle.rmsnorm_cast(xb, wt, 1e-6, w.group, w.out_dtype, w.round_pow2, w.scale_fmt), x[idx])
    got_q = q.cpu().numpy()[idx]
    got_s = s.cpu().numpy().view(np.uint32)[idx]
    assert np.array_equal(got_s, want_s.view(np.uint32)), first_mismatch(got_s, want_s.view(np.uint32))
    assert np.array_equal(got_q, want_q), first_mismatch(got_q, want_q)


def test_rmsnorm_zero_rows_and_large_eps():
    x = inputs.generate_small(4, 20, 7168, "normal")
    x[3] = 0
    x[7, 1::2] = 0x8000
    x[7, 0::2] = 0
    for eps in (1e-6, 0.25, 3.0):
        check_norm(x, None, eps, "f32", label=f"eps {eps}")


@pytest.mark.parametrize("dt,p2,sf,group", [("e4m3", True, "f32", 128), ("e2m1", True, "ue8m0", 32)])
def test_rmsnorm_cast_full_size(dt, p2, sf, group):
    w = inputs.WORKLOADS[1]
    x = inputs.generate(w, cache=True)
    check_norm_cast(x, _weight(7, w.cols), 1e-6, group, dt, p2, sf, label="4096x7168")


def test_rmsnorm_full_size_bf16():
    w = inputs.WORKLOADS[1]
    x = inputs.generate(w, cache=True)
    check_norm(x, _weight(7, w.cols), 1e-6, "bf16", label="4096x7168")


def test_rmsnorm_full_size_sampled_bf16():
    """32768 rows (the benchmark's plain-forward launch); a sample of rows
    checked by the oracle."""
    w = inputs.WORKLOADS[4]
    x = inputs.generate(w, cache=True)
    wt = _weight(7, w.cols)
    log(f"[gpu] rmsnorm full size {w.rows}x{w.cols} bf16")
    y = tk.rmsnorm(to_dev(x), _wdev(wt), 1e-6, "bf16")
    torch.cuda.synchronize()
    n = _wave_rows()
    pick = set(range(8)) | set(range(w.rows - 8, w.rows)) | set(range(0, w.rows, 97))
    for k in range(1, w.rows // n + 1):
        pick |= {r for r in range(k * n - 3, k * n + 3) if 0 <= r < w.rows}
    idx = np.array(sorted(pick))
    want = _rows_parallel(lambda xb: oracle.rmsnorm(xb, wt, 1e-6, "bf16"), x[idx])
    got = y.cpu().view(torch.int16).numpy().view(np.uint16)[idx]
    assert np.array_equal(got, want), first_mismatch(got, want)


def test_rmsnorm_cast_equals_cast_of_rmsnorm_output():
    """The fused kernel's codes equal the fp32-input cast of the plain
    kernel's fp32 output (both on the GPU)."""
    w = inputs.WORKLOADS[4]
    x = to_dev(inputs.generate(w, rows=1024))
    wt = _wdev(_weight(3, w.cols))
    log("[gpu] rmsnorm-cast vs rmsnorm f32 + cast_f32")
    y = tk.rmsnorm(x, wt, 1e-6, "f32")
    a = tk.per_token_cast(y, w.group, w.out_dtype, w.round_pow2, w.scale_fmt)
    b = tk.rmsnorm_cast(x, wt, 1e-6, w.group, w.out_dtype, w.round_pow2, w.scale_fmt)
    torch.cuda.synchronize()
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])


@pytest.mark.parametrize("dt,p2,sf", VARIANTS)
@pytest.mark.parametrize("cols,group", [(7168, 32), (7168, 128), (2048, 16), (16384, 64)])
def test_rmsnorm_cast_rounding_edges(dt, p2, sf, cols, group):
    """Rows on which y equals chosen bf16 values exactly (tests/norm_edges.py):
    every code value, every midpoint between codes, the subnormal codes,
    signed zeros and values that round to zero, at group scales 2^-24 .. 2^1
    and under the 1e-4 floor, through both RMSNorm kernels (one wave per row
    up to 7168 channels, a workgroup per row above)."""
    import norm_edges
    x, w = norm_edges.edge_rows(cols, group, dt)
    check_norm_cast(x, w, 1e-6, group, dt, p2, sf, label="rounding edges")
