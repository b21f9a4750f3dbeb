"""GPU parity: the HIP path (through the C ABI) against the CPU oracle.

Codes and scales must match bit for bit.  Every test prints its case before
touching the GPU.  Inputs come from the seeded generators; expected values come
only from the oracle.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
import activation_quantization_token_amd as tk
from activation_quantization_token_amd import inputs
from gpu_util import Guarded, first_mismatch, log, oracle_cast, to_dev

pytestmark = pytest.mark.gpu

FINITE_BF16 = np.array([b for b in range(65536) if (b & 0x7F80) != 0x7F80], dtype=np.uint16)


def widen(bits):
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def run_gpu(x_bits, group, dt, p2, sf, swiglu=False, x_ld=None, guard=True):
    """Run the library on bits [rows, in_cols]; returns (codes, scales, canaries_ok)."""
    rows, in_cols = x_bits.shape
    cols = in_cols // 2 if swiglu else in_cols
    x = to_dev(x_bits, x_ld)
    qcols = cols if dt == "e4m3" else cols // 2
    scols = cols // group if sf == "f32" else cols // group // 4
    if guard:
        q = Guarded(rows, qcols, torch.uint8, 24)
        s = Guarded(rows, scols, torch.float32 if sf == "f32" else torch.int32, 3)
        out = (q.view, s.view)
    else:
        out = None
    fn = tk.swiglu_per_token_cast if swiglu else tk.per_token_cast
    qq, ss = fn(x, group, dt, p2, sf, out=out)
    torch.cuda.synchronize()
    ok = q.canaries_intact() and s.canaries_intact() if guard else True
    return qq.cpu().numpy(), ss.cpu().numpy(), ok


def check(x_bits, group, dt, p2, sf, swiglu=False, x_ld=None, guard=True, label=""):
    log(f"[gpu] {label} rows={x_bits.shape[0]} in_cols={x_bits.shape[1]} G={group} {dt} pow2={p2} {sf} "
        f"swiglu={swiglu} x_ld={x_ld}")
    q, s, ok = run_gpu(x_bits, group, dt, p2, sf, swiglu, x_ld, guard)
    wq, ws = oracle_cast(x_bits, group, dt, p2, sf, swiglu)
    assert ok, "write outside the output views (canary overwritten)"
    assert np.array_equal(q, wq), "codes: " + first_mismatch(q, wq)
    assert np.array_equal(s.view(np.uint32), ws.view(np.uint32)), "scales: " + first_mismatch(
        s.view(np.uint32), ws.view(np.uint32))


# ---------------------------------------------------------------- silu32

def test_silu32_every_bf16_gate():
    log("[gpu] silu32 over all 65536 bf16 gates")
    g = torch.from_numpy(np.arange(65536, dtype=np.uint16).view(np.int16)).view(torch.bfloat16).cuda()
    got = tk.silu32_bf16(g).cpu().numpy()
    fin = FINITE_BF16.astype(np.int64)
    want = oracle.silu32(widen(FINITE_BF16))
    bad = np.nonzero(got[fin].view(np.uint32) != want.view(np.uint32))[0]
    assert bad.size == 0, f"{bad.size} gates differ, first bf16 {FINITE_BF16[bad[0]]:#06x}"


# ---------------------------------------------------------------- converters

def _characterisation_rows(dt: str, kmin=-40, kmax=40, cols=1024):
    """Groups of 16: [A_k, x_1 .. x_15] with A_k = D * 2^k (so the scale is
    exactly 2^k, with or without power-of-two rounding) and x_i running through
    every finite bf16 value with |x| <= A_k."""
    D = 448.0 if dt == "e4m3" else 6.0
    xv = widen(FINITE_BF16)
    groups = []
    for k in range(kmin, kmax + 1):
        A = np.float32(D * 2.0 ** k)
        a_bits = np.uint16(np.array([A], np.float32).view(np.uint32)[0] >> 16)
        assert widen(np.array([a_bits]))[0] == A
        xs = FINITE_BF16[np.abs(xv) <= A]
        n = -(-xs.size // 15)
        body = np.zeros(n * 15, dtype=np.uint16)
        body[:xs.size] = xs
        g = np.concatenate([np.full((n, 1), a_bits, np.uint16), body.reshape(n, 15)], axis=1)
        groups.append(g)
    g = np.concatenate(groups)
    per_row = cols // 16
    nrows = -(-g.shape[0] // per_row)
    pad = np.zeros((nrows * per_row - g.shape[0], 16), np.uint16)
    return np.concatenate([g, pad]).reshape(nrows, cols)


@pytest.mark.parametrize("dt", ["e4m3", "e2m1"])
@pytest.mark.parametrize("p2,sf", [(False, "f32"), (True, "f32"), (True, "ue8m0")])
def test_converter_all_bf16_times_scale_exponents(dt, p2, sf):
    x = _characterisation_rows(dt)
    check(x, 16, dt, p2, sf, label="characterisation")


def _division_hard_groups(dt, n_amax=400, per_amax=15, seed=17):
    """Groups [a, x1..x15] where x/s and x*(1/s) round to different codes."""
    rng = np.random.Generator(np.random.PCG64(seed))
    D = np.float32(448.0 if dt == "e4m3" else 6.0)
    xv = widen(FINITE_BF16)
    pos = FINITE_BF16[(FINITE_BF16 >= 0x3000) & (FINITE_BF16 < 0x6000)]
    amax = rng.choice(pos, n_amax, replace=False)
    a = widen(amax)
    s = (a / D).astype(np.float32)
    rows = []
    for ab, av, sv in zip(amax, a, s):
        sel = np.abs(xv) <= av
        xs = xv[sel]
        q1 = oracle.encode_e4m3(xs / sv) if dt == "e4m3" else oracle.encode_e2m1(xs / sv)
        r = (np.float32(1) / sv).astype(np.float32)
        q2 = oracle.encode_e4m3(xs * r) if dt == "e4m3" else oracle.encode_e2m1(xs * r)
        hits = FINITE_BF16[sel][q1 != q2][:per_amax]
        if hits.size:
            row = np.zeros(16, np.uint16)
            row[0] = ab
            row[1:1 + hits.size] = hits
            rows.append(row)
    g = np.stack(rows)
    n = -(-g.shape[0] // 64) * 64
    g = np.concatenate([g, np.zeros((n - g.shape[0], 16), np.uint16)])
    return g.reshape(-1, 1024)


@pytest.mark.parametrize("dt", ["e4m3", "e2m1"])
def test_plain_scale_division_hard_cases(dt):
    check(_division_hard_groups(dt), 16, dt, False, "f32", label="division-hard")


# ---------------------------------------------------------------- sweeps

VARIANTS = [(False, "f32"), (True, "f32"), (True, "ue8m0")]


def _sweep_cases():
    out = []
    for g in (16, 32, 64, 128):
        for dt in ("e4m3", "e2m1"):
            for p2, sf in VARIANTS:
                for rows, cols in [(1, g * 4), (3, 7168), (129, 512 + 4 * g), (5, 4 * g * 9), (2, 3584 + 4 * g)]:
                    out.append((g, dt, p2, sf, rows, cols))
    return out


@pytest.mark.parametrize("group,dt,p2,sf,rows,cols", _sweep_cases())
def test_cast_sweep(group, dt, p2, sf, rows, cols):
    x = inputs.generate_small(rows * 7 + cols + group, rows, cols, "student_t3" if rows % 2 else "normal")
    ld = cols + 8 * (1 + rows % 3)      # strided rows, still 16-byte aligned
    check(x, group, dt, p2, sf, x_ld=ld, label="sweep")


@pytest.mark.parametrize("group,dt,p2,sf", [(128, "e4m3", True, "f32"), (16, "e2m1", True, "ue8m0"),
                                          (32, "e4m3", False, "f32"), (64, "e2m1", True, "f32"),
                                          (32, "e2m1", True, "ue8m0"), (128, "e4m3", False, "f32")])
@pytest.mark.parametrize("rows,cols", [(1, 512), (7, 2048), (66, 1536 + 128), (3, 7168)])
def test_swiglu_sweep(group, dt, p2, sf, rows, cols):
    if cols % (4 * group) and sf == "ue8m0":
        pytest.skip("UE8M0 x4 needs a multiple of 4 groups")
    gate = inputs.generate_small(rows + cols, rows, cols)
    up = inputs.generate_small(rows + cols + 1, rows, cols, "student_t3")
    gate_up = np.concatenate([gate, up], axis=1)
    check(gate_up, group, dt, p2, sf, swiglu=True, x_ld=2 * cols + 16, label="swiglu-sweep")


@pytest.mark.parametrize("rows,cols,group,dt,p2,sf", [(2048, 2048, 128, "e4m3", True, "f32"),
                                                     (585, 7168, 32, "e2m1", True, "ue8m0"),
                                                     (2049, 2048, 128, "e4m3", True, "f32"),
                                                     (9000, 2048, 32, "e2m1", True, "ue8m0"),
                                                     (3000, 7168, 64, "e4m3", False, "f32")])
def test_swiglu_unit_sizes(rows, cols, group, dt, p2, sf):
    """Both SwiGLU unit sizes: one-segment units while rows x segments is at
    most the persistent grid's wave count (8192 on 256 CUs: 2048 x 2048 and
    585 x 7168 are such shapes), two-segment units above (2049 x 2048 and
    beyond)."""
    gate = inputs.generate_small(rows + cols + group, rows, cols)
    up = inputs.generate_small(rows + cols + group + 1, rows, cols, "student_t3")
    check(np.concatenate([gate, up], axis=1), group, dt, p2, sf, swiglu=True, label="swiglu-units")


@pytest.mark.parametrize("rows,cols,group,dt,p2,sf", [(4096, 7168, 128, "e4m3", True, "f32"),
                                                     (3000, 9728, 32, "e2m1", True, "ue8m0"),
                                                     (410, 40960, 16, "e2m1", True, "ue8m0"),
                                                     (4097, 7168, 128, "e4m3", True, "f32"),
                                                     (1000, 30720, 64, "e4m3", False, "f32"),
                                                     (2047, 7168, 32, "e4m3", True, "ue8m0")])
def test_cast_run_lengths(rows, cols, group, dt, p2, sf):
    """Both run lengths of the row-form cast.  4-segment runs for inputs of up
    to 4096 x 7168 values whose grid fills the chip's 32 x 256 wave slots (the
    first three shapes: at the boundary, a ragged last run, more runs than
    waves); 2-segment runs above that size and below that grid (the last
    three: 2047 rows of 4 runs are one wave short)."""
    x = inputs.generate_small(rows + cols + group, rows, cols, "student_t3" if rows % 2 else "normal")
    check(x, group, dt, p2, sf, label="run-lengths")


@pytest.mark.parametrize("rows,cols,group,dt,p2,sf,fp32", [
    (255, 7168, 128, "e4m3", True, "f32", False),     # under one group of 8 runs of 32 rows: own order
    (256, 7168, 128, "e4m3", True, "f32", False),     # exactly one group
    (2049, 7168, 32, "e2m1", True, "ue8m0", False),   # 8 groups and one row
    (4607, 7168, 32, "e4m3", True, "ue8m0", False),   # above 56 MiB: runs of 64 rows, a 511-row tail
    (4609, 3584, 64, "e2m1", False, "f32", False),    # 7 KiB rows: runs of 64 rows, one row over
    (1031, 7168, 16, "e4m3", True, "f32", True),      # fp32 rows: runs of 16, a 7-row tail
    (4100, 7168, 32, "e2m1", True, "ue8m0", True),    # fp32 above 56 MiB: runs of 32, a 4-row tail
])
def test_row_order_across_xcds(rows, cols, group, dt, p2, sf, fp32):
    """The row casts renumber their workgroups so that each XCD takes runs of
    consecutive rows; row counts on and around the edges of those groups,
    with guarded outputs: every row written once, and right."""
    if not fp32:
        x = inputs.generate_small(rows + cols, rows, cols, "student_t3" if rows % 2 else "normal")
        check(x, group, dt, p2, sf, label="xcd-order")
        return
    x = inputs.generate_small_f32(rows + group, rows, cols)
    log(f"[gpu] xcd-order fp32 rows={rows} cols={cols} G={group} {dt} pow2={p2} {sf}")
    q = Guarded(rows, cols if dt == "e4m3" else cols // 2, torch.uint8, 24)
    s = Guarded(rows, cols // group if sf == "f32" else cols // group // 4,
                torch.float32 if sf == "f32" else torch.int32, 3)
    tk.per_token_cast(torch.from_numpy(x).cuda(), group, dt, p2, sf, out=(q.view, s.view))
    torch.cuda.synchronize()
    wq, ws = oracle.per_token_cast_f32(x, group, dt, p2, sf)
    assert q.canaries_intact() and s.canaries_intact()
    got_q, got_s = q.view.cpu().numpy(), s.view.cpu().numpy()
    assert np.array_equal(got_q, wq), first_mismatch(got_q, wq)
    assert np.array_equal(got_s.view(np.uint32), ws.view(np.uint32))


def test_swiglu_every_gate_pattern():
    """Every finite bf16 gate appears once; the up value is 0.5 next to gates
    beyond 2^100 so that h stays finite."""
    rng = np.random.Generator(np.random.PCG64(5))
    gates = rng.permutation(FINITE_BF16).reshape(64, 1020)
    gates = np.pad(gates, ((0, 0), (0, 4)), constant_values=0x3F80)
    ups = inputs.generate_small(9, 64, 1024)
    ups[np.abs(widen(gates)) > 2.0 ** 100] = 0x3F00
    for group, dt, p2, sf in [(128, "e4m3", True, "f32"), (32, "e2m1", True, "ue8m0"),
                              (16, "e4m3", False, "f32")]:
        check(np.concatenate([gates, ups], axis=1), group, dt, p2, sf, swiglu=True, label="swiglu-gates")


# ---------------------------------------------------------------- full workloads

@pytest.mark.parametrize("w", inputs.WORKLOADS, ids=lambda w: f"workload{w.index}")
def test_workload_full_size(w):
    """The benchmark's workloads at full size, in the benchmark's launch
    configuration (the same library call), every row against the oracle."""
    log(f"[gpu] generating workload {w.index}: {w.name}")
    x = inputs.generate(w, cache=True)
    check(x, w.group, w.out_dtype, w.round_pow2, w.scale_fmt, swiglu=w.swiglu, guard=False,
          label=f"workload{w.index}")


# ---------------------------------------------------------------- edge cases

def test_zero_rows_leaves_outputs_untouched():
    log("[gpu] rows == 0")
    x = torch.zeros((0, 256), dtype=torch.bfloat16, device="cuda")
    q = torch.full((0, 256), 7, dtype=torch.uint8, device="cuda")
    s = torch.full((0, 8), 7.0, dtype=torch.float32, device="cuda")
    tk.per_token_cast(x, 32, "e4m3", False, "f32", out=(q, s))
    torch.cuda.synchronize()


def test_invalid_arguments_raise_and_launch_nothing():
    log("[gpu] invalid arguments")
    x = torch.zeros((4, 96), dtype=torch.bfloat16, device="cuda")
    q = torch.full((4, 96), 7, dtype=torch.uint8, device="cuda")
    s = torch.full((4, 1), 7, dtype=torch.int32, device="cuda")
    with pytest.raises(tk.TkError):
        tk.per_token_cast(x, 32, "e4m3", True, "ue8m0", out=(q, s))   # 3 groups: not a multiple of 4
    torch.cuda.synchronize()
    assert bool((q == 7).all()) and bool((s == 7).all())
    xm = torch.zeros((4, 64 + 4), dtype=torch.bfloat16, device="cuda")[:, 4:]   # 8-byte offset
    with pytest.raises(tk.TkError):
        tk.per_token_cast(xm, 32, "e4m3")


@pytest.mark.parametrize("dt", ["e4m3", "e2m1"])
def test_extreme_values(dt):
    """bf16 max magnitudes, subnormals, signed zeros, mixed within groups."""
    specials = np.array([0x7F7F, 0xFF7F, 0x0001, 0x8001, 0x0000, 0x8000, 0x007F, 0x807F, 0x0080,
                         0x3F80, 0xBF80, 0x7F00, 0x0100, 0x8100, 0x4000, 0xC000], dtype=np.uint16)
    rng = np.random.Generator(np.random.PCG64(3))
    rows = np.stack([rng.permutation(specials) for _ in range(256)])
    x = np.tile(rows, (1, 32))                          # 512 columns: 4 groups of 128
    x[::7, :128] = 0x8000                               # whole groups of -0.0
    x[::11, 128:256] = 0x0001                           # whole groups of the smallest subnormal
    for p2, sf in VARIANTS:
        check(x, 16, dt, p2, sf, label="extremes")
        check(x, 128, dt, p2, sf, label="extremes")


def test_many_rows_narrow():
    x = inputs.generate_small(99, 1 << 18, 64)
    check(x, 16, "e2m1", True, "ue8m0", guard=False, label="many-rows")
    check(x, 64, "e4m3", False, "f32", guard=False, label="many-rows")


def test_copy_stream_copies():
    log("[gpu] streaming copy diagnostic")
    src = torch.randint(0, 256, (3 << 20,), dtype=torch.uint8, device="cuda")
    dst = torch.zeros_like(src)
    tk.copy_stream(src, dst)
    torch.cuda.synchronize()
    assert torch.equal(src, dst)


@pytest.mark.parametrize("read_mib,write_mib", [(4, 1), (3, 3), (1, 5)])
def test_stream_rw_writes_every_unit(read_mib, write_mib):
    """The streaming-ceiling diagnostic reads its source and writes every
    16-byte unit of its destination (canaries past the end stay)."""
    log(f"[gpu] stream_rw {read_mib} MiB -> {write_mib} MiB")
    src = torch.randint(1, 2**31 - 1, (read_mib << 18,), dtype=torch.int32, device="cuda")
    n = write_mib << 18
    sentinel = -0x5A5A5A5B                      # 0xA5A5A5A5
    dst = torch.full((n + 64,), sentinel, dtype=torch.int32, device="cuda")
    tk.stream_rw(src, read_mib << 20, dst, write_mib << 20)
    torch.cuda.synchronize()
    units = dst[:n].view(-1, 4).cpu().numpy()
    untouched = np.all(units == sentinel, axis=1)
    assert np.count_nonzero(untouched) <= 1, "units left unwritten"   # equal to the sentinel only by chance
    assert bool((dst[n:] == sentinel).all().item()), "write past the end"


def test_side_stream_and_reuse():
    log("[gpu] side stream")
    x_bits = inputs.generate_small(1, 64, 7168)
    x = to_dev(x_bits)
    wq, ws = oracle_cast(x_bits, 128, "e4m3", True, "f32")
    side = torch.cuda.Stream()
    with torch.cuda.stream(side):
        outs = [tk.per_token_cast(x, 128, "e4m3", True, "f32") for _ in range(3)]
    side.synchronize()
    for q, s in outs:
        assert np.array_equal(q.cpu().numpy(), wq)
        assert np.array_equal(s.cpu().numpy(), ws)


# ---------------------------------------------------------------- SwiGLU tolerance

def test_swiglu_dequantised_within_quantisation_bound():
    """Dequantised SwiGLU codes against h computed independently in float64,
    over all 8192 rows of the SwiGLU workload as the benchmark launches it:
    |q*s - h| <= s * (half an e4m3 step at |h|/s + 1e-2 * |h|/s); also reports
    the relative L2 error."""
    w = inputs.WORKLOADS[3]
    x = inputs.generate(w, cache=True)
    log(f"[gpu] SwiGLU tolerance on all {x.shape[0]} rows of the SwiGLU workload")
    q, s, _ = run_gpu(x, w.group, w.out_dtype, w.round_pow2, w.scale_fmt, swiglu=True, guard=False)
    g = widen(x[:, :w.cols]).astype(np.float64)
    u = widen(x[:, w.cols:]).astype(np.float64)
    h = g / (1.0 + np.exp(-g)) * u
    t = torch.from_numpy(q).view(torch.float8_e4m3fn).to(torch.float32).numpy().astype(np.float64)
    sc = np.repeat(s.astype(np.float64), w.group, axis=1)
    dq = t * sc
    av = np.minimum(np.abs(h) / sc, 448.0)
    step = np.where(av < 2.0 ** -6, 2.0 ** -9, np.exp2(np.floor(np.log2(np.maximum(av, 2.0 ** -6)))) / 8)
    bound = sc * (step / 2 + 1e-2 * av) + 1e-30
    assert np.all(np.abs(dq - h) <= bound)
    rel_l2 = np.linalg.norm(dq - h) / np.linalg.norm(h)
    log(f"[gpu] SwiGLU dequantised rel-L2 error {rel_l2:.4f}")
    assert rel_l2 < 0.05


@pytest.mark.parametrize("group,dt,p2,sf,cols", [(16, "e4m3", False, "f32", 133120),
                                               (16, "e2m1", True, "ue8m0", 532480)])
def test_very_wide_rows(group, dt, p2, sf, cols):
    """Rows whose scale row exceeds the row form's LDS budget take the
    per-segment form; both must agree with the oracle."""
    x = inputs.generate_small(cols, 3, cols)
    check(x, group, dt, p2, sf, label="wide-rows")


@pytest.mark.parametrize("group,dt,p2,sf", [(g, dt, p2, sf) for g in (16, 32, 64, 128) for dt in ("e4m3", "e2m1")
                                          for p2, sf in VARIANTS])
@pytest.mark.parametrize("rows,extra", [(3, None), (129, 512), (4099, 512)])   # 4 and 2 pieces per wave
def test_fp32_input_cast(group, dt, p2, sf, rows, extra):
    cols = 7168 if extra is None else extra + 4 * group
    x = inputs.generate_small_f32(rows + group, rows, cols)
    log(f"[gpu] fp32-input cast rows={rows} cols={cols} G={group} {dt} pow2={p2} {sf}")
    ld = cols + 4 * (1 + rows % 3)
    buf = torch.full((rows, ld), float("nan"), dtype=torch.float32, device="cuda")
    buf[:, :cols] = torch.from_numpy(x).cuda()
    q = Guarded(rows, cols if dt == "e4m3" else cols // 2, torch.uint8, 24)
    s = Guarded(rows, cols // group if sf == "f32" else cols // group // 4,
                torch.float32 if sf == "f32" else torch.int32, 3)
    tk.per_token_cast(buf[:, :cols], group, dt, p2, sf, out=(q.view, s.view))
    torch.cuda.synchronize()
    wq, ws = oracle.per_token_cast_f32(x, group, dt, p2, sf)
    assert q.canaries_intact() and s.canaries_intact()
    got_q, got_s = q.view.cpu().numpy(), s.view.cpu().numpy()
    assert np.array_equal(got_q, wq), first_mismatch(got_q, wq)
    assert np.array_equal(got_s.view(np.uint32), ws.view(np.uint32))


@pytest.mark.parametrize("rows,cols,group,dt,p2,sf", [(18725, 7168, 64, "e4m3", False, "f32"),
                                                     (19001, 7168, 16, "e2m1", True, "ue8m0")])
def test_fp32_input_cast_half_rows(rows, cols, group, dt, p2, sf):
    """Above 512 MiB of fp32 input each row is cast by two workgroups, one per
    half, in XCD order over the halves; odd row counts leave a ragged last
    group.  The oracle checks the first and last 64 rows, every 37th row, and
    the rows around every 32-row boundary of the XCD runs."""
    x = inputs.generate_small_f32(rows + group, rows, cols)
    log(f"[gpu] fp32-input cast, half rows: rows={rows} cols={cols} G={group} {dt} pow2={p2} {sf}")
    q = Guarded(rows, cols if dt == "e4m3" else cols // 2, torch.uint8, 24)
    s = Guarded(rows, cols // group if sf == "f32" else cols // group // 4,
                torch.float32 if sf == "f32" else torch.int32, 3)
    tk.per_token_cast(torch.from_numpy(x).cuda(), group, dt, p2, sf, out=(q.view, s.view))
    torch.cuda.synchronize()
    assert q.canaries_intact() and s.canaries_intact()
    idx = set(range(64)) | set(range(rows - 64, rows)) | set(range(0, rows, 37))
    idx |= {r for b in range(0, rows, 32) for r in (b - 1, b) if 0 <= r < rows}
    idx = np.array(sorted(idx))
    wq, ws = oracle.per_token_cast_f32(np.ascontiguousarray(x[idx]), group, dt, p2, sf)
    got_q, got_s = q.view.cpu().numpy()[idx], s.view.cpu().numpy()[idx]
    assert np.array_equal(got_q, wq), first_mismatch(got_q, wq)
    assert np.array_equal(got_s.view(np.uint32), ws.view(np.uint32))


@pytest.mark.parametrize("wi", [1, 4])
def test_fp32_input_cast_full_size_sampled(wi):
    """The workload's input widened to fp32 (exact), cast at full size as the
    benchmark's fp32 operation launches it; the oracle checks a sample of rows
    (the first and last 8 and every 97th)."""
    w = inputs.WORKLOADS[wi]
    xb = inputs.generate(w, cache=True)
    log(f"[gpu] fp32-input cast full size {w.rows}x{w.cols} G={w.group} {w.out_dtype} {w.scale_fmt}")
    x = torch.from_numpy(xb.view(np.int16)).view(torch.bfloat16).cuda().float()
    q, s = tk.per_token_cast(x, w.group, w.out_dtype, w.round_pow2, w.scale_fmt)
    torch.cuda.synchronize()
    idx = np.array(sorted(set(range(8)) | set(range(w.rows - 8, w.rows)) | set(range(0, w.rows, 97))))
    xf = (xb[idx].astype(np.uint32) << 16).view(np.float32)
    wq, ws = oracle.per_token_cast_f32(xf, w.group, w.out_dtype, w.round_pow2, w.scale_fmt)
    got_q = q.cpu().numpy()[idx]
    got_s = s.cpu().numpy().view(np.uint32)[idx]
    assert np.array_equal(got_q, wq), first_mismatch(got_q, wq)
    assert np.array_equal(got_s, ws.view(np.uint32)), first_mismatch(got_s, ws.view(np.uint32))
