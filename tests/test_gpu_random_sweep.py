"""Randomised GPU parity: seeded random shapes, formats, row strides and value
ranges for every entry point, each case checked bit for bit against the oracle
through the same helpers as the fixed sweeps.  Every case is logged before it
runs, so a failure names its shape; the seeds are fixed, so it reproduces."""
from __future__ import annotations

import math

import numpy as np
import pytest
import torch

import oracle
import activation_quantization_token_amd as tk
from activation_quantization_token_amd import inputs
from gpu_util import Guarded, first_mismatch, log
from test_gpu_block import check_block, check_channel
from test_gpu_dequant import check_cast_back, check_dequant
from test_gpu_norm import check_norm, check_norm_cast
from test_gpu_parity import check

pytestmark = pytest.mark.gpu

VARIANTS = [("e4m3", False, "f32"), ("e4m3", True, "f32"), ("e4m3", True, "ue8m0"),
            ("e2m1", False, "f32"), ("e2m1", True, "f32"), ("e2m1", True, "ue8m0")]
GROUPS = (16, 32, 64, 128)
MAX_ELEMS = 6 << 20
CHUNKS, CASES_PER_CHUNK = 8, 60


class Cases:
    def __init__(self, rng: np.random.Generator):
        self.rng = rng

    def logu(self, lo, hi):
        """An integer drawn log-uniformly from [lo, hi]."""
        return int(round(math.exp(self.rng.uniform(math.log(lo), math.log(hi)))))

    def cols(self, unit, hi):
        return unit * max(1, self.logu(1, max(2, hi // unit)))

    def rows(self, cols, hi=6000):
        return max(1, min(self.logu(1, hi), MAX_ELEMS // cols))

    def variant(self):
        return int(self.rng.choice(GROUPS)), *VARIANTS[self.rng.integers(len(VARIANTS))]

    def x_ld(self, cols):
        return None if self.rng.random() < 0.6 else cols + 8 * int(self.rng.integers(1, 9))

    def values(self, rows, cols):
        """bf16 bits [rows, cols]: the small-sweep generator (normal or Student-t,
        log-uniform row scales, outliers, a zero row), rows scaled across the
        whole bf16 range, small integers times powers of two (many exact ties),
        or tiny values with 30 % zeros."""
        kind = str(self.rng.choice(["normal", "t3", "wide", "ints", "tiny"]))
        seed = int(self.rng.integers(1 << 30))
        if kind in ("normal", "t3"):
            return inputs.generate_small(seed, rows, cols, "normal" if kind == "normal" else "student_t3"), kind
        r = np.random.default_rng(seed)
        if kind == "wide":
            x = r.standard_normal((rows, cols)) * np.exp2(r.uniform(-130, 110, size=(rows, 1)))
        elif kind == "ints":
            x = r.integers(-8, 9, size=(rows, cols)).astype(np.float64) * np.exp2(r.integers(-4, 5, size=(rows, 1)))
        else:
            x = r.standard_normal((rows, cols)) * 1e-6
            x[r.random((rows, cols)) < 0.3] = 0.0
        return inputs.f64_to_bf16_bits(x), kind

    def cast(self):
        g, dt, p2, sf = self.variant()
        cols = self.cols(4 * g if sf == "ue8m0" else g, 40000 if self.rng.random() < 0.1 else 16384)
        x, kind = self.values(self.rows(cols), cols)
        check(x, g, dt, p2, sf, x_ld=self.x_ld(cols), label=f"random {kind}")

    def swiglu(self):
        g, dt, p2, sf = self.variant()
        cols = self.cols(4 * g if sf == "ue8m0" else g, 16384)
        rows = self.rows(2 * cols)
        x = inputs.generate_small(int(self.rng.integers(1 << 30)), rows, 2 * cols,
                                  str(self.rng.choice(["normal", "student_t3"])))
        check(x, g, dt, p2, sf, swiglu=True, x_ld=self.x_ld(2 * cols), label="random")

    def cast_f32(self):
        g, dt, p2, sf = self.variant()
        cols = self.cols(4 * g if sf == "ue8m0" else g, 16384)
        rows = self.rows(cols)
        x = inputs.generate_small_f32(int(self.rng.integers(1 << 30)), rows, cols)
        if self.rng.random() < 0.3:
            x = (x.astype(np.float64) * np.exp2(self.rng.uniform(-100, 80, size=(rows, 1)))).astype(np.float32)
        ld = cols + 4 * int(self.rng.integers(0, 5))
        log(f"[gpu] random fp32 cast rows={rows} cols={cols} ld={ld} G={g} {dt} pow2={p2} {sf}")
        buf = torch.full((rows, ld), float("nan"), dtype=torch.float32, device="cuda")
        buf[:, :cols] = torch.from_numpy(x).cuda()
        q = Guarded(rows, cols if dt == "e4m3" else cols // 2, torch.uint8, 24)
        s = Guarded(rows, cols // g if sf == "f32" else cols // g // 4,
                    torch.float32 if sf == "f32" else torch.int32, 3)
        tk.per_token_cast(buf[:, :cols], g, dt, p2, sf, out=(q.view, s.view))
        torch.cuda.synchronize()
        want_q, want_s = oracle.per_token_cast_f32(x, g, dt, p2, sf)
        assert q.canaries_intact() and s.canaries_intact(), "write outside the outputs"
        got_q, got_s = q.view.cpu().numpy(), s.view.cpu().numpy().view(np.uint32)
        assert np.array_equal(got_q, want_q), first_mismatch(got_q, want_q)
        assert np.array_equal(got_s, want_s.view(np.uint32)), first_mismatch(got_s, want_s.view(np.uint32))

    def dequant(self):
        g, dt, p2, sf = self.variant()
        cols = self.cols(4 * g if sf == "ue8m0" else g, 16384)
        x, kind = self.values(self.rows(cols), cols)
        check_dequant(x, g, dt, p2, sf, str(self.rng.choice(["bf16", "f32"])), label=f"random {kind}")

    def cast_back(self):
        g, dt, p2, _ = self.variant()
        cols = self.cols(g, 16384)
        x, kind = self.values(self.rows(cols), cols)
        check_cast_back(x, g, dt, p2, x_ld=self.x_ld(cols), label=f"random {kind}")

    def per_block(self):
        g, dt, p2, sf = self.variant()
        br = int(self.rng.choice([1, 2, 3, 7, 16, 32, 64, 100, 128, 129, 200, 255, 256]))
        cols = self.cols(4 * g if sf == "ue8m0" else g, 16384)
        x, kind = self.values(self.rows(cols, 8000), cols)
        check_block(x, br, g, dt, p2, sf, x_ld=self.x_ld(cols), label=f"random {kind}")

    def per_channel(self):
        _, dt, p2, sf = self.variant()
        cols = self.cols(8, 16384)
        rows = self.rows(cols, 40000)
        if self.rng.random() < 0.05:      # inputs above 64 MiB take the three-kernel form
            rows = max(1, min(self.logu(2000, 40000), (48 << 20) // cols))
        x, kind = self.values(rows, cols)
        check_channel(x, dt, p2, sf, x_ld=self.x_ld(cols), label=f"random {kind}")

    def rmsnorm(self):
        cols = self.cols(8, 16384)
        x, kind = self.values(self.rows(cols), cols)
        w = inputs.generate_small(int(self.rng.integers(1 << 30)), 1, cols)[0] if self.rng.random() < 0.7 else None
        eps = float(self.rng.choice([1e-6, 1e-5, 1e-2, 1.0]))
        check_norm(x, w, eps, str(self.rng.choice(["bf16", "f32"])), x_ld=self.x_ld(cols), label=f"random {kind}")

    def rmsnorm_cast(self):
        g, dt, p2, sf = self.variant()
        unit = 4 * g if sf == "ue8m0" else g
        cols = min(self.cols(unit, 16384), 16384 - 16384 % unit)
        x, kind = self.values(self.rows(cols), cols)
        w = inputs.generate_small(int(self.rng.integers(1 << 30)), 1, cols)[0] if self.rng.random() < 0.7 else None
        eps = float(self.rng.choice([1e-6, 1e-5, 1e-2]))
        check_norm_cast(x, w, eps, g, dt, p2, sf, x_ld=self.x_ld(cols), label=f"random {kind}")


OPS = [("cast", 4), ("swiglu", 2), ("cast_f32", 2), ("dequant", 1), ("cast_back", 1), ("per_block", 2),
       ("per_channel", 2), ("rmsnorm", 1), ("rmsnorm_cast", 2)]


@pytest.mark.parametrize("chunk", range(CHUNKS))
def test_random_cases(chunk):
    rng = np.random.default_rng([20261203, chunk])
    cases = Cases(rng)
    p = np.array([w for _, w in OPS], dtype=float)
    for i in range(CASES_PER_CHUNK):
        name = OPS[int(rng.choice(len(OPS), p=p / p.sum()))][0]
        log(f"[gpu] random sweep chunk {chunk} case {i}: {name}")
        getattr(cases, name)()
