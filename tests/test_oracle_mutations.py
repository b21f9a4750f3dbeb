"""Planted mistakes in the oracle must be caught by its pins (CPU only).

Each case copies ``oracle/tk_oracle.c``, makes one plausible mistake in the copy
(a dropped term, a wrong sign or index, a swapped operand, a cheaper but inexact
operation), builds it, points the ``oracle`` module at that build and runs the
pin checks from test_oracle_pins.py.  At least one pin must fail; the real
source is never modified.
"""
from __future__ import annotations

import pathlib

import pytest

import oracle
import test_oracle_block_pins as bpins
import test_oracle_rmsnorm_pins as rpins
import test_oracle_dequant_pins as dpins
import test_oracle_pins as pins

SRC = pathlib.Path(oracle.__file__).resolve().parent / "tk_oracle.c"

# (name, original text, replacement, occurrence index or None for all)
MUTATIONS = [
    ("ties away from the even code", "return (k % 2 == 0) ? k : k - 1;", "return k;", None),
    ("ties toward zero", "return (k % 2 == 0) ? k : k - 1;", "return k - 1;", None),
    ("e4m3 saturates at 240", "const float M = 448.0f;", "const float M = 240.0f;", None),
    ("scale by reciprocal multiply", "float s = a / D;", "float s = a * (1.0f / D);", None),
    ("x/s by reciprocal multiply", "float q = x[i] / s;", "float q = x[i] * (1.0f / s);", None),
    ("pow2 rounds down", "if (m != 0) E += 1;", "(void)m;", None),
    ("pow2 always bumps", "if (m != 0) E += 1;", "E += 1; (void)m;", None),
    ("no amax floor", "if (a < floor_value) a = floor_value;", "(void)floor_value;", None),
    ("floor 1e-3", "const float floor_value = 1e-4f;", "const float floor_value = 1e-3f;", None),
    ("amax without abs", "float a = fabsf(x[i]);", "float a = x[i];", None),
    ("sign of zero dropped", "int neg = signbit(v) != 0;", "int neg = v < 0;", 0),
    ("e2m1 nibbles swapped", "(c % 2 == 0) ? nib : (nib << 4)", "(c % 2 == 1) ? nib : (nib << 4)", None),
    ("UE8M0 big-endian", "<< (8 * (j % 4))", "<< (8 * (3 - j % 4))", None),
    ("e4m3 subnormal step 2^-10", "ldexp((double)m, -9)", "ldexp((double)m, -10)", None),
    ("e4m3 bias 8", "ldexp(1.0 + m / 8.0, e - 7)", "ldexp(1.0 + m / 8.0, e - 8)", None),
    ("e2m1 bias 2", "ldexp(1.0 + m / 2.0, e - 1)", "ldexp(1.0 + m / 2.0, e - 2)", None),
    ("silu sign flipped", "x / (1.0L + expl(-x))", "x / (1.0L + expl(x))", None),
    ("silu in fp32 with expf", "long double r = x / (1.0L + expl(-x));",
     "float r = (float)x / (1.0f + expf(-(float)x));", None),
    ("gate and up swapped", "float g = bf16_to_f32(row[c]);\n            float u = bf16_to_f32(row[cols + c]);",
     "float u = bf16_to_f32(row[c]);\n            float g = bf16_to_f32(row[cols + c]);", None),
    ("group offset off by one group", "const float *x = v + j * group;",
     "const float *x = v + ((j + 1) % ngroups) * group;", None),
    ("bf16 truncation", "return (uint16_t)((b + 0x7FFFu + lsb) >> 16);", "(void)lsb; return (uint16_t)(b >> 16);", None),
    ("bf16 ties away", "return (uint16_t)((b + 0x7FFFu + lsb) >> 16);", "(void)lsb; return (uint16_t)((b + 0x8000u) >> 16);", None),
    ("dequant UE8M0 exponent off by one", "s = f32_from_bits(e << 23);", "s = f32_from_bits((e + 1) << 23);", None),
    ("dequant nibbles swapped", "code = (c % 2 == 0) ? (byte & 0xF) : (byte >> 4);",
     "code = (c % 2 == 1) ? (byte & 0xF) : (byte >> 4);", None),
    ("block amax over its first row only",
     "for (int64_t r = r0; r < r1; ++r)\n                for (int64_t c = c0; c < c0 + block_cols; ++c) {\n                    float a",
     "for (int64_t r = r0; r < r0 + 1; ++r)\n                for (int64_t c = c0; c < c0 + block_cols; ++c) {\n                    float a", None),
    ("block rows rounded down", "int64_t nbr = (rows + block_rows - 1) / block_rows;",
     "int64_t nbr = rows / block_rows;", None),
    ("block UE8M0 big-endian", "<< (8 * (bj % 4))", "<< (8 * (3 - bj % 4))", None),
    ("block amax over one column", "for (int64_t c = c0; c < c0 + block_cols; ++c) {\n                    float a",
     "for (int64_t c = c0; c < c0 + 1; ++c) {\n                    float a", None),
    ("sum of squares in fp32", "for (int64_t j = 0; j < n; ++j) sq_add(acc, x[j]);\n    return sq_round_f32(acc);",
     "float f = 0.0f;\n    for (int64_t j = 0; j < n; ++j) f += bf16_to_f32(x[j]) * bf16_to_f32(x[j]);\n"
     "    (void)sq_add; (void)sq_round_f32;\n    return f;", None),
    ("sum of squares rounds ties up", "if (round && (sticky || (mant & 1u))) mant += 1;", "if (round) mant += 1;", None),
    ("sum of squares without subnormal rounding", "if (lsb < SQ_SHIFT - 149) lsb = SQ_SHIFT - 149;", "", None),
    ("eps added before the mean", "float t = ss / (float)cols;\n    t = t + eps;",
     "float t = (ss + eps) / (float)cols;", None),
    ("rsqrt rounded once", "float rs = sqrtf(t);\n    float r = 1.0f / rs;",
     "float r = (float)(1.0 / sqrt((double)t));", None),
    ("weight ignored", "y[j] = w ? v * bf16_to_f32(w[j]) : v;", "y[j] = v; (void)w;", None),
    ("decode drops the sign", "return (float)((code & 0x80) ? -m : m);", "return (float)m;", None),
]


def _checks():
    """Cheap, broad checks first; each mutant stops at the first failing one."""
    gold = pins._golden()
    out = [lambda c=c: pins.test_hand_examples(c) for c in gold["cases"]]
    out += [pins.test_e4m3_tie_table, pins.test_e2m1_tie_table, pins.test_floor_constant_bits,
            dpins.test_e4m3_code_values_vs_torch, dpins.test_e2m1_code_values_by_hand,
            dpins.test_bf16_rounding_vs_torch,
            lambda: dpins.test_dequant_vs_library_composition(32, "e2m1", "ue8m0", True, "bf16"),
            lambda: dpins.test_dequant_vs_library_composition(128, "e4m3", "f32", False, "f32"),
            lambda: dpins.test_cast_back_vs_library_composition(64, "e4m3", True),
            lambda: bpins.test_per_block_vs_library_composition("e4m3", True, "ue8m0", 32, 32, 37),
            lambda: [rpins.test_sum_squares_rounding_cases(v, e) for v, e in rpins.MIDPOINT_ROWS],
            lambda: rpins.test_sum_squares_exact("wide"),
            lambda: rpins.test_rmsnorm_vs_library_composition(True, 1e-6),
            lambda: rpins.test_rmsnorm_vs_library_composition(False, 0.5),
            lambda: bpins.test_per_block_vs_library_composition("e2m1", False, "f32", 16, 64, 37),
            lambda: pins.test_whole_tensor_vs_library_composition(32, "e2m1", True, "ue8m0", 3, 4),
            lambda: pins.test_whole_tensor_division_hard_cases("e4m3"),
            pins.test_e4m3_exhaustive_bf16_times_pow2_vs_torch,
            pins.test_e2m1_exhaustive_bf16_times_pow2_vs_quantum_rounding,
            lambda: pins.test_scale_division_exact_all_bf16_amax("e4m3", 448),
            lambda: pins.test_scale_division_exact_all_bf16_amax("e2m1", 6),
            pins.test_division_vs_exact_and_numpy,
            pins.test_swiglu_sweep_vs_library_composition,
            pins.test_silu32_every_bf16_gate_vs_60_digit_decimal,
            lambda: pins.test_pow2_round_up_exact("e4m3", 448)]
    return out


@pytest.mark.parametrize("name,old,new,occ", MUTATIONS, ids=[m[0] for m in MUTATIONS])
def test_planted_mistake_is_caught(tmp_path, name, old, new, occ):
    text = SRC.read_text()
    assert old in text, f"mutation anchor not found: {old!r}"
    if occ is None:
        mutated = text.replace(old, new)
    else:
        parts = text.split(old)
        mutated = old.join(parts[: occ + 1]) + new + old.join(parts[occ + 1:])
    assert mutated != text
    src = tmp_path / "mutant.c"
    src.write_text(mutated)
    lib = oracle.compile_source(src, tmp_path / "libmutant.so")
    caught = None
    with oracle.using(lib):
        for check in _checks():
            try:
                check()
            except (AssertionError, ValueError) as e:
                caught = e
                break
    assert caught is not None, f"no pin caught the planted mistake: {name}"


@pytest.mark.parametrize("name", ["scale by reciprocal multiply", "no amax floor", "floor 1e-3"])
def test_workload_division_pin_alone_catches(tmp_path, name):
    """The division pin on the five workloads' amax values fails, by itself,
    for an inexact scale division or a wrong or missing floor.  (x * (1/s) in
    the cast's own loop changes a code only at rounding edges, which the
    division-hard groups of test_whole_tensor_division_hard_cases construct.)"""
    _, old, new, occ = next(m for m in MUTATIONS if m[0] == name)
    src = tmp_path / "mutant.c"
    src.write_text(SRC.read_text().replace(old, new))
    lib = oracle.compile_source(src, tmp_path / "libmutant.so")
    with oracle.using(lib), pytest.raises(AssertionError):
        pins.test_division_on_workload_amax_values()
