"""The pins are sensitive: each plants one plausible mistake in a copy of the
oracle (a dropped term, a wrong sign, a changed order, a wrong rounding, an
off-by-one rule), builds it, and requires the pin file that guards that part
to fail against it.  The unmodified oracle passes the same files in the
main run.  CPU only.
"""
import os
import subprocess
import sys

import pytest

import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
ADAM = "tests/test_oracle_adam.py"
REDUCE = "tests/test_oracle_reduce_norm.py"
PART = "tests/test_oracle_partition_bytes.py"
INV = "tests/test_oracle_invariant.py"
FMT = "tests/test_oracle_formats.py::test_round_trip_and_boundaries"
FMT_ALL = "tests/test_oracle_formats.py::test_f16_to_f32_all_patterns"
QUANT = "tests/test_oracle_quant.py"

# (original text, planted mistake, pin files that must catch it)
MUTANTS = {
    "adam_no_bias_correction_m": ("float mhat = mi / bc1;", "float mhat = mi;", [ADAM]),
    "adam_no_bias_correction_v": ("float vhat = vi / bc2;", "float vhat = vi;", [ADAM]),
    "adam_eps_inside_sqrt": ("float u = mhat / (sqrtf(vhat) + eps);",
                             "float u = mhat / sqrtf(vhat + eps);", [ADAM]),
    "adam_decay_sign": ("p[i] = p[i] - lr * (u + wd * p[i]);",
                        "p[i] = p[i] - lr * (u - wd * p[i]);", [ADAM]),
    "adam_v_uses_g_not_g2": ("float vi = b2 * v[i] + omb2 * (gi * gi);",
                             "float vi = b2 * v[i] + omb2 * gi;", [ADAM]),
    "adam_swapped_betas": ("float mi = b1 * m[i] + omb1 * gi;",
                           "float mi = b2 * m[i] + omb2 * gi;", [ADAM]),
    "step_count_not_advanced": ("st->pow1 = st->pow1 * (double)hp->beta1;",
                                "st->pow1 = st->pow1;", [ADAM]),
    "clip_without_epsilon": ("double coef = (double)hp->max_grad_norm / (rep->norm + 1e-6);",
                             "double coef = (double)hp->max_grad_norm / rep->norm;", [ADAM]),
    "clip_only_above_max": ("if (coef < 1.0) rep->clip = (float)coef;",
                            "if (coef < 1.0 && rep->norm > (double)hp->max_grad_norm) "
                            "rep->clip = (float)coef;", [ADAM]),
    "clip_coefficient_in_fp32": ("double coef = (double)hp->max_grad_norm / (rep->norm + 1e-6);",
                                 "double coef = (double)(hp->max_grad_norm / "
                                 "(float)(rep->norm + 1e-6));", [ADAM]),
    "growth_overflows_to_inf": ("if (isfinite(twice)) st->scale = twice;", "st->scale = twice;",
                                [ADAM]),
    "scaler_no_halving": ("float half = st->scale * 0.5f;", "float half = st->scale;", [ADAM]),
    "reduce_reverse_order": (
        "for (int32_t k = 0; k < n; ++k) acc = acc + oracle_to_f32(C[(int64_t)k * stride + i], dtype);",
        "for (int32_t k = n - 1; k >= 0; --k) acc = acc + oracle_to_f32(C[(int64_t)k * stride + i], dtype);",
        [REDUCE]),
    "reduce_no_average": ("return (float)(1.0 / ((double)nranks * (double)loss_scale));",
                          "return (float)(1.0 / (double)loss_scale);", [REDUCE]),
    "overflow_not_flagged": (
        "oracle_to_f32(C[(int64_t)k * stride + i], dtype);\n        if (!isfinite(acc)) flag = 1;",
        "oracle_to_f32(C[(int64_t)k * stride + i], dtype);\n        if (isnan(acc)) flag = 1;",
        [REDUCE]),
    "reduce_q_overflow_not_flagged": (
        "zero[k][b]);\n        if (!isfinite(acc)) flag = 1;",
        "zero[k][b]);\n        if (acc != acc) flag = acc != acc;", [QUANT]),
    "norm_ignores_inf": ("if (isinf(x)) { a->has_inf = 1; continue; }", "if (isinf(x)) { continue; }",
                         [REDUCE]),
    "partition_floor": ("int64_t s = psi / nranks + (psi % nranks != 0 ? 1 : 0);",
                        "int64_t s = psi / nranks;", [PART]),
    "round_half_away": ("if (frac > 0.5 || (frac == 0.5 && (r & 1) != 0)) r += 1;",
                        "if (frac >= 0.5) r += 1;", [FMT]),
    "overflow_boundary_off_by_one": ("if (E > F->emax) return (uint16_t)(sign | F->inf);",
                                     "if (E >= F->emax) return (uint16_t)(sign | F->inf);", [FMT]),
    "subnormal_decode_exponent": ("mag = (double)f * pow2i(F->emin - fb);",
                                  "mag = (double)f * pow2i(F->emin - fb - 1);", [FMT_ALL]),
    "sumsq_bit_position": ("int p = 2 * e + 296;", "int p = 2 * e + 297;", [REDUCE]),
    "skip_ignores_overflow": ("rep->skip = rep->nonfinite;", "rep->skip = 0;", [ADAM]),
    "growth_without_reset": ("if (isfinite(twice)) st->scale = twice;\n                st->good = 0;",
                             "if (isfinite(twice)) st->scale = twice;", [ADAM]),
    "quant_no_zero_point": ("const float z = q_clamp_code(rintf(-lo / s), qmax);",
                            "const float z = 0.0f;", [QUANT]),
    "quant_truncates": ("q_clamp_code(rintf(x * inv) + z, qmax)", "q_clamp_code(truncf(x * inv) + z, qmax)",
                        [QUANT]),
    "quant_divides": ("q_clamp_code(rintf(x * inv) + z, qmax)", "q_clamp_code(rintf(x / s) + z, qmax)",
                      [QUANT]),
    "quant_round_half_away": ("q_clamp_code(rintf(x * inv) + z, qmax)",
                              "q_clamp_code(roundf(x * inv) + z, qmax)", [QUANT]),
    "quant_levels_off_by_one": ("const float qmax = (float)((1 << bits) - 1);",
                                "const float qmax = (float)(1 << bits);", [QUANT]),
    "quant_range_without_zero": ("float lo = 0.0f, hi = 0.0f;",
                                 "float lo = 3.0e38f, hi = -3.0e38f;", [QUANT]),
    "quant_nibble_order": ("(q << (4 * (i % 2)))", "(q << (4 * (1 - i % 2)))", [QUANT]),
    "quant_nan_ignored": ("if (!isfinite(x)) finite = 0;", "if (isinf(x)) finite = 0;", [QUANT]),
    "quant_block_size": ("#define ORACLE_QBLOCK 2048", "#define ORACLE_QBLOCK 1024", [QUANT]),
    "dequant_sign_of_zero_point": ("out[i] = scale[b] * (float)(q_code(codes, bits, i) - zero[b]);",
                                   "out[i] = scale[b] * (float)(q_code(codes, bits, i) + zero[b]);",
                                   [QUANT]),
    "reduce_q_reverse_order": ("for (int32_t k = 0; k < n; ++k)\n            acc = acc + scale[k][b]",
                               "for (int32_t k = n - 1; k >= 0; --k)\n            acc = acc + scale[k][b]",
                               [QUANT]),
}


@pytest.mark.parametrize("name", list(MUTANTS))
def test_pins_catch_planted_mistake(name, tmp_path):
    old, new, files = MUTANTS[name]
    src = open(os.path.join(ROOT, "oracle", "oracle.c")).read()
    assert src.count(old) == 1, f"mutation site for {name} not found exactly once"
    mut = tmp_path / "oracle.c"
    mut.write_text(src.replace(old, new))
    so = tmp_path / "liboracle_mutant.so"
    subprocess.run(["gcc", *oracle.GCC_FLAGS, "-o", str(so), str(mut), "-lm"], check=True)
    env = dict(os.environ, ORACLE_LIB=str(so))
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider",
                        "-m", "not gpu", *files], cwd=ROOT, env=env, capture_output=True, text=True)
    assert r.returncode == 1, f"{name}: pins did not fail (rc {r.returncode})\n{r.stdout[-2000:]}"
