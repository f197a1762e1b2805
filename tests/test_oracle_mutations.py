"""Plant plausible mistakes in a copy of the oracle (CPU only) and check
that the pin suite rejects every one of them: a dropped term, a wrong sign,
a wrong power, a wrong denominator, eps outside the root, a lost
weight_bias, a rounding format off by one bit.
"""
import os
import subprocess

import pytest

from oracle import oracle as O

import test_oracle_pins as P
import test_oracle_rounding as R

SRC = os.path.join(os.path.dirname(O.__file__), "rmsnorm_oracle.c")

# (name, exact text in the oracle source, replacement, occurrence to replace)
MUTATIONS = [
    ("fwd_mean_over_D_minus_1", "double ms = ss / (double)D;\n        double r = 1.0 / sqrt(ms + eps);\n        if (rstd)",
     "double ms = ss / (double)(D > 1 ? D - 1 : 1);\n        double r = 1.0 / sqrt(ms + eps);\n        if (rstd)"),
    ("fwd_eps_outside_root", "double r = 1.0 / sqrt(ms + eps);\n        if (rstd)",
     "double r = 1.0 / sqrt(ms) + eps;\n        if (rstd)"),
    ("fwd_drop_weight_bias", "yi[j] = xi[j] * r * (weight_bias + w[j]);", "yi[j] = xi[j] * r * w[j];"),
    ("vjp_sign_of_projection", "dxi[j] = r * g * dyi[j] - xi[j] * r3 * S / (double)D;",
     "dxi[j] = r * g * dyi[j] + xi[j] * r3 * S / (double)D;"),
    ("vjp_r_squared_not_cubed", "double r3 = r * r * r;", "double r3 = r * r;"),
    ("vjp_drop_projection", "dxi[j] = r * g * dyi[j] - xi[j] * r3 * S / (double)D;",
     "dxi[j] = r * g * dyi[j];"),
    ("vjp_S_without_weight_bias", "S += dyi[j] * (weight_bias + w[j]) * xi[j];", "S += dyi[j] * w[j] * xi[j];"),
    ("vjp_S_without_weight", "S += dyi[j] * (weight_bias + w[j]) * xi[j];", "S += dyi[j] * xi[j];"),
    ("vjp_dx_g_without_bias", "double g = weight_bias + w[j];", "double g = w[j];"),
    ("vjp_dw_without_r", "dw[j] += dyi[j] * xi[j] * r;", "dw[j] += dyi[j] * xi[j];"),
    ("vjp_dw_times_g", "dw[j] += dyi[j] * xi[j] * r;", "dw[j] += dyi[j] * xi[j] * r * (weight_bias + w[j]);"),
    ("vjp_mean_over_D_minus_1", "double ms = ss / (double)D;\n        double r = 1.0 / sqrt(ms + eps);\n        double S",
     "double ms = ss / (double)(D > 1 ? D - 1 : 1);\n        double r = 1.0 / sqrt(ms + eps);\n        double S"),
    ("vjp_divide_S_by_D_minus_1", "xi[j] * r3 * S / (double)D;", "xi[j] * r3 * S / (double)(D > 1 ? D - 1 : 1);"),
    ("fused_rounds_sum_first", "new_residual[i * D + j] = x[i * D + j] + residual[i * D + j];",
     "new_residual[i * D + j] = (double)(float)(x[i * D + j] + residual[i * D + j]) + 1e-3;"),
    ("fused_vjp_drops_residual_grad", "        dh[i] += d_new_residual[i];", "        dh[i] += 0.0 * d_new_residual[i];"),
    ("fused_vjp_subtracts_residual_grad", "        dh[i] += d_new_residual[i];", "        dh[i] -= d_new_residual[i];"),
    ("gate_sigmoid_sign", "y[i * d + j] = a[j] / (1.0 + exp(-a[j])) * b[j];", "y[i * d + j] = a[j] / (1.0 + exp(a[j])) * b[j];"),
    ("gate_swapped_halves", "y[i * d + j] = a[j] / (1.0 + exp(-a[j])) * b[j];", "y[i * d + j] = b[j] / (1.0 + exp(-b[j])) * a[j];"),
    ("gate_vjp_drop_sigmoid_slope", "da[j] = g * b[j] * sg * (1.0 + a[j] * (1.0 - sg));", "da[j] = g * b[j] * sg;"),
    ("gate_vjp_db_without_a", "db[j] = g * a[j] * sg;", "db[j] = g * sg;"),
    ("f16_one_bit_short", "return rne_to_format(v, 10, -14, 15);", "return rne_to_format(v, 9, -14, 15);"),
    ("f16_wrong_emin", "return rne_to_format(v, 10, -14, 15);", "return rne_to_format(v, 10, -15, 15);"),
    ("bf16_truncates", "double n = nearbyint(q);", "double n = trunc(q);"),
    ("round_ties_away", "double n = nearbyint(q);", "double n = round(q);"),
]

# The pin checks run against each mutant (each call either passes or raises).
CHECKS = [
    lambda: [P.test_fwd_unit_weight_mean_square(e, d) for e in (1e-5, 0.25) for d in (1, 7, 64)],
    lambda: [P.test_fwd_constant_row(c) for c in (0.5, 3.0)],
    P.test_fwd_zero_row_and_D1,
    lambda: [P.test_fwd_eps_inside_root_homogeneity(c) for c in (2.0, 0.5)],
    P.test_fwd_scaled_weight_and_gemma,
    P.test_hand_worked_examples,
    P.test_fused_is_add_then_norm_of_unrounded_sum,
    lambda: [P.test_vjp_finite_differences(r, d, wb) for r in (1, 3) for d in (1, 5, 8) for wb in (0.0, 1.0)],
    lambda: [P.test_vjp_torch_fp64_autograd(wb) for wb in (0.0, 1.0)],
    P.test_vjp_projection_identity,
    P.test_vjp_D1_and_zero_row,
    P.test_dw_independent_of_weight,
    lambda: [P.test_fused_vjp_finite_differences(r, d, wb) for (r, d) in ((1, 1), (2, 3)) for wb in (0.0, 1.0)],
    P.test_silu_gate_odd_part_identity,
    P.test_silu_gate_special_values_and_torch,
    P.test_silu_gate_vjp_finite_differences,
    P.test_silu_gate_vjp_torch_and_special_values,
    R.test_f16_exhaustive_round_trip,
    R.test_f16_midpoints_and_random_match_numpy,
    R.test_bf16_matches_brute_force_nearest,
    lambda: [R.test_rounding_special_values(*a) for a in [
        ("float16", 1.0 + 2 ** -11, 1.0), ("float16", 65520.0, float("inf")),
        ("bfloat16", 1.0 + 2 ** -8, 1.0), ("float16", 3 * 2.0 ** -26, 2.0 ** -24)]],
]


@pytest.fixture(scope="module")
def source():
    with open(SRC) as f:
        return f.read()


@pytest.mark.parametrize("name,old,new", MUTATIONS, ids=[m[0] for m in MUTATIONS])
def test_pins_catch_mutation(name, old, new, source, tmp_path):
    assert source.count(old) == 1, f"mutation anchor for {name} not unique"
    mutated = source.replace(old, new)
    src = tmp_path / "mut.c"
    src.write_text(mutated)
    lib = tmp_path / "libmut.so"
    subprocess.check_call(["gcc", "-O2", "-ffp-contract=off", "-shared", "-fPIC",
                           "-o", str(lib), str(src), "-lm"])
    caught = []
    O.swap_library(str(lib))
    try:
        for i, check in enumerate(CHECKS):
            try:
                check()
            except AssertionError:
                caught.append(i)
    finally:
        O.swap_library(None)
    assert caught, f"no pin caught the planted mistake {name}"


def test_real_oracle_passes_every_check():
    for check in CHECKS:
        check()
