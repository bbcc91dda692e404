"""Mutation check of the oracle's pins (CPU only).

Each case plants one plausible mistake in a private copy of the oracle's C
source, builds it, and runs the pins against that copy: at least one pin must
fail.  This shows the pins constrain the oracle beyond agreeing with itself.
"""
from __future__ import annotations

from pathlib import Path

import pytest

import oracle as oracle_pkg
from tests import test_oracle_pins as pins
from tests import test_oracle_alloc_pins as apins
from tests import test_oracle_gate_pins as gpins
from tests import test_oracle_refit_pins as rpins
from tests import test_oracle_eq2_pins as epins

SRC = Path(oracle_pkg.__file__).resolve().parent / "stq_oracle.c"
ALLOC_SRC = Path(oracle_pkg.__file__).resolve().parent / "stq_alloc_oracle.c"

# (name, text in the oracle source, replacement)
MUTANTS = [
    ("u transposed (S k instead of S^T k)",
     "acc += S[(size_t)i * dv + j] * k[i];", "acc += S[(size_t)j * dv + i] * k[i];"),
    ("sign of the delta correction", "(v[j] - alpha * u[j])", "(v[j] + alpha * u[j])"),
    ("gate dropped on S^T k", "(v[j] - alpha * u[j])", "(v[j] - u[j])"),
    ("gate dropped on S", "*x = alpha * (*x) + ", "*x = (*x) + "),
    ("beta dropped", "beta * k[i] * (v[j]", "k[i] * (v[j]"),
    ("readout with k instead of q",
     "acc += S[(size_t)i * dv + j] * q[i];", "acc += S[(size_t)i * dv + j] * k[i];"),
    ("round half away from zero", "return (fmod(f, 2.0) == 0.0) ? f : f + 1.0;",
     "return f + 1.0;"),
    ("nibble order swapped", "(j % 2 == 0) ? (byte & 0x0F) : (byte >> 4)",
     "(j % 2 == 0) ? (byte >> 4) : (byte & 0x0F)"),
    ("nibble not sign-extended", "return nib >= 8 ? nib - 16 : nib;", "return nib;"),
    ("row factor from the mean instead of the max", "if (fabs(x) > m) m = fabs(x);",
     "m += fabs(x) / s->dv;"),
    ("physical order ignored in dequant",
     "int i = perm[p];\n        for (int j = 0; j < s->dv; ++j) {\n            double rc",
     "int i = p;\n        for (int j = 0; j < s->dv; ++j) {\n            double rc"),
    ("column factor ignored in requant", "double x = row[j] / (double)c[j];",
     "double x = row[j];"),
    ("q_b off by one", "(1 << (bits - 1)) - 1", "(1 << (bits - 1))"),
    ("no floor on the row factor", "if (rr < floor_r) rr = floor_r;", ""),
    ("wrong GQA map", "int hk = h / (s->hv / s->hk); /* reading R5 */", "int hk = h % s->hk;"),
    ("row factor not rounded to fp32", "double rr = (double)(float)(m / (double)qb);",
     "double rr = m / (double)qb;"),
    ("row score of |S| instead of S^2", "acc += x * x;", "acc += fabs(x);"),
    ("ties to the higher row", "(sc[a] == sc[i] && a < i)", "(sc[a] == sc[i] && a > i)"),
    ("zero column kept at 0", "(m > 0.0) ? (float)m : 1.0f", "(float)m"),
    ("bit width from the logical row", "int qb = qmax_of_bits(row_bits(p, s->n8));",
     "int qb = qmax_of_bits(row_bits(i, s->n8));"),
    ("refit weights dropped", "double wt = (double)w2[i];", "double wt = 1.0;"),
    ("refit weight by physical row", "double wt = (double)w2[i];", "double wt = (double)w2[p];"),
    ("refit denominator unweighted", "den += wt * vij * vij;", "den += vij * vij;"),
    ("refit v includes the old column factor",
     "double vij = (double)r[p] * (double)read_code(p8, p4, s->n8, s->dv, p, j);",
     "double vij = (double)r[p] * (double)c[j] * (double)read_code(p8, p4, s->n8, s->dv, p, j);"),
    ("refit on a zero denominator", "if (den > 0.0) {", "if (den >= 0.0) {"),
    ("impact without beta", "double gi = a * ((double)qq[i] - be * (double)kk[i] * kq);",
     "double gi = a * ((double)qq[i] - (double)kk[i] * kq);"),
    ("impact without the gate", "double gi = a * ((double)qq[i] - be * (double)kk[i] * kq);",
     "double gi = ((double)qq[i] - be * (double)kk[i] * kq);"),
    ("row gate dropped on S^T k", "acc += d[i] * S[(size_t)i * dv + j] * k[i];",
     "acc += S[(size_t)i * dv + j] * k[i];"),
    ("row gate dropped on S", "*x = d[i] * (*x) + ", "*x = (*x) + "),
    ("row gate applied by column", "*x = d[i] * (*x) + ", "*x = d[j] * (*x) + "),
    ("row gate read in reversed row order", "d[i] = (double)gate[(size_t)u * dk + i];",
     "d[i] = (double)gate[(size_t)u * dk + (dk - 1 - i)];"),
    ("impact row gate from row 0", "double a = gate ? (double)gate[((size_t)b * hv + h) * dk + i]",
     "double a = gate ? (double)gate[((size_t)b * hv + h) * dk + 0]"),
    ("impact weight exponent 1/8", "pow(omega[(size_t)h * dk + i] / mean, 0.25)",
     "pow(omega[(size_t)h * dk + i] / mean, 0.125)"),
]


def _pin_cases():
    return [
        (pins.test_rhe_matches_numpy_rint_on_half_grid, {}),
        (pins.test_dequant_golden_layout, {}),
        (pins.test_pack_golden_half_ties, {"fixture": "requant_ties.json"}),
        (pins.test_pack_golden_half_ties, {"fixture": "requant_fp32_factor.json"}),
        (pins.test_quantizer_round_trip_brute_force, {"d": 32, "n8": 13}),
        (pins.test_pack_error_within_half_step, {"n8": 5}),
        (pins.test_int8row_equals_textbook_rowwise_absmax, {}),
        (pins.test_step_fixed_point, {"d": 16, "n8": 8}),
        (pins.test_step_delta_write_closed_form, {"d": 64, "n8": 32}),
        (pins.test_step_from_zero_state_closed_form, {}),
        (pins.test_step_requant_within_half_step, {"d": 32, "n8": 8}),
        (pins.test_proposition1_readout_error, {"d": 16, "n8": 8}),
        (pins.test_delta_feedback_norm_identity, {"d": 16}),
        (pins.test_isolated_row_read_error, {"d": 16}),
        (pins.test_error_recursion_and_drift_bound, {}),
        (pins.test_calibration_matches_numpy_max_and_stable_argsort, {}),
        (rpins.test_refit_recovers_exact_column_factors, {"d": 16, "n8": 8}),
        (rpins.test_refit_covariant_under_column_scaling, {"lam": 4.0}),
        (rpins.test_refit_minimises_weighted_objective, {}),
        (rpins.test_refit_zero_column_keeps_previous_factor, {}),
        (rpins.test_refit_step_fixed_point, {"d": 16, "n8": 8}),
        (rpins.test_impact_closed_form_unit_vectors, {}),
        (rpins.test_impact_weights_fourth_root_of_normalised_impact, {}),
        (gpins.test_uniform_gate_is_the_scalar_gate, {"d": 16, "n8": 8}),
        (gpins.test_one_hot_gate_keeps_one_logical_row, {}),
        (gpins.test_gated_delta_write_closed_form, {"d": 16, "n8": 16}),
        (gpins.test_gated_fp_step_one_hot, {}),
        (gpins.test_gated_impact_closed_form, {}),
        (gpins.test_gated_refit_uniform_gate_is_scalar, {}),
        (epins.test_mixed_step_equals_eq2, {"d": 16, "n8": 8, "gated": False}),
        (epins.test_mixed_step_equals_eq2, {"d": 32, "n8": 13, "gated": True}),
        (epins.test_refit_step_equals_eq2, {"d": 32, "n8": 16}),
    ]


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_pins_catch_planted_mistake(tmp_path, name, old, new):
    src = SRC.read_text()
    assert src.count(old) >= 1, f"mutation site missing: {name}"
    mutated = src.replace(old, new)
    msrc = tmp_path / "mutant.c"
    msrc.write_text(mutated)
    lib = oracle_pkg.compile_oracle(msrc, tmp_path / "libmutant.so")
    mut = oracle_pkg.Oracle(lib)
    caught = []
    for fn, kw in _pin_cases():
        try:
            fn(mut, **kw)
        except AssertionError:
            caught.append(fn.__name__)
        except (ValueError, FloatingPointError, OverflowError):
            caught.append(fn.__name__)
    assert caught, f"no pin caught the planted mistake: {name}"


# mistakes planted in the ragged-format oracle (stq_alloc_oracle.c)
ALLOC_MUTANTS = [
    ("6-bit high field position", "int hi = (row[d / 2 + j / 4] >> (2 * (j % 4))) & 0x3;",
     "int hi = (row[d / 2 + j / 4] >> (j % 4)) & 0x3;"),
    ("6-bit sign threshold", "return u >= 32 ? u - 64 : u;", "return u >= 31 ? u - 64 : u;"),
    ("2-bit code not sign-extended", "return u >= 2 ? u - 4 : u;", "return u;"),
    ("binary16 ties away from zero", "double n = oracle_rhe(ldexp(a, -qe));",
     "double n = floor(ldexp(a, -qe) + 0.5);"),
    ("binary16 subnormal quantum", "if (qe < -24) qe = -24;", "if (qe < -25) qe = -25;"),
    ("pivot row keeps a row factor", "r_out[p] = 0.0f;", "r_out[p] = 1.0f;"),
    ("q_b of the 2-bit rows", "static int qmax_of(int k) { return (1 << (kBits[k] - 1)) - 1; }",
     "static int qmax_of(int k) { return k == 4 ? 2 : (1 << (kBits[k] - 1)) - 1; }"),
    ("6-bit row size", "case 2: return 3 * d / 4;", "case 2: return d / 2 + d / 8;"),
    ("segment not padded", "L->seg = (off + 15) / 16 * 16;", "L->seg = off;"),
    ("lifetime without the square", "acc += exp(2.0 * (double)j * ell);",
     "acc += exp((double)j * ell);"),
    ("pivot score at 8 bits", "pv[u].score = Lw[u] * (dist[(size_t)u * NCLS + knom]",
     "pv[u].score = Lw[u] * (dist[(size_t)u * NCLS + 1]"),
    ("segments cheapest saving first", "if (x->slope > y->slope) return -1;\n    if (x->slope < y->slope) return 1;",
     "if (x->slope > y->slope) return 1;\n    if (x->slope < y->slope) return -1;"),
    ("budget counts pivots", "long budget = (long)nominal * n_int;", "long budget = (long)nominal * N;"),
    ("FP16 distortion from fp32 rounding",
     "double y = oracle_f16_to_double(oracle_f16_from_double(row[j]));",
     "double y = (double)(float)row[j];"),
]


def _alloc_pin_cases():
    return [
        (apins.test_f16_matches_numpy, {}),
        (apins.test_layout_golden_d16, {}),
        (apins.test_two_class_layout_equals_mixed_format, {"d": 16, "n8": 8}),
        (apins.test_round_trip_every_class, {"d": 16}),
        (apins.test_pack_error_within_half_step, {}),
        (apins.test_step_fixed_point_with_pivots, {"gated": False}),
        (apins.test_step_delta_write_closed_form, {}),
        (apins.test_step_refit_excludes_pivots_and_matches_pack, {}),
        (apins.test_distortion_pins, {}),
        (apins.test_lifetime_closed_form, {}),
        (apins.test_assignment_optimal_on_convex_instances, {"seed": 0}),
        (apins.test_assignment_optimal_on_convex_instances, {"seed": 3}),
        (apins.test_assignment_budget_pivots_and_layout, {}),
        (apins.test_pivot_ranking_uses_the_nominal_width, {}),
        (epins.test_ragged_step_equals_eq2, {"d": 16, "gated": False}),
        (epins.test_ragged_step_equals_eq2, {"d": 64, "gated": True}),
    ]


@pytest.mark.parametrize("name,old,new", ALLOC_MUTANTS, ids=[m[0] for m in ALLOC_MUTANTS])
def test_alloc_pins_catch_planted_mistake(tmp_path, name, old, new):
    src = ALLOC_SRC.read_text()
    assert src.count(old) >= 1, f"mutation site missing: {name}"
    msrc = tmp_path / "alloc_mutant.c"
    msrc.write_text(src.replace(old, new))
    lib = oracle_pkg.compile_oracle(SRC, tmp_path / "libmutant.so", alloc_src=msrc)
    mut = oracle_pkg.Oracle(lib)
    caught = []
    for fn, kw in _alloc_pin_cases():
        try:
            fn(mut, **kw)
        except (AssertionError, ValueError, FloatingPointError, OverflowError):
            caught.append(fn.__name__)
    assert caught, f"no pin caught the planted mistake: {name}"


# the update and readout mistakes above, each of which the pins against the
# dense form of Eq. (2) must catch on their own (both gates, every format)
UPDATE_MUTANTS = ["u transposed (S k instead of S^T k)", "sign of the delta correction",
                  "gate dropped on S^T k", "gate dropped on S", "beta dropped",
                  "readout with k instead of q", "wrong GQA map", "row gate dropped on S^T k",
                  "row gate dropped on S", "row gate applied by column",
                  "row gate read in reversed row order"]


@pytest.mark.parametrize("name", UPDATE_MUTANTS)
def test_eq2_pins_alone_catch_update_mistakes(tmp_path, name):
    old, new = {m[0]: (m[1], m[2]) for m in MUTANTS}[name]
    src = SRC.read_text()
    assert src.count(old) >= 1, f"mutation site missing: {name}"
    msrc = tmp_path / "mutant.c"
    msrc.write_text(src.replace(old, new))
    mut = oracle_pkg.Oracle(oracle_pkg.compile_oracle(msrc, tmp_path / "libmutant.so"))
    caught = []
    for fn, kw in ((epins.test_mixed_step_equals_eq2, {"d": 16, "n8": 8, "gated": False}),
                   (epins.test_mixed_step_equals_eq2, {"d": 32, "n8": 13, "gated": True}),
                   (epins.test_refit_step_equals_eq2, {"d": 32, "n8": 16}),
                   (epins.test_ragged_step_equals_eq2, {"d": 64, "gated": True}),
                   (epins.test_ragged_step_equals_eq2, {"d": 16, "gated": False})):
        try:
            fn(mut, **kw)
        except (AssertionError, ValueError, FloatingPointError, OverflowError):
            caught.append(fn.__name__)
    assert caught, f"the Eq. (2) pins missed: {name}"
