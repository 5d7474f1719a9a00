"""The pins must catch plausible mistakes in the oracle.

Each case copies the oracle's C source, plants one mistake by a text
substitution (a flipped sign, a transposed index, a dropped term, a changed
tie rule, ...), builds the copy with the same compiler flags and runs a fast
selection of the pins against it: at least one must fail.  The unmodified
copy must pass the same selection.  Everything here runs on the CPU.
"""
from __future__ import annotations

import os
import shutil

import numpy as np
import pytest

import oracle
import test_oracle_pins as pins

SRC_DIR = os.path.dirname(oracle.__file__)
IMPL = "gesv_oracle_impl.h"

MUTANTS = {
    "update_sign": ("FMA(-l, M[(size_t)k * n + c], M[(size_t)r * n + c])",
                    "FMA(l, M[(size_t)k * n + c], M[(size_t)r * n + c])"),
    "update_transposed": ("FMA(-l, M[(size_t)k * n + c], M[(size_t)r * n + c])",
                          "FMA(-l, M[(size_t)c * n + k], M[(size_t)r * n + c])"),
    "rhs_update_dropped": ("Y[(size_t)r * nrhs + j] = FMA(-l, Y[(size_t)k * nrhs + j], "
                           "Y[(size_t)r * nrhs + j]);",
                           "(void)0;"),
    "rhs_swap_dropped": ("SFX(swap_rows)(Y, nrhs, k, p);", "(void)0;"),
    "tie_to_last": ("if (SFX(ranks_above)(v, m)) {", "if (SFX(ranks_above)(v, m) || v == m) {"),
    "candidate_skipped": ("for (int r = k + 1; r < n; ++r) {\n        REAL v = FABS",
                          "for (int r = k + 2; r < n; ++r) {\n        REAL v = FABS"),
    "reciprocal_multiplier": ("const REAL l = M[(size_t)r * n + k] / d;",
                              "const REAL l = M[(size_t)r * n + k] * ((REAL)1 / d);"),
    "backsub_transposed": ("FMA(-M[(size_t)r * n + k], Y[(size_t)k * nrhs + j]",
                           "FMA(-M[(size_t)k * n + r], Y[(size_t)k * nrhs + j]"),
    "backsub_no_division": ("Y[(size_t)k * nrhs + j] = Y[(size_t)k * nrhs + j] / ukk;",
                            "Y[(size_t)k * nrhs + j] = Y[(size_t)k * nrhs + j];"),
    "colmajor_as_rowmajor": ("? a[(size_t)r * n + c] : a[(size_t)c * n + r]",
                             "? a[(size_t)r * n + c] : a[(size_t)r * n + c]"),
    "info_zero_based": ("info = k + 1;\n            break;", "info = k;\n            break;"),
    "failed_piv_kept": ("piv[r] = -1;", "(void)0;"),
    "lu_multiplier_not_stored": ("lu[(size_t)r * n + k] = l;\n", "(void)l;\n"),
    "getrs_swaps_reversed": ("for (int k = 0; k < n; ++k)\n        if (ipiv[k] != k)",
                             "for (int k = n - 1; k >= 0; --k)\n        if (ipiv[k] != k)"),
    "getrs_lower_transposed": ("const REAL l = SFX(load_a)(lu, layout, n, r, k);",
                               "const REAL l = SFX(load_a)(lu, layout, n, k, r);"),
    "getrs_upper_transposed": ("const REAL u = SFX(load_a)(lu, layout, n, r, k);",
                               "const REAL u = SFX(load_a)(lu, layout, n, k, r);"),
    "getrs_unit_diagonal_divided": (
        "    for (int k = 0; k < n; ++k)\n        for (int r = k + 1; r < n; ++r) {",
        "    for (int k = 0; k < n; ++k)\n        for (int r = k + 1 + 0 * (int)(Y[(size_t)k * nrhs] "
        "/= SFX(load_a)(lu, layout, n, k, k)); r < n; ++r) {"),
    "chol_diag_sign": ("s = FMA(-L[(size_t)j * n + k], L[(size_t)j * n + k], s);",
                       "s = FMA(L[(size_t)j * n + k], L[(size_t)j * n + k], s);"),
    "chol_offdiag_transposed": ("t = FMA(-L[(size_t)i * n + k], L[(size_t)j * n + k], t);",
                                "t = FMA(-L[(size_t)k * n + i], L[(size_t)j * n + k], t);"),
    "chol_no_sqrt": ("const REAL d = SQRT(s);", "const REAL d = s;"),
    "chol_wrong_column": ("REAL t = SFX(load_a)(a, layout, n, i, j);",
                          "REAL t = SFX(load_a)(a, layout, n, i, (j + 1) % n);"),
    "chol_status_zero_based": ("if (!(s > 0))\n            return j + 1;",
                               "if (!(s > 0))\n            return j;"),
    "chol_no_symmetry_check": ("                return -2;", "                (void)0;"),
    "chol_shift_ignored": ("REAL s = SFX(load_a)(a, layout, n, j, j) + shift;",
                           "REAL s = SFX(load_a)(a, layout, n, j, j);"),
    "chol_back_transposed": ("FMA(-L[(size_t)k * n + i], Y[(size_t)k * nrhs + j], "
                             "Y[(size_t)i * nrhs + j]);\n    }\n    if (!SFX(all_finite)",
                             "FMA(-L[(size_t)i * n + k], Y[(size_t)k * nrhs + j], "
                             "Y[(size_t)i * nrhs + j]);\n    }\n    if (!SFX(all_finite)"),
    "nan_never_wins": ("    if (isnan(v))\n        return !isnan(m);\n", ""),
    "input_check_dropped": ("        info = -1;\n    else if (scale)", "        info = 0;\n    else if (scale)"),
    "factor_check_dropped": ("        info = -3; /* L, U or y */", "        info = 0;"),
    "solution_check_dropped": ("            info = -3; /* x */", "            info = 0;"),
    "getrf_check_dropped": ("    if (info == 0 && !SFX(all_finite)(lu, (size_t)n * n))\n        info = -3;",
                            "    (void)0;"),
    "scale_rhs_not_scaled": ("        Y[e] = Y[e] / s;", "        Y[e] = Y[e];"),
    "scale_u_not_restored": ("lu[(size_t)r * n + c] = lu[(size_t)r * n + c] * sc;",
                             "lu[(size_t)r * n + c] = lu[(size_t)r * n + c];"),
    "scale_signed_max": ("        if (FABS(M[e]) > s)\n            s = FABS(M[e]);",
                         "        if (M[e] > s)\n            s = M[e];"),
    "chol_input_check_dropped": ("    if (!SFX(all_finite)(a, (size_t)n * n))\n        return -1;", ""),
    "chol_factor_check_dropped": ("    return SFX(all_finite)(L, (size_t)n * n) ? 0 : -3;",
                                  "    return 0;"),
    "posv_solution_check_dropped": ("        SFX(zero_rhs)(layout, n, nrhs, x); /* x */\n        return -3;",
                                    "        (void)0;"),
    "potrs_back_transposed": ("const REAL lki = SFX(load_a)(l, layout, n, k, i);",
                              "const REAL lki = SFX(load_a)(l, layout, n, i, k);"),
    "potrs_forward_no_division": (
        "        const REAL d = SFX(load_a)(l, layout, n, k, k);\n        for (int j = 0; j < nrhs; ++j)\n"
        "            Y[(size_t)k * nrhs + j] = Y[(size_t)k * nrhs + j] / d;\n        for (int i = k + 1;",
        "        const REAL d = SFX(load_a)(l, layout, n, k, k);\n        for (int j = 0; j < nrhs; ++j)\n"
        "            Y[(size_t)k * nrhs + j] = Y[(size_t)k * nrhs + j] + 0 * d;\n        for (int i = k + 1;"),
    "potrs_failed_not_detected": ("    if (SFX(load_a)(l, layout, n, 0, 0) == 0) {",
                                  "    if (0) {"),
    "getrs_failed_negative_zero": (
        "x[SFX(rhs_index)(layout, n, nrhs, r, j)] = (REAL)0;\n        return;",
        "x[SFX(rhs_index)(layout, n, nrhs, r, j)] = -(REAL)0;\n        return;"),
}


def _selection():
    """A fast subset of the pins, enough to cover every step."""
    yield lambda: pins.test_golden_examples(np.float64, "row", None)
    yield lambda: pins.test_golden_examples(np.float32, "col", 8)
    yield lambda: pins.test_lapack_pivots(np.float64, "row")
    yield lambda: pins.test_lapack_pivots(np.float32, "col")
    yield lambda: pins.test_reconstruction_bound(np.float64, "row")
    yield lambda: pins.test_exact_singularity_constructions(np.float64, "row")
    yield lambda: pins.test_exact_singularity_constructions(np.float32, "col")
    yield lambda: pins.test_cramer_exact(np.float64, "col", 3)
    yield lambda: pins.test_getrs_exact_integer_factors(np.float64, "row")
    yield lambda: pins.test_getrs_exact_integer_factors(np.float32, "col")
    yield lambda: pins.test_getrs_failed_factorization_gives_zero(np.float64)
    yield lambda: pins.test_cholesky_exact_integer_factors(np.float64, "row")
    yield lambda: pins.test_cholesky_exact_integer_factors(np.float32, "col")
    yield lambda: pins.test_cholesky_symmetry_and_shift(np.float64)
    yield lambda: pins.test_cholesky_first_failing_minor()
    yield lambda: pins.test_nonfinite_input_status(np.float64, "row")
    yield lambda: pins.test_overflow_gives_minus3(np.float32, "col")
    yield lambda: pins.test_nan_candidate_ranks_above_zero(np.float64)
    yield lambda: pins.test_scaling_by_power_of_two_is_exact(np.float64, "row")
    yield lambda: pins.test_scaling_general(np.float64)
    yield lambda: pins.test_cholesky_nonfinite_statuses(np.float32)
    yield lambda: pins.test_potrs_exact_integer_factors(np.float64, "col")
    yield lambda: pins.test_potrs_matches_lapack_and_posv(np.float64)


def _build_variant(tmp_path, name, mutation):
    d = tmp_path / name
    d.mkdir()
    for f in ("gesv_oracle.c", IMPL):
        shutil.copy(os.path.join(SRC_DIR, f), d / f)
    if mutation is not None:
        old, new = mutation
        text = (d / IMPL).read_text(encoding="utf-8")
        assert text.count(old) >= 1, f"mutation site of {name} not found"
        (d / IMPL).write_text(text.replace(old, new, 1), encoding="utf-8")
    return oracle.build(source_dir=str(d), out=str(d / "lib.so"))


def _failures(lib_path):
    failed = []
    with oracle.use_library(lib_path):
        for i, check in enumerate(_selection()):
            try:
                check()
            except AssertionError:
                failed.append(i)
    return failed


def test_unmodified_copy_passes(tmp_path):
    assert _failures(_build_variant(tmp_path, "control", None)) == []


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(tmp_path, name):
    failed = _failures(_build_variant(tmp_path, name, MUTANTS[name]))
    assert failed, f"no pin caught the planted mistake {name}"
