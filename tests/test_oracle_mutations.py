"""Plant plausible mistakes in copies of the oracle's C source (CPU only) and
check that the pins in ``test_oracle.py`` catch every one of them.  This shows
the pins are sensitive to a dropped term, a wrong sign, a wrong index or a
transposed operand anywhere in the oracle."""
import os
import subprocess

import pytest

import oracle
import test_oracle as pins

SRC = os.path.join(os.path.dirname(oracle.__file__), "oracle.c")

# (name, text in oracle.c, replacement).  Each replacement is a mistake that
# still compiles and still produces finite numbers.
MUTATIONS = [
    ("fwd_pivot_sign", "d -= AT(L, ldl, j, k) * AT(L, ldl, j, k);",
     "d += AT(L, ldl, j, k) * AT(L, ldl, j, k);"),
    ("fwd_row_index", "s -= AT(L, ldl, i, k) * AT(L, ldl, j, k);",
     "s -= AT(L, ldl, i, k) * AT(L, ldl, i, k);"),
    ("fwd_no_divide", "AT(L, ldl, i, j) = s / ljj;", "AT(L, ldl, i, j) = s;"),
    ("fwd_pivot_no_sqrt", "const double ljj = sqrt(d);", "const double ljj = d;"),
    ("adj_M_transposed", "const double lki = AT(L, ldl, k, i);",
     "const double lki = AT(L, ldl, i, k);"),
    ("adj_M_uses_upper_adjL", "mrow[j] += lki * AT(adjL, ldal, k, j);",
     "mrow[j] += lki * AT(adjL, ldal, j, k);"),
    ("adj_phi_no_halving", "M[(size_t)i * n + i] *= 0.5;", "M[(size_t)i * n + i] *= 1.0;"),
    ("adj_solve1_no_divide", "xi[c] = ri[c] / lii;", "xi[c] = ri[c];"),
    ("adj_solve1_wrong_sign", "rt[c] -= lit * xi[c];", "rt[c] += lit * xi[c];"),
    ("adj_solve1_transposed", "const double lit = AT(L, ldl, i, t);",
     "const double lit = AT(L, ldl, t, i);"),
    ("adj_solve2_transposed", "rr[k] -= srj * AT(L, ldl, j, k);",
     "rr[k] -= srj * AT(L, ldl, k, j);"),
    ("adj_solve2_no_divide", "const double srj = rr[j] / AT(L, ldl, j, j);",
     "const double srj = rr[j];"),
    ("adj_sym_half_offdiag", ": S[(size_t)i * n + j] + S[(size_t)j * n + i];",
     ": 0.5 * (S[(size_t)i * n + j] + S[(size_t)j * n + i]);"),
    ("adj_sym_lower_only", ": S[(size_t)i * n + j] + S[(size_t)j * n + i];",
     ": S[(size_t)i * n + j];"),
    ("adj_diag_doubled", "const double g = (i == j) ? S[(size_t)i * n + i]",
     "const double g = (i == j) ? 2.0 * S[(size_t)i * n + i]"),
    ("adj_overwrites_when_accumulating", "AT(adjA, ldaa, i, j) += g;", "AT(adjA, ldaa, i, j) = g;"),
    ("dot_reversed_index", "y += a[k] * b[k];", "y += a[k] * b[n - 1 - k];"),
    ("upper_reads_lower", "At[(size_t)i * n + j] = AT(A, lda, j, i);",
     "At[(size_t)i * n + j] = AT(A, lda, i, j);"),
    ("upper_not_transposed_back", "AT(U, ldu, i, j) = (j >= i) ? L[(size_t)j * n + i] : 0.0;",
     "AT(U, ldu, i, j) = (j >= i) ? L[(size_t)i * n + j] : 0.0;"),
    ("upper_adj_not_transposed", "const double g = G[(size_t)j * n + i];",
     "const double g = G[(size_t)i * n + j];"),
    ("upper_adj_uses_lower_adjU", "aL[(size_t)i * n + j] = AT(adjU, ldau, j, i);",
     "aL[(size_t)i * n + j] = AT(adjU, ldau, i, j);"),
    ("zpotrf_no_conj", "s -= ZAT(L, ldl, i, k) * conj(ZAT(L, ldl, j, k));",
     "s -= ZAT(L, ldl, i, k) * ZAT(L, ldl, j, k);"),
    ("zadj_M_no_conj", "const double complex lki = conj(ZAT(L, ldl, k, i));",
     "const double complex lki = ZAT(L, ldl, k, i);"),
    ("zadj_phi_no_halving", "M[(size_t)i * n + i] = 0.5 * creal(M[(size_t)i * n + i]);",
     "M[(size_t)i * n + i] = creal(M[(size_t)i * n + i]);"),
    ("zadj_solve1_no_conj", "s -= conj(ZAT(L, ldl, t, i)) * X[(size_t)t * n + c];",
     "s -= ZAT(L, ldl, t, i) * X[(size_t)t * n + c];"),
    ("zadj_sym_no_conj", ": S[(size_t)i * n + j] + conj(S[(size_t)j * n + i]);",
     ": S[(size_t)i * n + j] + S[(size_t)j * n + i];"),
    ("potrs_forward_sign", "s -= AT(L, ldl, i, k) * AT(X, ldx, k, c);",
     "s += AT(L, ldl, i, k) * AT(X, ldx, k, c);"),
    ("potrs_back_not_transposed", "s -= AT(L, ldl, k, i) * AT(X, ldx, k, c);",
     "s -= AT(L, ldl, i, k) * AT(X, ldx, k, c);"),
    ("potrs_one_solve_only", "        for (int64_t i = n - 1; i >= 0; --i) {\n            double s = AT(X, ldx, i, c);",
     "        for (int64_t i = n - 1; i >= n; --i) {\n            double s = AT(X, ldx, i, c);"),
    ("potrs_adj_one_sided_W",
     "w += AT(adjB, ldab, i, c) * AT(X, ldx, k, c) + AT(X, ldx, i, c) * AT(adjB, ldab, k, c);",
     "w += AT(adjB, ldab, i, c) * AT(X, ldx, k, c);"),
    ("potrs_adj_sign", "AT(adjL, ldal, i, j) -= g;", "AT(adjL, ldal, i, j) += g;"),
    ("potrs_adj_L_transposed", "g += W[(size_t)i * n + k] * AT(L, ldl, k, j);",
     "g += W[(size_t)i * n + k] * AT(L, ldl, j, k);"),
    ("dot_adjoint_swapped", "abar[k] += ybar * b[k];", "abar[k] += ybar * a[k];"),
    ("sum_skips_last", "for (int64_t k = 0; k < n; ++k)\n        y += a[k];", "for (int64_t k = 0; k + 1 < n; ++k)\n        y += a[k];"),
    ("sum_adjoint_halved", "abar[k] += ybar;", "abar[k] += 0.5 * ybar;"),
]

PINS = [
    lambda: pins.test_closed_form_factor_is_E(16),
    pins.test_n2_worked_example_forward_exact,
    lambda: pins.test_residual_random_spd(64, 5),
    pins.test_diagonal_matrix_gives_sqrt_exactly,
    pins.test_scalar_case,
    lambda: pins.test_adjoint_central_finite_differences(5, 2),
    lambda: pins.test_n2_worked_example_adjoint_exact("G_e10", (1, 0)),
    lambda: pins.test_n2_worked_example_adjoint_exact("G_e11", (1, 1)),
    pins.test_scalar_adjoint,
    lambda: pins.test_adjL_equal_L_gives_half_identity(10),
    lambda: pins.test_symmetric_pair_invariant(12, 7, 3),
    pins.test_upper_of_adjL_ignored_and_upper_of_adjA_untouched,
    pins.test_tile_dot_values_from_warp_1374,
    lambda: pins.test_potrs_matches_library_solve(17, 3),
    pins.test_potrs_closed_forms,
    lambda: pins.test_potrs_adjoint_central_finite_differences(6, 3),
    pins.test_potrs_adjoint_chained_with_factor_adjoint_matches_matrix_calculus,
    lambda: pins.test_upper_factor_against_library_and_residual(7),
    pins.test_upper_factor_closed_form_and_upper_only,
    lambda: pins.test_upper_adjoint_central_finite_differences(3),
    pins.test_upper_adjoint_ignores_lower_inputs_and_keeps_lower_output,
    pins.test_sum_closed_form_and_adjoint,
    lambda: pins.test_complex_factor_against_library(9),
    pins.test_complex_factor_special_cases,
    lambda: pins.test_complex_adjoint_central_finite_differences(5),
    pins.test_complex_adjoint_invariants,
]


def _caught(lib_path):
    with oracle._use_library(lib_path):
        for pin in PINS:
            try:
                pin()
            except Exception:  # an assertion, or any failure the mistake causes
                return True
    return False


def test_unmutated_copy_passes_every_pin(tmp_path):
    out = tmp_path / "liboracle_copy.so"
    subprocess.run(["gcc", "-O2", "-std=c11", "-fopenmp", "-ffp-contract=off", "-fPIC", "-shared",
                    SRC, "-o", str(out), "-lm"], check=True)
    assert not _caught(str(out))


@pytest.mark.parametrize("name,old,new", MUTATIONS, ids=[m[0] for m in MUTATIONS])
def test_planted_mistake_is_caught(tmp_path, name, old, new):
    text = open(SRC).read()
    assert text.count(old) == 1, f"mutation anchor for {name} not unique in oracle.c"
    src = tmp_path / "oracle_mut.c"
    src.write_text(text.replace(old, new))
    out = tmp_path / "liboracle_mut.so"
    subprocess.run(["gcc", "-O2", "-std=c11", "-fopenmp", "-ffp-contract=off", "-fPIC", "-shared",
                    str(src), "-o", str(out), "-lm"], check=True)
    assert _caught(str(out)), f"no pin caught the planted mistake {name}"
