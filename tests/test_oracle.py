"""Pins for the CPU oracle, each against something other than the oracle itself:
closed forms from the pages' generator, a hand-derived worked example, the
pages' printed tile_dot values, finite differences, identities that hold at any
size, special cases with a textbook answer, and an independent algorithm."""
import numpy as np
import pytest

import oracle
import workloads
from golden.fixtures import load


# ---------------------------------------------------------------- forward ----

@pytest.mark.parametrize("n", [2, 16, 512])
def test_closed_form_factor_is_E(n):
    # jaxmg docs, "Cholesky factorization": A = E E^T must factor to E.
    A, E = workloads.closed_form(n)
    L, info = oracle.potrf(A)
    assert info == 0
    assert np.max(np.abs(L - E)) <= 1e-14
    # entries off the two bands are exactly zero (and so is the strict upper triangle)
    band = np.tril(np.ones((n, n), bool)) & ~np.tril(np.ones((n, n), bool), -2)
    assert np.all(L[~band] == 0.0)


def test_n2_worked_example_forward_exact():
    g = load("n2_worked_example.txt")
    L, info = oracle.potrf(g["A"].reshape(2, 2))
    assert info == 0
    assert np.array_equal(L, g["L"].reshape(2, 2))


def test_n2_generator_matches_fixture():
    A, E = workloads.closed_form(2)
    g = load("n2_worked_example.txt")
    assert np.array_equal(A, g["A"].reshape(2, 2))
    assert np.array_equal(E, g["L"].reshape(2, 2))


@pytest.mark.parametrize("n,seed", [(1, 3), (7, 4), (64, 5), (300, 6)])
def test_residual_random_spd(n, seed):
    A = workloads.gram_spd(n, seed=seed, shift=1.0)
    L, info = oracle.potrf(A)
    assert info == 0
    assert np.all(np.triu(L, 1) == 0.0)
    assert np.all(np.diag(L) > 0)
    res = np.linalg.norm(L @ L.T - A) / np.linalg.norm(A)
    assert res <= 1e-13


def test_diagonal_matrix_gives_sqrt_exactly():
    d = np.array([4.0, 2.0, 9.0, 1e-300, 3.5, 1e300])
    L, info = oracle.potrf(np.diag(d))
    assert info == 0
    assert np.array_equal(L, np.diag(np.sqrt(d)))


def test_scalar_case():
    L, info = oracle.potrf(np.array([[6.25]]))
    assert info == 0 and L[0, 0] == 2.5


def test_only_lower_triangle_is_read():
    A = workloads.gram_spd(20, seed=7)
    B = A.copy()
    B[np.triu_indices(20, 1)] = np.nan
    La, _ = oracle.potrf(A)
    Lb, _ = oracle.potrf(B)
    assert np.array_equal(La, Lb)


@pytest.mark.parametrize("n", [3, 17, 64])
def test_matches_numpy_cholesky(n):
    # third-party sanity check (LAPACK through NumPy), forward only
    A = workloads.gram_spd(n, seed=11, shift=0.5)
    L, info = oracle.potrf(A)
    assert info == 0
    ref = np.linalg.cholesky(A)
    assert np.max(np.abs(L - ref)) <= 1e-12 * np.max(np.abs(ref))


@pytest.mark.parametrize("n,col,val", [(6, 3, -1.0), (6, 0, 0.0), (5, 4, np.nan), (9, 8, -2.0)])
def test_info_first_failing_column(n, col, val):
    A = workloads.spd_with_bad_pivot(n, col, val)
    _, info = oracle.potrf(A)
    assert info == col + 1


def test_info_exact_zero_pivot():
    _, info = oracle.potrf(np.array([[1.0, 1.0], [1.0, 1.0]]))
    assert info == 2


def test_batched_equals_single():
    A = workloads.batched_spd(9, 12, seed=2, dtype=np.float64)
    A[4, 5, 5] = -3.0
    Lb, info = oracle.potrf(A)
    for b in range(9):
        L1, i1 = oracle.potrf(A[b])
        assert i1 == info[b]
        if i1 == 0:
            assert np.array_equal(L1, Lb[b])
    assert info[4] == 6 and np.count_nonzero(info) == 1


# ---------------------------------------------------------------- adjoint ----

def _f(A, adjL):
    L, info = oracle.potrf(A)
    assert info == 0
    return float(np.sum(np.tril(adjL) * L))


@pytest.mark.parametrize("n,seed", [(1, 0), (2, 1), (5, 2), (8, 3)])
def test_adjoint_central_finite_differences(n, seed):
    # f(A) = <adj_L, chol(A)>; perturb each lower entry the forward reads.
    A = workloads.gram_spd(n, seed=seed, shift=1.0)
    adjL = workloads.lower_normal(n, seed=seed + 100)
    L, _ = oracle.potrf(A)
    G = oracle.potrf_adjoint(L, adjL)
    fd = np.zeros_like(A)
    for i in range(n):
        for j in range(i + 1):
            h = 1e-5 * max(1.0, abs(A[i, j]))
            Ap = A.copy(); Ap[i, j] += h
            Am = A.copy(); Am[i, j] -= h
            fd[i, j] = (_f(Ap, adjL) - _f(Am, adjL)) / (2 * h)
    scale = max(1.0, np.max(np.abs(fd)))
    assert np.max(np.abs(np.tril(G) - fd)) <= 1e-7 * scale
    assert np.all(np.triu(G, 1) == 0.0)


@pytest.mark.parametrize("key,pos", [("G_e00", (0, 0)), ("G_e10", (1, 0)), ("G_e11", (1, 1))])
def test_n2_worked_example_adjoint_exact(key, pos):
    g = load("n2_worked_example.txt")
    L = g["L"].reshape(2, 2)
    adjL = np.zeros((2, 2)); adjL[pos] = 1.0
    G = oracle.potrf_adjoint(L, adjL)
    got = np.array([G[0, 0], G[1, 0], G[1, 1]])
    assert np.array_equal(got, g[key])


def test_scalar_adjoint():
    # N = 1: L = sqrt(a), dL/da = 1 / (2 L); pins the diagonal halving of Phi.
    G = oracle.potrf_adjoint(np.array([[2.5]]), np.array([[3.0]]))
    assert G[0, 0] == 3.0 / 5.0


@pytest.mark.parametrize("n", [10, 50])
def test_adjL_equal_L_gives_half_identity(n):
    # <L, L> = tr(A), so the gradient of (1/2)||L||^2 in the lower entries is I / 2.
    A = workloads.gram_spd(n, seed=21)
    L, _ = oracle.potrf(A)
    G = oracle.potrf_adjoint(L, L)
    assert np.max(np.abs(G - 0.5 * np.eye(n))) <= 1e-13


@pytest.mark.parametrize("n,p,q", [(12, 7, 3), (12, 11, 0), (40, 25, 24), (40, 13, 13)])
def test_symmetric_pair_invariant(n, p, q):
    # adj_L = tril(2 W L), W symmetric  =>  G = Phi(2 W).  With W = e_p e_q^T + e_q e_p^T
    # (p > q) that is 2 e_p e_q^T; with p == q and W = e_p e_p^T it is e_p e_p^T.
    A = workloads.gram_spd(n, seed=22)
    L, _ = oracle.potrf(A)
    W = np.zeros((n, n))
    W[p, q] = 1.0
    W[q, p] = 1.0
    adjL = np.tril(2.0 * W @ L)
    G = oracle.potrf_adjoint(L, adjL)
    expect = np.zeros((n, n))
    expect[p, q] = 2.0 if p != q else 1.0
    assert np.max(np.abs(G - expect)) <= 1e-12


def test_adjoint_is_linear_in_adjL():
    n = 30
    A = workloads.gram_spd(n, seed=23)
    L, _ = oracle.potrf(A)
    x = workloads.lower_normal(n, seed=24)
    y = workloads.lower_normal(n, seed=25)
    gx = oracle.potrf_adjoint(L, x)
    gy = oracle.potrf_adjoint(L, y)
    gxy = oracle.potrf_adjoint(L, 2.0 * x - 3.0 * y)
    assert np.max(np.abs(gxy - (2.0 * gx - 3.0 * gy))) <= 1e-12 * np.max(np.abs(gxy))


def test_upper_of_adjL_ignored_and_upper_of_adjA_untouched():
    n = 15
    A = workloads.gram_spd(n, seed=26)
    L, _ = oracle.potrf(A)
    adjL = np.random.default_rng(27).standard_normal((n, n))
    base = np.random.default_rng(28).standard_normal((n, n))
    g1 = oracle.potrf_adjoint(L, adjL, base, accumulate=True)
    g2 = oracle.potrf_adjoint(L, np.tril(adjL), base, accumulate=True)
    assert np.array_equal(g1, g2)
    assert np.array_equal(np.triu(g1, 1), np.triu(base, 1))
    g0 = oracle.potrf_adjoint(L, adjL, base, accumulate=False)
    assert np.array_equal(np.tril(g1), np.tril(g0) + np.tril(base)) or \
        np.max(np.abs(np.tril(g1) - np.tril(g0) - np.tril(base))) <= 1e-13 * np.max(np.abs(g1))
    assert np.array_equal(np.triu(g0, 1), np.triu(base, 1))


@pytest.mark.parametrize("n,seed", [(1, 30), (9, 31), (64, 32), (256, 33)])
def test_formula_matches_independent_sweep(n, seed):
    A = workloads.gram_spd(n, seed=seed, shift=1.0)
    adjL = workloads.lower_normal(n, seed=seed + 1)
    L, _ = oracle.potrf(A)
    g_formula = oracle.potrf_adjoint(L, adjL, method="formula")
    g_sweep = oracle.potrf_adjoint(L, adjL, method="sweep")
    assert np.max(np.abs(g_formula - g_sweep)) <= 1e-12 * np.max(np.abs(g_sweep))


def test_batched_adjoint_equals_single():
    A = workloads.batched_spd(5, 10, seed=3, dtype=np.float64)
    adjL = workloads.lower_normal(10, seed=4, batch=5)
    L, _ = oracle.potrf(A)
    Gb = oracle.potrf_adjoint(L, adjL)
    for b in range(5):
        assert np.array_equal(Gb[b], oracle.potrf_adjoint(L[b], adjL[b]))


# ------------------------------------------------------------- tile_dot ----

def test_tile_dot_values_from_warp_1374():
    g = load("tile_dot_warp1374.txt")
    assert oracle.dot(g["a"], g["b"]) == g["forward"][0]
    abar, bbar = oracle.dot_adjoint(g["a"], g["b"], 1.0)
    assert np.array_equal(abar, g["grad_a"])
    assert np.array_equal(bbar, g["grad_b"])
    assert not np.array_equal(abar, g["grad_a_missing_broadcast"])


# ------------------------------------------------------------------ solve ----
# The solve with the factor (X = A^{-1} B for A = L L^T) and its adjoint, pinned
# against a library solve, closed forms, finite differences and, for the
# adjoint, the matrix-calculus gradient of <C, A^{-1} B> with respect to A.

def _spd_and_factor(n, seed):
    rng = np.random.default_rng(seed)
    G = rng.standard_normal((n, n))
    A = G @ G.T / n + np.eye(n)
    L, info = oracle.potrf(A)
    assert info == 0
    return rng, A, L


@pytest.mark.parametrize("n,nrhs", [(1, 1), (5, 1), (17, 3), (64, 64), (130, 7)])
def test_potrs_matches_library_solve(n, nrhs):
    rng, A, L = _spd_and_factor(n, 10 + n)
    B = rng.standard_normal((n, nrhs))
    X = oracle.potrs(L, B)
    Xref = np.linalg.solve(L @ L.T, B)
    assert np.max(np.abs(X - Xref)) <= 1e-12 * max(1.0, np.max(np.abs(Xref)))
    # and the residual against A itself
    assert np.max(np.abs(A @ X - B)) <= 1e-11 * max(1.0, np.max(np.abs(B)))


def test_potrs_closed_forms():
    rng = np.random.default_rng(4)
    B = rng.standard_normal((6, 2))
    # identity factor: X = B exactly
    assert np.array_equal(oracle.potrs(np.eye(6), B), B)
    # diagonal factor: X_ic = B_ic / d_i^2
    d = np.array([1.0, 2.0, 0.5, 4.0, 3.0, 0.25])
    X = oracle.potrs(np.diag(d), B)
    assert np.max(np.abs(X - B / (d * d)[:, None])) <= 1e-15 * np.max(np.abs(B / (d * d)[:, None]))
    # 1 x 1: x = b / l^2
    assert oracle.potrs(np.array([[3.0]]), np.array([18.0]))[0] == 2.0
    # 2 x 2 by hand: L = [[2, 0], [1, 3]], A = [[4, 2], [2, 10]], b = (6, 14):
    # y = (3, 11/3), x2 = 11/9, x1 = (3 - 11/9) / 2 = 8/9; check A x = b
    x = oracle.potrs(np.array([[2.0, 0.0], [1.0, 3.0]]), np.array([6.0, 14.0]))
    assert np.max(np.abs(x - np.array([8.0 / 9.0, 11.0 / 9.0]))) <= 4e-16


def test_potrs_reads_only_the_lower_triangle():
    rng, A, L = _spd_and_factor(9, 5)
    B = rng.standard_normal((9, 2))
    Lu = L.copy()
    Lu[np.triu_indices(9, 1)] = np.nan
    assert np.array_equal(oracle.potrs(Lu, B), oracle.potrs(L, B))


@pytest.mark.parametrize("n,nrhs", [(1, 1), (3, 2), (6, 3)])
def test_potrs_adjoint_central_finite_differences(n, nrhs):
    rng, A, L = _spd_and_factor(n, 20 + n)
    B = rng.standard_normal((n, nrhs))
    C = rng.standard_normal((n, nrhs))                 # adj_X
    X = oracle.potrs(L, B)
    adjB, adjL = oracle.potrs_adjoint(L, X, C)
    f = lambda L_, B_: float(np.sum(C * oracle.potrs(L_, B_)))
    eps = 1e-6
    for i in range(n):
        for c in range(nrhs):
            Bp, Bm = B.copy(), B.copy()
            Bp[i, c] += eps
            Bm[i, c] -= eps
            fd = (f(L, Bp) - f(L, Bm)) / (2 * eps)
            assert abs(fd - adjB[i, c]) <= 1e-7 * max(1.0, abs(fd))
        for j in range(i + 1):
            Lp, Lm = L.copy(), L.copy()
            Lp[i, j] += eps
            Lm[i, j] -= eps
            fd = (f(Lp, B) - f(Lm, B)) / (2 * eps)
            assert abs(fd - adjL[i, j]) <= 1e-7 * max(1.0, abs(fd))
    assert np.all(np.triu(adjL, 1) == 0.0)


def test_potrs_adjoint_chained_with_factor_adjoint_matches_matrix_calculus():
    # f(A) = <C, A^{-1} B> with A symmetric, parameterised by its lower entries:
    # df/dA = -(A^{-1} C)(A^{-1} B)^T =: -W, so the lower-entry gradient is
    # -(W + W^T) below the diagonal and -W_ii on it.  Chaining the solve's
    # adjoint (adj_L) into the factor's adjoint must give exactly that.
    n, nrhs = 12, 4
    rng, A, L = _spd_and_factor(n, 31)
    B = rng.standard_normal((n, nrhs))
    C = rng.standard_normal((n, nrhs))
    X = oracle.potrs(L, B)
    _, adjL = oracle.potrs_adjoint(L, X, C)
    adjA = oracle.potrf_adjoint(L, adjL)
    W = np.linalg.solve(A, C) @ np.linalg.solve(A, B).T
    want = -(W + W.T)
    want[np.diag_indices(n)] = -np.diag(W)
    want = np.tril(want)
    assert np.max(np.abs(np.tril(adjA) - want)) <= 1e-11 * np.max(np.abs(want))


def test_potrs_adjoint_accumulate_and_overwrite():
    n, nrhs = 7, 2
    rng, A, L = _spd_and_factor(n, 41)
    X = oracle.potrs(L, rng.standard_normal((n, nrhs)))
    C = rng.standard_normal((n, nrhs))
    start = rng.standard_normal((n, n))
    _, g0 = oracle.potrs_adjoint(L, X, C)
    _, acc = oracle.potrs_adjoint(L, X, C, adjL=start, accumulate=True)
    _, ovw = oracle.potrs_adjoint(L, X, C, adjL=start, accumulate=False)
    low = np.tril(np.ones((n, n), bool))
    assert np.allclose(acc[low], start[low] + g0[low], rtol=0, atol=1e-14)
    assert np.array_equal(ovw[low], g0[low])
    assert np.array_equal(acc[~low], start[~low]) and np.array_equal(ovw[~low], start[~low])


# ------------------------------------------------------------ upper factor ----
# uplo = U: A = U^T U from A's upper triangle, and its adjoint.

@pytest.mark.parametrize("n", [1, 2, 7, 64, 200])
def test_upper_factor_against_library_and_residual(n):
    A = workloads.gram_spd(n, seed=60 + n)
    U, info = oracle.potrf_upper(A)
    assert info == 0
    # the library's lower factor, transposed (a textbook identity: U = L^T)
    assert np.max(np.abs(U - np.linalg.cholesky(A).T)) <= 1e-12 * np.max(np.abs(U))
    assert np.all(np.tril(U, -1) == 0.0) and np.all(np.diag(U) > 0)
    assert np.max(np.abs(U.T @ U - A)) <= 1e-13 * np.max(np.abs(A))


def test_upper_factor_closed_form_and_upper_only():
    A, E = workloads.closed_form(16)
    U, info = oracle.potrf_upper(A)
    assert info == 0 and np.max(np.abs(U - E.T)) <= 1e-14
    Al = A.copy()
    Al[np.tril_indices(16, -1)] = np.nan               # the lower triangle is never read
    assert np.array_equal(oracle.potrf_upper(Al)[0], U)
    bad = A.copy()
    bad[5, 5] = -1.0                                   # pivot 6 fails, as in the lower form
    assert oracle.potrf_upper(bad)[1] == 6


@pytest.mark.parametrize("n", [1, 3, 5])
def test_upper_adjoint_central_finite_differences(n):
    A = workloads.gram_spd(n, seed=70 + n)
    U, _ = oracle.potrf_upper(A)
    rng = np.random.default_rng(71)
    adjU = np.triu(rng.standard_normal((n, n)))
    G = oracle.potrf_adjoint_upper(U, adjU)
    f = lambda M: float(np.sum(adjU * oracle.potrf_upper(M)[0]))
    eps = 1e-6
    for i in range(n):
        for j in range(i, n):
            # perturb the upper entry only: the lower triangle is not read
            Ap, Am = A.copy(), A.copy()
            Ap[i, j] += eps
            Am[i, j] -= eps
            fd = (f(Ap) - f(Am)) / (2 * eps)
            assert abs(fd - G[i, j]) <= 1e-7 * max(1.0, abs(fd))
    assert np.all(np.tril(G, -1) == 0.0)


def test_upper_adjoint_ignores_lower_inputs_and_keeps_lower_output():
    n = 9
    A = workloads.gram_spd(n, seed=81)
    U, _ = oracle.potrf_upper(A)
    rng = np.random.default_rng(82)
    adjU = np.triu(rng.standard_normal((n, n)))
    start = rng.standard_normal((n, n))
    G0 = oracle.potrf_adjoint_upper(U, adjU)
    Un, aUn = U.copy(), adjU.copy()
    Un[np.tril_indices(n, -1)] = np.nan
    aUn[np.tril_indices(n, -1)] = np.nan
    G = oracle.potrf_adjoint_upper(Un, aUn, adjA=start, accumulate=True)
    up = np.triu(np.ones((n, n), bool))
    assert np.allclose(G[up], start[up] + G0[up], rtol=0, atol=1e-14)
    assert np.array_equal(G[~up], start[~up])


def test_sum_closed_form_and_adjoint():
    # y = sum a, a_bar = y_bar everywhere; with a = 1..16 (the repro's vector) y = 136
    a = np.arange(1.0, 17.0)
    assert oracle.wsum(a) == 136.0
    assert oracle.wsum(np.array([])) == 0.0
    assert np.array_equal(oracle.wsum_adjoint(16, 2.5), np.full(16, 2.5))
    # central differences on a random vector
    rng = np.random.default_rng(5)
    v = rng.standard_normal(9)
    g = oracle.wsum_adjoint(9, 1.0)
    for k in range(9):
        e = np.zeros(9); e[k] = 1e-3
        assert abs((oracle.wsum(v + e) - oracle.wsum(v - e)) / 2e-3 - g[k]) <= 1e-12


# ------------------------------------------------------- Hermitian complex ----
# A = L L^H (complex128) and its adjoint, gradients as d/dRe + i d/dIm.

def _herm(n, seed):
    rng = np.random.default_rng(seed)
    G = rng.standard_normal((n, n)) + 1j * rng.standard_normal((n, n))
    A = G @ G.conj().T / n + np.eye(n)
    return rng, (A + A.conj().T) / 2


@pytest.mark.parametrize("n", [1, 2, 9, 100])
def test_complex_factor_against_library(n):
    rng, A = _herm(n, 90 + n)
    L, info = oracle.zpotrf(A)
    assert info == 0
    assert np.max(np.abs(L - np.linalg.cholesky(A))) <= 1e-12 * np.max(np.abs(L))
    assert np.all(np.triu(L, 1) == 0) and np.all(np.diag(L).imag == 0) and np.all(np.diag(L).real > 0)
    assert np.max(np.abs(L @ L.conj().T - A)) <= 1e-13 * np.max(np.abs(A))


def test_complex_factor_special_cases():
    # a closed form: A = E E^H with E lower, real positive diagonal, complex subdiagonal
    n = 12
    E = np.diag(np.linspace(1.0, 2.0, n)).astype(complex)
    E[np.arange(1, n), np.arange(n - 1)] = 0.5 - 0.25j
    L, info = oracle.zpotrf(E @ E.conj().T)
    assert info == 0 and np.max(np.abs(L - E)) <= 1e-14
    # real input: exactly the real factor
    _, A = _herm(8, 3)
    Ar = A.real.copy()
    Ar = (Ar + Ar.T) / 2 + 0 * np.eye(8)
    Lr, _ = oracle.potrf(Ar)
    assert np.array_equal(oracle.zpotrf(Ar.astype(complex))[0], Lr.astype(complex))
    # only the lower triangle and the real part of the diagonal are read
    Ap = A.copy()
    Ap[np.triu_indices(8, 1)] = np.nan
    Ap[np.diag_indices(8)] += 5j
    assert np.array_equal(oracle.zpotrf(Ap)[0], oracle.zpotrf(A)[0])
    bad = A.copy()
    bad[4, 4] = -1.0
    assert oracle.zpotrf(bad)[1] == 5


@pytest.mark.parametrize("n", [1, 3, 5])
def test_complex_adjoint_central_finite_differences(n):
    rng, A = _herm(n, 95 + n)
    L, _ = oracle.zpotrf(A)
    aL = np.tril(rng.standard_normal((n, n)) + 1j * rng.standard_normal((n, n)))
    G = oracle.zpotrf_adjoint(L, aL)
    f = lambda M: float(np.real(np.sum(np.conj(aL) * oracle.zpotrf(M)[0])))
    eps = 1e-6
    for i in range(n):
        for j in range(i + 1):
            for part in ((1.0,) if i == j else (1.0, 1j)):
                Ap, Am = A.copy(), A.copy()
                Ap[i, j] += eps * part
                Am[i, j] -= eps * part
                fd = (f(Ap) - f(Am)) / (2 * eps)
                got = G[i, j].real if part == 1.0 else G[i, j].imag
                assert abs(fd - got) <= 1e-7 * max(1.0, abs(fd)), (i, j, part)
    assert np.all(np.diag(G).imag == 0) and np.all(np.triu(G, 1) == 0)


def test_complex_adjoint_invariants():
    rng, A = _herm(10, 97)
    L, _ = oracle.zpotrf(A)
    # adj_L = L gives half the identity, as in the real case
    assert np.max(np.abs(oracle.zpotrf_adjoint(L, L) - 0.5 * np.eye(10))) <= 1e-14
    # real factor and real adj_L: the real adjoint
    Ar = A.real.copy()
    Lr, _ = oracle.potrf((Ar + Ar.T) / 2)
    aL = np.tril(rng.standard_normal((10, 10)))
    assert np.max(np.abs(oracle.zpotrf_adjoint(Lr, aL) - oracle.potrf_adjoint(Lr, aL))) <= 1e-14
    # linear in adj_L over the reals, and accumulate / overwrite
    aL1 = np.tril(rng.standard_normal((10, 10)) + 1j * rng.standard_normal((10, 10)))
    aL2 = np.tril(rng.standard_normal((10, 10)) + 1j * rng.standard_normal((10, 10)))
    g1, g2 = oracle.zpotrf_adjoint(L, aL1), oracle.zpotrf_adjoint(L, aL2)
    assert np.max(np.abs(oracle.zpotrf_adjoint(L, 2 * aL1 - aL2) - (2 * g1 - g2))) <= 1e-13
    start = rng.standard_normal((10, 10)) + 1j * rng.standard_normal((10, 10))
    acc = oracle.zpotrf_adjoint(L, aL1, adjA=start, accumulate=True)
    ovw = oracle.zpotrf_adjoint(L, aL1, adjA=start, accumulate=False)
    low = np.tril(np.ones((10, 10), bool))
    assert np.allclose(acc[low], start[low] + g1[low], rtol=0, atol=1e-14)
    assert np.array_equal(ovw[low], g1[low]) and np.array_equal(acc[~low], start[~low])
