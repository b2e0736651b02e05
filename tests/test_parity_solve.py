"""GPU parity of the solve with the factor (chol_potrs*) and its adjoint
against the CPU oracle, through the C-ABI.  Both sides get the same factor L
(the oracle's, cast to the working dtype) and the same right-hand sides.
Tolerances: fp64 1e-10, fp32 2e-4 (relative, atol = rtol * max|oracle| per
matrix), as for the factor; inputs are well conditioned (A = G G^T / n + I)
except where a condition number is named."""
import numpy as np
import pytest

import oracle
import workloads
from parity_util import assert_close

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

RTOL = {np.float64: 1e-10, np.float32: 2e-4}


def dc():
    import differentiable_cholesky_amd
    return differentiable_cholesky_amd


def dev(x):
    return torch.from_numpy(np.ascontiguousarray(x)).cuda()


def host(t):
    torch.cuda.synchronize()
    return t.cpu().numpy()


def _factor(n, seed, dt, batch=None):
    if batch is None:
        A = workloads.gram_spd(n, seed=seed)
        L, info = oracle.potrf(A)
        assert info == 0
    else:
        A = workloads.batched_spd(batch, n, seed=seed, dtype=np.float64)
        L, info = oracle.potrf(A)
        assert np.all(info == 0)
    # the working-precision factor is what both sides solve with
    return L.astype(dt)


# ------------------------------------------------------------ batched, n <= 64 ----

@pytest.mark.parametrize("dt", [np.float64, np.float32])
@pytest.mark.parametrize("n,nrhs", [(1, 1), (5, 3), (8, 8), (16, 9), (17, 1), (32, 20), (33, 2), (64, 8),
                                    (64, 17)])
def test_batched_solve_and_adjoint(n, nrhs, dt):
    batch = 37
    L = _factor(n, 100 + n, dt, batch)
    B = workloads.normal_rhs(n, nrhs, seed=3, batch=batch, dtype=dt)
    X = host(dc().chol_potrs_batched(dev(L), dev(B)))
    Xo = oracle.potrs(L, B)
    for b in range(batch):
        assert_close(X[b], Xo[b], RTOL[dt], f"X[{b}]")
    adjX = workloads.normal_rhs(n, nrhs, seed=4, batch=batch, dtype=dt)
    start = workloads.lower_normal(n, seed=5, batch=batch, dtype=dt) + np.triu(np.ones((n, n), dt), 1)
    for acc in (True, False):
        aB, aL = dc().chol_potrs_adjoint_batched(dev(L), dev(X), dev(adjX), adjL=dev(start), accumulate=acc)
        aB, aL = host(aB), host(aL)
        aBo, aLo = oracle.potrs_adjoint(L, X, adjX, adjL=start, accumulate=acc)
        for b in range(batch):
            assert_close(aB[b], aBo[b], RTOL[dt], f"adj_B[{b}]")
            # the oracle's output keeps the start's strict upper triangle; so must the GPU's
            assert_close(aL[b], aLo[b], RTOL[dt], f"adj_L[{b}] acc={acc}")
        assert np.array_equal(np.triu(aL, 1), np.triu(start, 1))


@pytest.mark.parametrize("dt", [np.float64, np.float32])
def test_batched_in_place_and_strided(dt):
    n, nrhs, batch = 24, 5, 9
    L = _factor(n, 7, dt, batch)
    B = workloads.normal_rhs(n, nrhs, seed=8, batch=batch, dtype=dt)
    Xo = oracle.potrs(L, B)
    # in place: X is B
    Bd = dev(B)
    out = dc().chol_potrs_batched(dev(L), Bd, X=Bd)
    assert out.data_ptr() == Bd.data_ptr()
    for b in range(batch):
        assert_close(host(Bd)[b], Xo[b], RTOL[dt], f"in place X[{b}]")
    # padded rows and batch strides on every array
    Lp = torch.zeros(batch, n, n + 3, dtype=dev(L).dtype, device="cuda")[:, :, :n]
    Lp.copy_(dev(L))
    Bp = torch.zeros(batch, n, nrhs + 6, dtype=Lp.dtype, device="cuda")[:, :, 2:2 + nrhs]
    Bp.copy_(dev(B))
    Xp = torch.full((batch, n, nrhs + 1), 7.0, dtype=Lp.dtype, device="cuda")[:, :, :nrhs]
    dc().chol_potrs_batched(Lp, Bp, X=Xp)
    full = host(Xp.as_strided((batch, n, nrhs + 1), Xp.stride()))
    for b in range(batch):
        assert_close(full[b, :, :nrhs], Xo[b], RTOL[dt], f"strided X[{b}]")
    assert np.all(full[:, :, nrhs] == 7.0)        # the padding column is not written


@pytest.mark.parametrize("dt", [np.float64, np.float32])
def test_single_small_solve_through_potrs(dt):
    for n in (1, 2, 40, 64):
        L = _factor(n, 50 + n, dt)
        b = workloads.normal_rhs(n, 1, seed=9, dtype=dt)[:, 0]
        x = host(dc().chol_potrs(dev(L), dev(b)))
        assert_close(x[:, None], oracle.potrs(L, b)[:, None], RTOL[dt], f"x n={n}")


# ---------------------------------------------------------------- blocked ----

@pytest.mark.parametrize("dt", [np.float64, np.float32])
@pytest.mark.parametrize("n,nrhs,nb", [(65, 1, 0), (100, 3, 32), (129, 1, 0), (300, 7, 64), (520, 130, 96),
                                       (1000, 16, 0), (1030, 1, 128), (400, 64, 0), (400, 65, 0)])
def test_blocked_solve_and_adjoint(n, nrhs, nb, dt):
    L = _factor(n, 200 + n, dt)
    B = workloads.normal_rhs(n, nrhs, seed=11, dtype=dt)
    X = host(dc().chol_potrs(dev(L), dev(B), nb=nb))
    Xo = oracle.potrs(L, B)
    assert_close(X, Xo, RTOL[dt], "X")
    adjX = workloads.normal_rhs(n, nrhs, seed=12, dtype=dt)
    start = workloads.lower_normal(n, seed=13, dtype=dt) + np.triu(np.full((n, n), 3.0, dt), 1)
    for acc in (True, False):
        aB, aL = dc().chol_potrs_adjoint(dev(L), dev(X), dev(adjX), adjL=dev(start), accumulate=acc, nb=nb)
        aB, aL = host(aB), host(aL)
        aBo, aLo = oracle.potrs_adjoint(L, X, adjX, adjL=start, accumulate=acc)
        assert_close(aB, aBo, RTOL[dt], "adj_B")
        assert_close(np.tril(aL), np.tril(aLo), RTOL[dt], f"adj_L acc={acc}")
        assert np.array_equal(np.triu(aL, 1), np.triu(start, 1))


def test_blocked_solve_in_place_vector_and_adjoint_in_place():
    n = 700
    L = _factor(n, 5, np.float64)
    b = workloads.normal_rhs(n, 1, seed=2)[:, 0]
    bd = dev(b)
    dc().chol_potrs(dev(L), bd, X=bd)
    xo = oracle.potrs(L, b)
    assert_close(host(bd)[:, None], xo[:, None], 1e-10, "x in place")
    # adj_B written over adj_X
    g = workloads.normal_rhs(n, 1, seed=6)[:, 0]
    gd = dev(g)
    aB, aL = dc().chol_potrs_adjoint(dev(L), dev(xo), gd, adjB=gd, accumulate=False)
    aBo, aLo = oracle.potrs_adjoint(L, xo, g, accumulate=False)
    assert aB.data_ptr() == gd.data_ptr()
    assert_close(host(aB)[:, None], aBo[:, None], 1e-10, "adj_B in place")
    assert_close(np.tril(host(aL)), np.tril(aLo), 1e-10, "adj_L")


def test_blocked_solve_fp32_condition_1e3():
    # the fp32 tolerance holds up to condition number 1e3
    n, nrhs = 600, 4
    A = workloads.spd_condition(n, 1e3, seed=21)
    L, info = oracle.potrf(A)
    assert info == 0
    L = L.astype(np.float32)
    B = workloads.normal_rhs(n, nrhs, seed=22, dtype=np.float32)
    X = host(dc().chol_potrs(dev(L), dev(B)))
    assert_close(X, oracle.potrs(L, B), 2e-4, "X kappa 1e3")


def test_blocked_solve_larger_fp64():
    # several row tiles of 128 and a ragged tail on both sweeps, wide right-hand side
    n, nrhs = 2500, 40
    L = _factor(n, 77, np.float64)
    B = workloads.normal_rhs(n, nrhs, seed=78)
    X = host(dc().chol_potrs(dev(L), dev(B)))
    assert_close(X, oracle.potrs(L, B), 1e-10, "X")
    adjX = workloads.normal_rhs(n, nrhs, seed=79)
    aB, aL = dc().chol_potrs_adjoint(dev(L), dev(X), dev(adjX))
    aBo, aLo = oracle.potrs_adjoint(L, X, adjX)
    assert_close(host(aB), aBo, 1e-10, "adj_B")
    assert_close(np.tril(host(aL)), np.tril(aLo), 1e-10, "adj_L")


def test_solve_then_factor_adjoint_chain_matches_matrix_calculus():
    # end to end on the GPU: L = chol(A), x = potrs(L, b); the gradient of
    # <c, x> with respect to lower(A) through both adjoints equals the closed
    # form -(W + W^T) (diagonal -W_ii), W = (A^{-1} c)(A^{-1} b)^T
    n = 300
    A = workloads.gram_spd(n, seed=91)
    b = workloads.normal_rhs(n, 1, seed=92)
    c = workloads.normal_rhs(n, 1, seed=93)
    Ld, _ = dc().chol_potrf(dev(A))
    xd = dc().chol_potrs(Ld, dev(b))
    _, aL = dc().chol_potrs_adjoint(Ld, xd, dev(c), accumulate=False)
    G = host(dc().chol_potrf_adjoint(Ld, aL))
    W = np.linalg.solve(A, c) @ np.linalg.solve(A, b).T
    want = np.tril(-(W + W.T))
    want[np.diag_indices(n)] = -np.diag(W)
    assert_close(np.tril(G), want, 1e-9, "d<c, A^-1 b>/dA")
