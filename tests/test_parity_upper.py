"""GPU parity of the upper-factor form (A = U^T U from A's upper triangle) and
its adjoint against the oracle, through the C-ABI; tolerances as for the lower
form (fp64 1e-10, fp32 2e-4, relative with atol = rtol * max|oracle|)."""
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


def _poison_lower(A):
    B = A.copy()
    n = A.shape[-1]
    il = np.tril_indices(n, -1)
    if B.ndim == 2:
        B[il] = np.nan
    else:
        B[:, il[0], il[1]] = np.nan
    return B


@pytest.mark.parametrize("dt", [np.float64, np.float32])
@pytest.mark.parametrize("n", [1, 5, 16, 32, 33, 64])
def test_batched_upper_factor_and_adjoint(n, dt):
    batch = 29
    A = workloads.batched_spd(batch, n, seed=300 + n, dtype=dt)
    U, info = dc().chol_potrf_upper_batched(dev(_poison_lower(A)))   # the lower triangle is never read
    U = host(U)
    assert np.all(host(info) == 0)
    Uo, io = oracle.potrf_upper(A)
    assert np.all(io == 0)
    for b in range(batch):
        assert_close(U[b], Uo[b], RTOL[dt], f"U[{b}]")
    assert np.all(np.tril(U, -1) == 0)
    adjU = np.triu(workloads.normal_rhs(n, n, seed=301, batch=batch, dtype=dt))
    start = workloads.normal_rhs(n, n, seed=302, batch=batch, dtype=dt)
    for acc in (True, False):
        G = host(dc().chol_potrf_adjoint_upper_batched(dev(_poison_lower(Uo.astype(dt))),
                                                       dev(_poison_lower(adjU)), adjA=dev(start),
                                                       accumulate=acc))
        Go = oracle.potrf_adjoint_upper(Uo.astype(dt), adjU, adjA=start, accumulate=acc)
        for b in range(batch):
            assert_close(G[b], Go[b], RTOL[dt], f"adj_A[{b}] acc={acc}")
        assert np.array_equal(np.tril(G, -1), np.tril(start, -1))


@pytest.mark.parametrize("dt", [np.float64, np.float32])
@pytest.mark.parametrize("n,nb", [(10, 0), (65, 0), (130, 32), (300, 64), (777, 96), (1000, 0)])
def test_upper_factor_and_adjoint(n, nb, dt):
    A = workloads.gram_spd(n, seed=400 + n).astype(dt)
    U, info = dc().chol_potrf_upper(dev(_poison_lower(A)), nb=nb)
    U = host(U)
    assert int(host(info)[0]) == 0
    Uo, io = oracle.potrf_upper(A)
    assert io == 0
    assert_close(U, Uo, RTOL[dt], "U")
    assert np.all(np.tril(U, -1) == 0)
    adjU = np.triu(workloads.normal_rhs(n, n, seed=401, dtype=dt))
    start = workloads.normal_rhs(n, n, seed=402, dtype=dt)
    for acc in (True, False):
        G = host(dc().chol_potrf_adjoint_upper(dev(_poison_lower(Uo.astype(dt))), dev(_poison_lower(adjU)),
                                               adjA=dev(start), accumulate=acc, nb=nb))
        Go = oracle.potrf_adjoint_upper(Uo.astype(dt), adjU, adjA=start, accumulate=acc)
        assert_close(np.triu(G), np.triu(Go), RTOL[dt], f"adj_A acc={acc}")
        assert np.array_equal(np.tril(G, -1), np.tril(start, -1))


def test_upper_in_place_and_info():
    n = 300
    A = workloads.gram_spd(n, seed=5)
    Ad = dev(A)
    U, info = dc().chol_potrf_upper(Ad, U=Ad)
    assert U.data_ptr() == Ad.data_ptr() and int(host(info)[0]) == 0
    assert_close(host(Ad), oracle.potrf_upper(A)[0], 1e-10, "U in place")
    bad = A.copy()
    bad[200, 200] = -5.0
    _, info = dc().chol_potrf_upper(dev(bad))
    assert int(host(info)[0]) == oracle.potrf_upper(bad)[1] == 201
    # adjoint written over adj_U
    Uo = oracle.potrf_upper(A)[0]
    adjU = np.triu(workloads.normal_rhs(n, n, seed=6))
    g = dev(adjU)
    out = dc().chol_potrf_adjoint_upper(dev(Uo), g, adjA=g, accumulate=False)
    assert out.data_ptr() == g.data_ptr()
    assert_close(np.triu(host(g)), np.triu(oracle.potrf_adjoint_upper(Uo, adjU, accumulate=False)), 1e-10, "in place")
