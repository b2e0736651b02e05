"""GPU parity of the small-tile family (n <= 64) against the CPU oracle, through
the C-ABI.  Tolerances: fp64 1e-10, fp32 2e-4 (relative, with atol = rtol *
max|oracle| per matrix); residual ||L L^T - A|| / ||A|| <= 1e-13 (fp64) or 1e-5
(fp32)."""
import numpy as np
import pytest

import oracle
import workloads
from golden.fixtures import load
from parity_util import assert_close, residual

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

RTOL = {np.float64: 1e-10, np.float32: 2e-4}
RES = {np.float64: 1e-13, np.float32: 1e-5}
TDT = {np.float64: torch.float64, np.float32: torch.float32}


def dc():
    import differentiable_cholesky_amd
    return differentiable_cholesky_amd


def dev(x):
    return torch.from_numpy(np.ascontiguousarray(x)).cuda()


def host(t):
    torch.cuda.synchronize()
    return t.cpu().numpy()


# ----------------------------------------------- closed form, single matrix ----

def test_cfg_fp64_n16_closed_form_forward_and_adjoint():
    A, E = workloads.closed_form(16)
    adjL = workloads.lower_normal(16, seed=workloads.SEED_ADJ)
    L, info = dc().chol_potrf(dev(A))
    Lh = host(L)
    assert int(host(info)[0]) == 0
    assert np.max(np.abs(Lh - E)) <= 1e-14
    Lo, _ = oracle.potrf(A)
    assert_close(Lh, Lo, 1e-10, "L")
    assert residual(Lh, A) <= 1e-13
    G = host(dc().chol_potrf_adjoint(dev(Lh), dev(adjL)))
    Go = oracle.potrf_adjoint(Lo, adjL)
    assert_close(G, Go, 1e-10, "adj_A")


def test_n2_worked_example_on_gpu():
    g = load("n2_worked_example.txt")
    A = g["A"].reshape(2, 2)
    L, info = dc().chol_potrf(dev(A))
    Lh = host(L)
    assert np.array_equal(Lh, g["L"].reshape(2, 2))
    for key, pos in (("G_e00", (0, 0)), ("G_e10", (1, 0)), ("G_e11", (1, 1))):
        adjL = np.zeros((2, 2)); adjL[pos] = 1.0
        G = host(dc().chol_potrf_adjoint(dev(Lh), dev(adjL)))
        assert np.max(np.abs(np.array([G[0, 0], G[1, 0], G[1, 1]]) - g[key])) <= 1e-15


# ---------------------------------------------------------- batched fp32 ----

def test_cfg_batched_fp32_65536_n32():
    batch, n = 65536, 32
    A = workloads.batched_spd(batch, n, seed=workloads.SEED_MATRIX, dtype=np.float32)
    adjL = workloads.lower_normal(n, seed=workloads.SEED_ADJ, batch=batch, dtype=np.float32)
    base = np.tril(np.random.default_rng(7).standard_normal((batch, n, n)).astype(np.float32))
    Ad = dev(A)
    L, info = dc().chol_potrf_batched(Ad)
    adjA = dev(base)
    dc().chol_potrf_adjoint_batched(L, dev(adjL), adjA, accumulate=True)
    Lh, Gh, ih = host(L), host(adjA), host(info)
    assert np.all(ih == 0)
    Lo, io = oracle.potrf(A)
    assert np.all(io == 0)
    assert_close(Lh, Lo, 2e-4, "L")
    assert np.max(residual(Lh, A)) <= 1e-5
    Go = oracle.potrf_adjoint(Lh, adjL, base, accumulate=True)
    assert_close(Gh, Go, 2e-4, "adj_A")


@pytest.mark.parametrize("n,batch", [(8, 4096), (16, 4096), (32, 4096), (64, 1024)])
def test_batched_fp32_condition_1e3(n, batch):
    """fp32 tolerance clause: 2e-4 elementwise and residual 1e-5 on matrices of
    condition number 1e3 (A = Q diag(logspace(0, -3, n)) Q^T)."""
    A = workloads.spd_condition(n, 1e3, seed=500 + n, batch=batch, dtype=np.float32)
    adjL = workloads.lower_normal(n, seed=600 + n, batch=batch, dtype=np.float32)
    L, info = dc().chol_potrf_batched(dev(A))
    Lh = host(L)
    assert np.all(host(info) == 0)
    Lo, io = oracle.potrf(A)
    assert np.all(io == 0)
    assert_close(Lh, Lo, 2e-4, "L")
    assert np.max(residual(Lh, A)) <= 1e-5
    G = host(dc().chol_potrf_adjoint_batched(dev(Lh), dev(adjL), accumulate=False))
    Go = oracle.potrf_adjoint(Lh, adjL, accumulate=False)
    assert_close(G, Go, 2e-4, "adj_A")


# ------------------------------------------------------ ragged sizes, edges ----

SIZES = [1, 2, 3, 4, 5, 7, 8, 9, 13, 16, 17, 24, 31, 32, 33, 47, 63, 64]


@pytest.mark.parametrize("dtype", [np.float64, np.float32])
@pytest.mark.parametrize("n", SIZES)
def test_batched_ragged_forward_adjoint(n, dtype):
    batch = 37  # not a multiple of the matrices-per-block count
    A = workloads.batched_spd(batch, n, seed=100 + n, dtype=dtype)
    adjL = workloads.lower_normal(n, seed=200 + n, batch=batch, dtype=dtype)
    L, info = dc().chol_potrf_batched(dev(A))
    Lh = host(L)
    assert np.all(host(info) == 0)
    Lo, _ = oracle.potrf(A)
    assert_close(Lh, Lo, RTOL[dtype], "L")
    assert np.all(np.triu(Lh, 1) == 0)
    assert np.max(residual(Lh, A)) <= RES[dtype]
    G = host(dc().chol_potrf_adjoint_batched(dev(Lh), dev(adjL), accumulate=False))
    Go = oracle.potrf_adjoint(Lh, adjL, accumulate=False)
    assert_close(G, Go, RTOL[dtype], "adj_A")


@pytest.mark.parametrize("dtype", [np.float64, np.float32])
@pytest.mark.parametrize("n", [5, 32, 64])
def test_single_matrix_entry_points_small(n, dtype):
    A = workloads.gram_spd(n, seed=300 + n, dtype=dtype)
    adjL = workloads.lower_normal(n, seed=400 + n, dtype=dtype)
    L, info = dc().chol_potrf(dev(A))
    Lh = host(L)
    assert int(host(info)[0]) == 0
    Lo, _ = oracle.potrf(A)
    assert_close(Lh, Lo, RTOL[dtype], "L")
    base = np.random.default_rng(5).standard_normal((n, n)).astype(dtype)
    G = host(dc().chol_potrf_adjoint(dev(Lh), dev(adjL), dev(base), accumulate=True))
    Go = oracle.potrf_adjoint(Lh, adjL, base, accumulate=True)
    assert_close(np.tril(G), np.tril(Go), RTOL[dtype], "adj_A")
    assert np.array_equal(np.triu(G, 1), np.triu(base, 1))   # strict upper untouched


def test_strided_views_and_in_place():
    n, batch, ld = 20, 9, 27
    A = workloads.batched_spd(batch, n, seed=11, dtype=np.float64)
    big = np.full((batch, ld + 3, ld), 7.0)
    big[:, :n, :n] = A
    Ab = dev(big)
    view = Ab[:, :n, :n]                       # ld = 27, stride = 30 * 27
    out_of_place, _ = dc().chol_potrf_batched(view.contiguous())
    L_ip, info = dc().chol_potrf_batched(view, L=view)
    bigh = host(Ab)
    assert np.all(host(info) == 0)
    assert np.array_equal(bigh[:, :n, :n], host(out_of_place))
    assert np.all(bigh[:, :n, n:] == 7.0) and np.all(bigh[:, n:, :] == 7.0)   # outside untouched
    # adjoint in place over adj_L (accumulate = 0)
    Lh = bigh[:, :n, :n].copy()
    adjL = workloads.lower_normal(n, seed=12, batch=batch)
    ref = host(dc().chol_potrf_adjoint_batched(dev(Lh), dev(adjL), accumulate=False))
    buf = dev(adjL)
    dc().chol_potrf_adjoint_batched(dev(Lh), buf, buf, accumulate=False)
    assert np.array_equal(np.tril(host(buf)), np.tril(ref))


@pytest.mark.parametrize("n", [16, 32])
def test_fp32_row_alignment_paths_agree(n):
    """fp32 tiles of edge 16 or 32 whose rows start on 16-byte boundaries move
    through 16-byte accesses; other leading dimensions take 4-byte accesses.
    Both must give the same bits, write nothing outside the lower triangle
    (adjoint) or the n x n tile (factor), and work in place."""
    batch = 13
    A = workloads.batched_spd(batch, n, seed=21 + n, dtype=np.float32)
    adjL = workloads.lower_normal(n, seed=22 + n, batch=batch, dtype=np.float32)
    base = np.random.default_rng(23).standard_normal((batch, n, n)).astype(np.float32)
    results = {}
    for ld in (n, n + 4, n + 1):                      # aligned, aligned view, unaligned view
        big = np.full((batch, n + 2, ld), 5.0, dtype=np.float32)
        big[:, :n, :n] = A
        Ab = dev(big)
        view = Ab[:, :n, :n]
        _, info = dc().chol_potrf_batched(view, L=view)        # in place
        bigh = host(Ab)
        assert np.all(host(info) == 0)
        assert np.all(bigh[:, :n, n:] == 5.0) and np.all(bigh[:, n:, :] == 5.0)
        Lh = bigh[:, :n, :n].copy()
        gbig = np.full((batch, n + 2, ld), 5.0, dtype=np.float32)
        gbig[:, :n, :n] = base
        Gb = dev(gbig)
        gview = Gb[:, :n, :n]
        dc().chol_potrf_adjoint_batched(dev(Lh), dev(adjL), gview, accumulate=True)
        gh = host(Gb)
        assert np.array_equal(np.triu(gh[:, :n, :n], 1), np.triu(base, 1))    # strict upper untouched
        assert np.all(gh[:, :n, n:] == 5.0) and np.all(gh[:, n:, :] == 5.0)
        results[ld] = (Lh, gh[:, :n, :n].copy())
    Lo, _ = oracle.potrf(A)
    assert_close(results[n][0], Lo, 2e-4, "L")
    Go = oracle.potrf_adjoint(results[n][0], adjL, base, accumulate=True)
    assert_close(np.tril(results[n][1]), np.tril(Go), 2e-4, "adj_A")
    for ld in (n + 4, n + 1):
        assert np.array_equal(results[ld][0], results[n][0])
        assert np.array_equal(results[ld][1], results[n][1])
    # adjoint in place over adj_L (accumulate = 0) on the 16-byte path
    buf = dev(adjL)
    dc().chol_potrf_adjoint_batched(dev(results[n][0]), buf, buf, accumulate=False)
    ref = host(dc().chol_potrf_adjoint_batched(dev(results[n][0]), dev(adjL), accumulate=False))
    assert np.array_equal(np.tril(host(buf)), np.tril(ref))


@pytest.mark.parametrize("dtype", [np.float64, np.float32])
@pytest.mark.parametrize("n", [12, 32])
def test_info_per_batch_element(n, dtype):
    batch = 10
    A = workloads.batched_spd(batch, n, seed=13, dtype=np.float64)
    A[2, 0, 0] = -1.0
    A[5, 7, 7] = -50.0
    A[8, n - 1, n - 1] = np.nan
    A = A.astype(dtype)
    _, info = dc().chol_potrf_batched(dev(A))
    _, io = oracle.potrf(A)
    assert np.array_equal(host(info), io)
    assert list(np.nonzero(io)[0]) == [2, 5, 8]


def test_single_matrix_info_and_empty():
    A = workloads.spd_with_bad_pivot(9, 4, -1.0)
    _, info = dc().chol_potrf(dev(A))
    assert int(host(info)[0]) == 5
    e = torch.empty(0, 0, dtype=torch.float64, device="cuda")
    L, info = dc().chol_potrf(e)
    assert L.shape == (0, 0)


# ------------------------------------------- broadcast of a one-lane result ----

@pytest.mark.parametrize("dtype", [np.float32, np.float64])
@pytest.mark.parametrize("staging", [0, 1])
def test_wave_dot_one_lane_result(dtype, staging):
    g = load("tile_dot_warp1374.txt")
    a, b = dev(g["a"].astype(dtype)), dev(g["b"].astype(dtype))
    ybar = dev(np.array([1.0], dtype=dtype))
    y, abar, bbar = dc().chol_wave_dot_fwd_adj(a, b, ybar, staging=staging)
    assert float(host(y)[0]) == g["forward"][0]
    assert np.array_equal(host(abar).astype(np.float64), g["grad_a"])
    assert np.array_equal(host(bbar).astype(np.float64), g["grad_b"])
    # gradients accumulate into existing buffers
    y, abar2, _ = dc().chol_wave_dot_fwd_adj(a, b, dev(np.array([2.0], dtype=dtype)), abar=abar,
                                             staging=staging)
    assert np.array_equal(host(abar2).astype(np.float64), 3.0 * g["grad_a"])


@pytest.mark.parametrize("staging", [0, 1])
@pytest.mark.parametrize("dtype", [np.float32, np.float64])
def test_wave_sum_one_lane_result(dtype, staging):
    # the sum's result is written by one lane; its upstream gradient is read
    # by one lane and must reach every element's gradient
    a = np.arange(1.0, 17.0).astype(dtype)
    y, abar = dc().chol_wave_sum_fwd_adj(dev(a), dev(np.array([2.0], dtype=dtype)), staging=staging)
    assert float(host(y)[0]) == oracle.wsum(a) == 136.0
    assert np.array_equal(host(abar).astype(np.float64), oracle.wsum_adjoint(16, 2.0))
    y, abar = dc().chol_wave_sum_fwd_adj(dev(a), dev(np.array([1.0], dtype=dtype)), abar=abar, staging=staging)
    assert np.array_equal(host(abar).astype(np.float64), np.full(16, 3.0))
    rng = np.random.default_rng(7)
    v = rng.standard_normal(61).astype(dtype)
    y, _ = dc().chol_wave_sum_fwd_adj(dev(v), dev(np.array([1.0], dtype=dtype)), staging=staging)
    assert abs(float(host(y)[0]) - oracle.wsum(v)) <= (1e-12 if dtype == np.float64 else 1e-5) * np.sum(np.abs(v))
