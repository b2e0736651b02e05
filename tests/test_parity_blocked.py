"""GPU parity of the blocked family (n > 64) against the CPU oracle, through
the C-ABI, at sizes the oracle finishes in seconds (several tiles, ragged
tails), plus checks at the full benchmark sizes (8192, 16384) on outputs the
oracle can compute on its own (leading blocks, sampled rows) and on
identities that hold at any size."""
import numpy as np
import pytest

import oracle
import workloads
from parity_util import assert_close, residual

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

RTOL = {np.float64: 1e-10, np.float32: 2e-4}
RES = {np.float64: 1e-13, np.float32: 1e-5}


def dc():
    import differentiable_cholesky_amd
    return differentiable_cholesky_amd


def dev(x):
    return torch.from_numpy(np.ascontiguousarray(x)).cuda()


def host(t):
    torch.cuda.synchronize()
    return t.cpu().numpy()


def test_cfg_fp64_n512_closed_form_nb128():
    A, E = workloads.closed_form(512)
    L, info = dc().chol_potrf(dev(A), nb=128)
    Lh = host(L)
    assert int(host(info)[0]) == 0
    assert np.max(np.abs(Lh - E)) <= 1e-14
    Lo, _ = oracle.potrf(A)
    assert_close(Lh, Lo, 1e-10, "L")
    assert residual(Lh, A) <= 1e-13


CASES = [(65, 0), (100, 32), (127, 64), (128, 64), (129, 128), (200, 64), (255, 128), (256, 128),
         (257, 128), (300, 96), (513, 128), (1000, 0), (1000, 100)]


@pytest.mark.parametrize("n,nb", CASES)
def test_blocked_fp64_forward_adjoint(n, nb):
    A = workloads.gram_spd(n, seed=n, shift=1.0)
    adjL = workloads.lower_normal(n, seed=n + 1)
    L, info = dc().chol_potrf(dev(A), nb=nb)
    Lh = host(L)
    assert int(host(info)[0]) == 0
    Lo, _ = oracle.potrf(A)
    assert_close(Lh, Lo, 1e-10, "L")
    assert np.all(np.triu(Lh, 1) == 0)
    assert residual(Lh, A) <= 1e-13
    base = np.random.default_rng(n + 2).standard_normal((n, n))
    G = host(dc().chol_potrf_adjoint(dev(Lh), dev(adjL), dev(base), accumulate=True, nb=nb))
    Go = oracle.potrf_adjoint(Lh, adjL, base, accumulate=True)
    assert_close(np.tril(G), np.tril(Go), 1e-10, "adj_A")
    assert np.array_equal(np.triu(G, 1), np.triu(base, 1))


@pytest.mark.parametrize("n,nb", [(100, 0), (300, 64), (1000, 128)])
def test_blocked_fp32(n, nb):
    A = workloads.gram_spd(n, seed=n + 5, shift=1.0, dtype=np.float32)   # condition number ~ 5
    adjL = workloads.lower_normal(n, seed=n + 6, dtype=np.float32)
    L, info = dc().chol_potrf(dev(A), nb=nb)
    Lh = host(L)
    assert int(host(info)[0]) == 0
    Lo, _ = oracle.potrf(A)
    assert_close(Lh, Lo, 2e-4, "L")
    assert residual(Lh, A) <= 1e-5
    G = host(dc().chol_potrf_adjoint(dev(Lh), dev(adjL), accumulate=False, nb=nb))
    Go = oracle.potrf_adjoint(Lh, adjL, accumulate=False)
    assert_close(np.tril(G), np.tril(Go), 2e-4, "adj_A")


def test_blocked_in_place_matches_out_of_place_bitwise():
    n = 700
    A = workloads.gram_spd(n, seed=9)
    ref, _ = dc().chol_potrf(dev(A), nb=128)
    buf = dev(A)
    dc().chol_potrf(buf, L=buf, nb=128)
    assert np.array_equal(host(buf), host(ref))
    # adjoint: accumulate = 0 out of place, and in place over adj_L
    Lh = host(ref)
    adjL = workloads.lower_normal(n, seed=10)
    g0 = host(dc().chol_potrf_adjoint(dev(Lh), dev(adjL), accumulate=False, nb=128))
    b = dev(adjL)
    dc().chol_potrf_adjoint(dev(Lh), b, b, accumulate=False, nb=128)
    assert np.array_equal(np.tril(host(b)), np.tril(g0))


def test_blocked_repeatable_bitwise():
    # n = 6000: the far-triangle updates take several rounds of tiles from the
    # persistent grid and the symmetric products are split over the
    # contraction; tiles go to whichever block asks first, but every sum is
    # formed in a fixed order, so two runs agree to the bit
    n = 6000
    A = workloads.gram_spd(n, seed=21, shift=1.0, device="cuda")
    L1, i1 = dc().chol_potrf(A, nb=128)
    L2, i2 = dc().chol_potrf(A, nb=128)
    torch.cuda.synchronize()
    assert int(i1.item()) == 0 and int(i2.item()) == 0
    assert torch.equal(L1, L2)
    anorm = A.norm().item() / np.sqrt(n)
    for i in (0, n // 2, n - 1):
        r = (L1[i:i + 1, :] @ L1.T - A[i:i + 1, :]).norm().item() / anorm
        assert r <= 1e-13, (i, r)
    adjL = torch.from_numpy(workloads.lower_normal(n, seed=22)).cuda()
    G1 = dc().chol_potrf_adjoint(L1, adjL, accumulate=False, nb=128)
    G2 = dc().chol_potrf_adjoint(L1, adjL, accumulate=False, nb=128)
    torch.cuda.synchronize()
    assert torch.equal(torch.tril(G1), torch.tril(G2))
    # adj_L = L gives I / 2 at any size
    G = dc().chol_potrf_adjoint(L1, L1, accumulate=False, nb=128)
    assert (G.diagonal() - 0.5).abs().max().item() <= 0.5e-10
    assert torch.tril(G, -1).abs().max().item() <= 0.5e-10


def test_blocked_leading_dimension():
    n, ld = 300, 333
    A = workloads.gram_spd(n, seed=14)
    big = np.full((n, ld), 3.0)
    big[:, :n] = A
    Bd = dev(big)
    L, info = dc().chol_potrf(Bd[:, :n], nb=64)
    Lo, _ = oracle.potrf(A)
    assert_close(host(L), Lo, 1e-10, "L")
    assert np.all(host(Bd)[:, n:] == 3.0)


@pytest.mark.parametrize("n,col,nb", [(300, 0, 64), (300, 200, 64), (300, 299, 128), (1000, 517, 128)])
def test_blocked_info(n, col, nb):
    A = workloads.gram_spd(n, seed=15)
    A[col, col] = -1.0
    _, info = dc().chol_potrf(dev(A), nb=nb)
    _, io = oracle.potrf(A)
    assert io == col + 1
    assert int(host(info)[0]) == io


def test_blocked_info_resets_on_success():
    n = 200
    A = workloads.gram_spd(n, seed=16)
    info = torch.full((1,), 77, dtype=torch.int32, device="cuda")
    dc().chol_potrf(dev(A), info=info, nb=64)
    assert int(host(info)[0]) == 0


# --------------------------------------------------- full benchmark sizes ----

def _full_size_checks(n, shift, nb):
    """Factor and adjoint at full size, checked on what the oracle can compute
    independently: the leading m x m block (chol of A's leading block), sampled
    rows i (last row of chol of the principal submatrix on {0..m-1, i}), a
    sampled residual, and the adjoint identities adj_L = L => I/2 and
    adj_L = tril(2 W L) => Phi(2 W), plus the leading-block adjoint."""
    A = workloads.gram_spd(n, seed=workloads.SEED_MATRIX, shift=shift, device="cuda")
    L, info = dc().chol_potrf(A, nb=nb)
    torch.cuda.synchronize()
    assert int(info.item()) == 0
    m = 768
    Ah = A[:m, :m].cpu().numpy()
    Lo, io = oracle.potrf(Ah)
    assert io == 0
    assert_close(L[:m, :m].cpu().numpy(), Lo, 1e-10, "leading block")
    rng = np.random.default_rng(1)
    rows = np.sort(rng.choice(np.arange(m, n), size=6, replace=False))
    for i in rows:
        idx = np.r_[np.arange(m), i]
        Asub = A[idx][:, idx].cpu().numpy()
        Ls, _ = oracle.potrf(Asub)
        assert_close(L[i, :m].cpu().numpy()[None, :], Ls[m, :m][None, :], 1e-10, f"row {i}")
    # sampled residual rows: (L L^T)[i, :] vs A[i, :], scaled by the mean row norm of A
    anorm = A.norm().item() / np.sqrt(n)
    for i in list(rows) + [n - 1]:
        li = L[i:i + 1, :]
        r = (li @ L.T - A[i:i + 1, :]).norm().item() / anorm
        assert r <= 1e-13, (i, r)
    assert torch.all(torch.triu(L, 1) == 0).item()
    # adjoint identities at full size (tolerance 1e-10 relative to max|expected|)
    G = dc().chol_potrf_adjoint(L, L, accumulate=False, nb=nb)
    assert (G.diagonal() - 0.5).abs().max().item() <= 0.5e-10
    assert torch.tril(G, -1).abs().max().item() <= 0.5e-10
    p, q = n - 3, n // 3
    adjL = torch.zeros_like(L)
    adjL[p, :] = 2.0 * L[q, :]
    adjL[q, :q + 1] = 2.0 * L[p, :q + 1]
    G = dc().chol_potrf_adjoint(L, adjL, accumulate=False, nb=nb)
    assert abs(G[p, q].item() - 2.0) <= 2e-10
    G[p, q] = 0.0
    assert torch.tril(G).abs().max().item() <= 2e-10
    # adj_L supported on the leading block: G is the leading block's own adjoint
    adjL.zero_()
    small = workloads.lower_normal(m, seed=workloads.SEED_ADJ)
    adjL[:m, :m] = torch.from_numpy(small).cuda()
    G = dc().chol_potrf_adjoint(L, adjL, accumulate=False, nb=nb)
    Go = oracle.potrf_adjoint(L[:m, :m].cpu().numpy(), small, accumulate=False)
    assert_close(torch.tril(G[:m, :m]).cpu().numpy(), Go, 1e-10, "leading-block adjoint")
    assert torch.tril(G)[m:, :].abs().max().item() == 0.0


@pytest.mark.slow
def test_cfg_fp64_n8192_full_size():
    _full_size_checks(8192, 1.0, 128)


@pytest.mark.slow
def test_cfg_fp64_n16384_full_size():
    _full_size_checks(16384, 0.1, 128)
