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

def _say(*a):
    print(*a, flush=True)


def _gpu_residual(L, A):
    """||L L^T - A||_F / ||A||_F on the device (plain torch fp64 products)."""
    R = torch.tril(L) @ torch.tril(L).T
    R -= A
    return (R.norm() / A.norm()).item()


def _vjp_identity(L, adjL, G, seeds):
    """Defining property of the adjoint, at any size: for a lower-triangular
    direction E (symmetric perturbation E + strict(E)^T of A), the forward
    derivative of L is dL = L Phi(L^{-1} (E + strict(E)^T) L^{-T}), and
    <adj_L, dL> must equal sum_{i>=j} G_ij E_ij.  Computed with torch's fp64
    triangular solves and products on the device; returns the relative
    mismatches."""
    out = []
    n = L.shape[0]
    for s in seeds:
        g = torch.Generator(device="cpu").manual_seed(s)
        E = torch.tril(torch.randn(n, n, generator=g, dtype=torch.float64)).to(L.device)
        Es = E + torch.tril(E, -1).T
        Y = torch.linalg.solve_triangular(L, Es, upper=False)            # L^{-1} Es
        Z = torch.linalg.solve_triangular(L, Y.T.contiguous(), upper=False).T   # L^{-1} Es L^{-T}
        del Y, Es
        Z = torch.tril(Z)
        Z.diagonal().mul_(0.5)
        dL = L @ Z
        del Z
        lhs = (torch.tril(adjL) * dL).sum().item()
        rhs = (torch.tril(G) * E).sum().item()
        out.append(abs(lhs - rhs) / max(abs(lhs), 1e-300))
        del dL, E
    return out


@pytest.mark.slow
@pytest.mark.timeout(900)
def test_cfg_fp64_n8192_full_elementwise():
    """fp64 8192 x 8192, A = G G^T / 8192 + I (seed 0), adj_L = tril(N(0,1))
    (seed 1): the whole factor and the whole lower adjoint against the oracle,
    for the 128 tile and for a ragged 96 tile (8192 = 85 * 96 + 32).  The
    adjoint's input is the oracle's own factor, so that both tile sizes are
    compared with one oracle adjoint."""
    n = 8192
    A = workloads.gram_spd(n, seed=workloads.SEED_MATRIX, shift=1.0, device="cuda")
    Ah = A.cpu().numpy()
    _say(f"  n={n}: oracle factor")
    Lo, io = oracle.potrf(Ah)
    assert io == 0
    adjL_h = workloads.lower_normal(n, seed=workloads.SEED_ADJ)
    _say(f"  n={n}: oracle adjoint")
    Go = oracle.potrf_adjoint(Lo, adjL_h, accumulate=False)
    Lo_d = dev(Lo)
    adjL = dev(adjL_h)
    for nb in (128, 96):
        _say(f"  n={n} nb={nb}: GPU factor + adjoint")
        L, info = dc().chol_potrf(A, nb=nb)
        torch.cuda.synchronize()
        assert int(info.item()) == 0
        Lh = L.cpu().numpy()
        assert_close(Lh, Lo, 1e-10, f"L nb={nb}")
        assert np.all(np.triu(Lh, 1) == 0)
        assert _gpu_residual(L, A) <= 1e-13
        del L
        G = dc().chol_potrf_adjoint(Lo_d, adjL, torch.zeros_like(A), accumulate=True, nb=nb)
        Gh = np.tril(host(G))
        assert np.all(np.triu(host(G), 1) == 0)
        assert_close(Gh, np.tril(Go), 1e-10, f"adj_A nb={nb}")
        del G


@pytest.mark.slow
@pytest.mark.timeout(900)
def test_cfg_fp64_n16384_leading_block_and_identities():
    """fp64 16384 x 16384, A = G G^T / 16384 + 0.1 I (seed 0).  The oracle at
    this size takes too long, so the factor is compared with it on the leading
    8192 block (the leading block of L is the factor of A's leading block) and
    on sampled rows (row i of L restricted to columns < m is the last row of
    the factor of the principal submatrix on {0..m-1, i}); the residual is
    taken whole.  The adjoint is compared with the oracle for adj_L supported
    on the leading 8192 block (G is then that block's own adjoint and zero
    elsewhere), and for the benchmark's dense adj_L through the adjoint's
    defining identity and two exact identities (adj_L = L gives I/2;
    adj_L = tril(2 W L) gives Phi(2 W))."""
    n, m = 16384, 8192
    A = workloads.gram_spd(n, seed=workloads.SEED_MATRIX, shift=0.1, device="cuda")
    _say(f"  n={n}: GPU factor")
    L, info = dc().chol_potrf(A, nb=128)
    torch.cuda.synchronize()
    assert int(info.item()) == 0
    assert torch.all(torch.triu(L, 1) == 0).item()
    assert _gpu_residual(L, A) <= 1e-13
    _say(f"  n={n}: oracle factor of the leading {m} block")
    Lo, io = oracle.potrf(A[:m, :m].cpu().numpy())
    assert io == 0
    assert_close(L[:m, :m].cpu().numpy(), Lo, 1e-10, "leading block")
    del Lo
    ms = 768
    rows = np.sort(np.random.default_rng(1).choice(np.arange(ms, n), size=6, replace=False))
    for i in rows:
        idx = np.r_[np.arange(ms), i]
        Ls, _ = oracle.potrf(A[idx][:, idx].cpu().numpy())
        assert_close(L[i, :ms].cpu().numpy()[None, :], Ls[ms, :ms][None, :], 1e-10, f"row {i}")
    # adj_L on the leading block
    _say(f"  n={n}: adjoint, adj_L on the leading {m} block")
    small = workloads.lower_normal(m, seed=workloads.SEED_ADJ)
    adjL = torch.zeros_like(L)
    adjL[:m, :m] = dev(small)
    G = dc().chol_potrf_adjoint(L, adjL, accumulate=False, nb=128)
    torch.cuda.synchronize()
    Gh = torch.tril(G[:m, :m]).cpu().numpy()
    assert torch.tril(G)[m:, :].abs().max().item() == 0.0
    del G
    _say(f"  n={n}: oracle adjoint of the leading block")
    Go = oracle.potrf_adjoint(L[:m, :m].cpu().numpy(), small, accumulate=False)
    assert_close(Gh, Go, 1e-10, "leading-block adjoint")
    del Gh, Go
    # the benchmark's dense adj_L: the defining identity of the adjoint
    _say(f"  n={n}: dense adj_L, adjoint identity")
    adjL = dev(workloads.lower_normal(n, seed=workloads.SEED_ADJ))
    G = dc().chol_potrf_adjoint(L, adjL, torch.zeros_like(L), accumulate=True, nb=128)
    torch.cuda.synchronize()
    assert torch.all(torch.isfinite(G)).item()
    mism = _vjp_identity(L, adjL, G, seeds=(11, 12))
    assert max(mism) <= 1e-10, mism
    del G, adjL
    # exact identities
    G = dc().chol_potrf_adjoint(L, L, accumulate=False, nb=128)
    assert (G.diagonal() - 0.5).abs().max().item() <= 0.5e-10
    assert torch.tril(G, -1).abs().max().item() <= 0.5e-10
    p, q = n - 3, n // 3
    adjL = torch.zeros_like(L)
    adjL[p, :] = 2.0 * L[q, :]
    adjL[q, :q + 1] = 2.0 * L[p, :q + 1]
    G = dc().chol_potrf_adjoint(L, adjL, accumulate=False, nb=128)
    assert abs(G[p, q].item() - 2.0) <= 2e-10
    G[p, q] = 0.0
    assert torch.tril(G).abs().max().item() <= 2e-10


@pytest.mark.slow
@pytest.mark.timeout(600)
def test_multi_launch_far_triangle_elementwise():
    """n = 5000, nb = 128: the far triangle of a group is cut into several
    persistent launches (checked on the executor's own plan); the whole factor
    and the whole adjoint (dense adj_L) are compared with the oracle."""
    n = 5000
    plan = dc().chol_potrf_plan(n, 128, copy=True, slots=2 * (torch.cuda.get_device_properties(0).multi_processor_count - 16))
    tri = plan[plan[:, 0] == 4]
    per_group = {}
    for r in tri:
        per_group[(int(r[3]), int(r[5]))] = per_group.get((int(r[3]), int(r[5])), 0) + 1
    assert max(per_group.values()) >= 2, per_group
    A = workloads.gram_spd(n, seed=n, shift=1.0)
    L, info = dc().chol_potrf(dev(A), nb=128)
    Lh = host(L)
    assert int(host(info)[0]) == 0
    Lo, _ = oracle.potrf(A)
    assert_close(Lh, Lo, 1e-10, "L")
    assert residual(Lh, A) <= 1e-13
    adjL = workloads.lower_normal(n, seed=n + 1)
    G = host(dc().chol_potrf_adjoint(dev(Lo), dev(adjL), accumulate=False, nb=128))
    Go = oracle.potrf_adjoint(Lo, adjL, accumulate=False)
    assert_close(np.tril(G), np.tril(Go), 1e-10, "adj_A")


# ------------------------------------------- fp32 at condition number 1e3 ----

@pytest.mark.parametrize("n,nb", [(300, 64), (1000, 128)])
def test_blocked_fp32_condition_1e3(n, nb):
    A = workloads.spd_condition(n, 1e3, seed=n + 7, dtype=np.float32)
    adjL = workloads.lower_normal(n, seed=n + 8, dtype=np.float32)
    L, info = dc().chol_potrf(dev(A), nb=nb)
    Lh = host(L)
    assert int(host(info)[0]) == 0
    Lo, _ = oracle.potrf(A)
    assert_close(Lh, Lo, 2e-4, "L")
    assert residual(Lh, A) <= 1e-5
    G = host(dc().chol_potrf_adjoint(dev(Lh), dev(adjL), accumulate=False, nb=nb))
    Go = oracle.potrf_adjoint(Lh, adjL, accumulate=False)
    assert_close(np.tril(G), np.tril(Go), 2e-4, "adj_A")
