"""The allocation-free adjoint entry point, chol_potrf_adjoint_noalloc, called
through the C-ABI and checked against the workspace entry point
chol_potrf_adjoint (and the oracle) on two calls in a row, the second with a
smaller input; device memory must not change across the calls."""
import ctypes

import numpy as np
import pytest

import oracle
import workloads
from parity_util import assert_close

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


def _noalloc(lib, L, adjL, adjA, accumulate, nb):
    code = 1 if L.dtype == torch.float64 else 0
    st = lib.chol_potrf_adjoint_noalloc(code, L.shape[0], ctypes.c_void_p(L.data_ptr()), L.stride(0),
                                        ctypes.c_void_p(adjL.data_ptr()), adjL.stride(0),
                                        ctypes.c_void_p(adjA.data_ptr()), adjA.stride(0), 1 if accumulate else 0,
                                        nb, ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert st == 0, st


@pytest.mark.parametrize("dtype", [np.float64, np.float32])
def test_noalloc_adjoint_matches_workspace_entry_point(dtype):
    import differentiable_cholesky_amd as dc
    lib = dc.lib
    rtol = 1e-10 if dtype == np.float64 else 2e-4
    tdt = torch.float64 if dtype == np.float64 else torch.float32
    dc.chol_init()
    # two calls in a row, the second smaller; the first fills the whole
    # scratch layout of n = 1024 (accumulate: with the n x n gradient copy)
    cases = [(1024, 128, True, 40), (300, 64, False, 41)]
    prepared = []
    for n, nb, acc, seed in cases:
        A = workloads.gram_spd(n, seed=seed, shift=1.0)
        Lo, info = oracle.potrf(A)
        assert info == 0
        L = torch.from_numpy(Lo.astype(dtype)).cuda()
        adjL = torch.from_numpy(workloads.lower_normal(n, seed=seed + 1, dtype=dtype)).cuda()
        base = torch.from_numpy(np.random.default_rng(seed + 2).standard_normal((n, n)).astype(dtype)).cuda()
        ref = dc.chol_potrf_adjoint(L, adjL, base.clone(), accumulate=acc, nb=nb)   # workspace entry point
        out = base.clone()
        prepared.append((n, nb, acc, L, adjL, base, ref, out))
    torch.cuda.synchronize()
    free0 = torch.cuda.mem_get_info()[0]
    for n, nb, acc, L, adjL, base, ref, out in prepared:
        _noalloc(lib, L, adjL, out, acc, nb)
    torch.cuda.synchronize()
    assert torch.cuda.mem_get_info()[0] == free0
    for n, nb, acc, L, adjL, base, ref, out in prepared:
        got, want = out.cpu().numpy(), ref.cpu().numpy()
        assert_close(np.tril(got), np.tril(want), rtol, f"n={n} against chol_potrf_adjoint")
        assert np.array_equal(np.triu(got, 1), np.triu(base.cpu().numpy(), 1))
        Go = oracle.potrf_adjoint(L.cpu().numpy(), adjL.cpu().numpy(), base.cpu().numpy(), accumulate=acc)
        assert_close(np.tril(got), np.tril(Go), rtol, f"n={n} against the oracle")


def test_noalloc_in_place_and_size_limit():
    import differentiable_cholesky_amd as dc
    n = 500
    A = workloads.gram_spd(n, seed=50)
    Lo, _ = oracle.potrf(A)
    L = torch.from_numpy(Lo).cuda()
    adjL_h = workloads.lower_normal(n, seed=51)
    buf = torch.from_numpy(adjL_h).cuda()
    _noalloc(dc.lib, L, buf, buf, False, 0)          # adj_A == adj_L, accumulate = 0
    Go = oracle.potrf_adjoint(Lo, adjL_h, accumulate=False)
    assert_close(np.tril(buf.cpu().numpy()), np.tril(Go), 1e-10, "in place")
    big = torch.zeros(1025, 1025, dtype=torch.float64, device="cuda")
    st = dc.lib.chol_potrf_adjoint_noalloc(1, 1025, ctypes.c_void_p(big.data_ptr()), 1025,
                                           ctypes.c_void_p(big.data_ptr() + 8), 1025,
                                           ctypes.c_void_p(big.data_ptr() + 16), 1025, 0, 0, None)
    from differentiable_cholesky_amd import _lib
    assert st == _lib.CHOL_ERR_NOT_SUPPORTED
