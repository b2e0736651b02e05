"""Comparison helpers shared by the GPU parity tests."""
import numpy as np


def assert_close(got, ref, rtol, what=""):
    """|got - ref| <= rtol * (|ref| + max|ref|) elementwise, per matrix (last two axes).

    A relative bound alone is ill-posed for entries near zero; the max|ref| term
    makes it an allclose with atol = rtol * max|ref| of each matrix.
    """
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (got.shape, ref.shape)
    assert np.all(np.isfinite(got)), f"{what}: non-finite values"
    if ref.ndim == 2:
        got, ref = got[None], ref[None]
    scale = np.max(np.abs(ref), axis=(-2, -1), keepdims=True)
    bound = rtol * (np.abs(ref) + scale)
    err = np.abs(got - ref)
    bad = err > bound
    if np.any(bad):
        idx = np.argwhere(bad)[0]
        ratio = float(np.max(err / np.maximum(bound, 1e-300)))
        raise AssertionError(f"{what}: {int(bad.sum())} entries out of tolerance (rtol {rtol}); first at "
                             f"{tuple(idx)}: got {got[tuple(idx)]!r} ref {ref[tuple(idx)]!r}; worst err/bound {ratio:.3g}")


def residual(L, A):
    """||L L^T - A||_F / ||A||_F per matrix, A symmetrised from its lower triangle (fp64)."""
    L = np.asarray(L, dtype=np.float64)
    A = np.asarray(A, dtype=np.float64)
    As = np.tril(A) + np.swapaxes(np.tril(A, -1), -1, -2)
    R = np.matmul(L, np.swapaxes(L, -1, -2)) - As
    return np.linalg.norm(R, axis=(-2, -1)) / np.linalg.norm(As, axis=(-2, -1))
