"""Comparison helpers shared by the GPU parity tests."""
import numpy as np

# Entries whose oracle value is within this fraction of the matrix's largest
# entry are also held to a purely relative bound |got - ref| <= rtol |ref|.
# fp64: three decades (two correct fp64 implementations differ by ~1e-12
# relative there at n = 4096).  fp32: one decade, because at condition number
# 1e3 the forward error of any fp32 algorithm is about kappa * u relative to
# the largest entry, so smaller entries carry proportionally larger relative
# errors while staying inside the allclose bound.
REL_FRAC = {np.float64: 1e-3, np.float32: 1e-1}


def close_stats(got, ref, rel_frac=1e-3):
    """(allclose ratio, max relative error over |ref| >= rel_frac * max|ref|) per
    matrix stack: the first is max |got - ref| / (|ref| + max|ref|)."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    if ref.ndim == 2:
        got, ref = got[None], ref[None]
    scale = np.max(np.abs(ref), axis=(-2, -1), keepdims=True)
    err = np.abs(got - ref)
    ac = float(np.max(err / np.maximum(np.abs(ref) + scale, 1e-300)))
    big = np.abs(ref) >= rel_frac * scale
    big &= scale > 0
    rel = float(np.max(np.where(big, err / np.maximum(np.abs(ref), 1e-300), 0.0)))
    return ac, rel


def assert_close(got, ref, rtol, what="", rel_frac=None):
    """Elementwise parity, per matrix (last two axes):

    * |got - ref| <= rtol * (|ref| + max|ref|) everywhere: an allclose with
      atol = rtol * max|ref| of each matrix (a relative bound alone is
      ill-posed for entries near zero);
    * |got - ref| <= rtol * |ref| on the entries with |ref| >= rel_frac *
      max|ref| (default by precision: REL_FRAC), so the bound is a relative
      one wherever the entry is not small next to the matrix's largest.
    """
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (got.shape, ref.shape)
    assert np.all(np.isfinite(got)), f"{what}: non-finite values"
    if rel_frac is None:
        rel_frac = REL_FRAC[np.float64] if rtol < 1e-6 else REL_FRAC[np.float32]
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
    big = (np.abs(ref) >= rel_frac * scale) & (scale > 0)
    rbad = big & (err > rtol * np.abs(ref))
    if np.any(rbad):
        idx = np.argwhere(rbad)[0]
        worst = float(np.max(np.where(big, err / np.maximum(np.abs(ref), 1e-300), 0.0)))
        raise AssertionError(f"{what}: {int(rbad.sum())} entries above {rel_frac} * max|ref| exceed relative "
                             f"{rtol}; first at {tuple(idx)}: got {got[tuple(idx)]!r} ref {ref[tuple(idx)]!r}; "
                             f"worst relative error {worst:.3g}")


def residual(L, A):
    """||L L^T - A||_F / ||A||_F per matrix, A symmetrised from its lower triangle (fp64)."""
    L = np.asarray(L, dtype=np.float64)
    A = np.asarray(A, dtype=np.float64)
    As = np.tril(A) + np.swapaxes(np.tril(A, -1), -1, -2)
    R = np.matmul(L, np.swapaxes(L, -1, -2)) - As
    return np.linalg.norm(R, axis=(-2, -1)) / np.linalg.norm(As, axis=(-2, -1))
