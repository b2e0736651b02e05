"""Seeded synthetic inputs shared by the tests, the smoke check and the benchmark.

This module builds inputs only; it holds none of the factorisation's or the
adjoint's arithmetic, and imports neither the GPU library nor the oracle.  All
matrices are assembled on the host in fp64 (or, for the largest sizes, their
Gram product is formed on a torch device), mirrored from the lower triangle
so that A is exactly symmetric, and only then cast to the working dtype.  The
same bits therefore reach the oracle and the GPU.

Workloads (each is a stand-in built from the recipe the pages or the
benchmark configuration give; no dataset is involved):

* ``closed_form``   -- A = E E^T with E = diag(linspace(1, 2, n)) plus 0.5 on
                       the first subdiagonal (jaxmg docs, "Cholesky
                       factorization", "Common setup" generator); its factor is E.
* ``gram_spd``      -- A = G G^T / n + shift * I, G iid N(0, 1) from a seed.
* ``batched_spd``   -- A_b = B_b B_b^T / n + I, B iid N(0, 1) from a seed.
* ``lower_normal``  -- a lower-triangular N(0, 1) upstream gradient adj_L.
* ``normal_rhs``    -- iid N(0, 1) right-hand sides (and their upstream
                       gradients) for the solve with the factor.
* ``spd_condition`` -- A = Q diag(logspace(0, -log10(kappa), n)) Q^T with Q the
                       orthogonal factor of an iid N(0, 1) matrix: condition
                       number exactly kappa (the fp32 tolerance applies to
                       condition numbers up to 1e3).

Random numbers come from ``numpy.random.default_rng(seed)`` (PCG64)
``standard_normal`` in fp64.
"""
from __future__ import annotations

import numpy as np

SEED_MATRIX = 0
SEED_ADJ = 1


def symmetrize_from_lower(A: np.ndarray) -> np.ndarray:
    """Copy the strict lower triangle onto the upper one (last two axes)."""
    low = np.tril(A)
    strict = np.tril(A, -1)
    return low + np.swapaxes(strict, -1, -2)


def closed_form(n: int, dtype=np.float64):
    """Return (A, E): the tridiagonal SPD matrix A = E E^T and its factor E.

    E has diag(linspace(1, 2, n)) and 0.5 on the first subdiagonal.  A is
    written entry by entry from the two nonzero products per entry so that any
    n (up to the largest benchmark size) is cheap to build.
    """
    d = np.linspace(1.0, 2.0, n, dtype=np.float64)
    E = np.zeros((n, n), dtype=np.float64)
    idx = np.arange(n)
    E[idx, idx] = d
    if n > 1:
        E[idx[1:], idx[:-1]] = 0.5
    A = np.zeros((n, n), dtype=np.float64)
    diag = d * d
    diag[1:] += 0.25
    A[idx, idx] = diag
    if n > 1:
        off = 0.5 * d[:-1]
        A[idx[1:], idx[:-1]] = off
        A[idx[:-1], idx[1:]] = off
    return A.astype(dtype), E.astype(dtype)


def gram_spd(n: int, seed: int = SEED_MATRIX, shift: float = 1.0, dtype=np.float64,
             device=None):
    """A = G G^T / n + shift * I with G iid N(0, 1) (PCG64 ``seed``).

    With ``device`` (a torch device string) the Gram product is formed there
    in fp64 and a torch tensor of ``dtype`` on that device is returned; the
    random G is still drawn on the host so the input does not depend on the
    device.  Without it a NumPy array is returned.
    """
    rng = np.random.default_rng(seed)
    G = rng.standard_normal((n, n))
    if device is None:
        A = G @ G.T
        A /= n
        A[np.arange(n), np.arange(n)] += shift
        return symmetrize_from_lower(A).astype(dtype)
    import torch

    Gt = torch.from_numpy(G).to(device)
    del G
    A = Gt @ Gt.T
    del Gt
    A /= n
    A.diagonal().add_(shift)
    low = torch.tril(A)
    A = low + torch.tril(A, -1).T
    tdt = {np.float64: torch.float64, np.float32: torch.float32}[np.dtype(dtype).type]
    return A.to(tdt).contiguous()


def batched_spd(batch: int, n: int, seed: int = SEED_MATRIX, dtype=np.float32):
    """A_b = B_b B_b^T / n + I, B iid N(0, 1); shape [batch, n, n]."""
    rng = np.random.default_rng(seed)
    B = rng.standard_normal((batch, n, n))
    A = np.matmul(B, np.swapaxes(B, -1, -2))
    A /= n
    A[:, np.arange(n), np.arange(n)] += 1.0
    return symmetrize_from_lower(A).astype(dtype)


def lower_normal(n: int, seed: int = SEED_ADJ, batch: int | None = None, dtype=np.float64):
    """tril(N(0, 1)) of shape [n, n] or [batch, n, n]."""
    rng = np.random.default_rng(seed)
    shape = (n, n) if batch is None else (batch, n, n)
    return np.tril(rng.standard_normal(shape)).astype(dtype)


def normal_rhs(n: int, nrhs: int, seed: int = SEED_ADJ, batch: int | None = None, dtype=np.float64):
    """N(0, 1) of shape [n, nrhs] or [batch, n, nrhs]."""
    rng = np.random.default_rng(seed)
    shape = (n, nrhs) if batch is None else (batch, n, nrhs)
    return rng.standard_normal(shape).astype(dtype)


def spd_condition(n: int, kappa: float, seed: int = SEED_MATRIX, batch: int | None = None,
                  dtype=np.float64):
    """A = Q diag(logspace(0, -log10(kappa), n)) Q^T, Q orthogonal from the QR
    factorisation of an iid N(0, 1) matrix; shape [n, n] or [batch, n, n].
    Built in fp64, mirrored from the lower triangle, then cast."""
    rng = np.random.default_rng(seed)
    shape = (n, n) if batch is None else (batch, n, n)
    Q, _ = np.linalg.qr(rng.standard_normal(shape))
    d = np.logspace(0.0, -np.log10(kappa), n)
    A = np.matmul(Q * d, np.swapaxes(Q, -1, -2))
    return symmetrize_from_lower(A).astype(dtype)


def spd_with_bad_pivot(n: int, col: int, value: float = -1.0, dtype=np.float64):
    """Identity with A[col, col] = value: the first failing pivot is at ``col``
    when ``value`` is not > 0 (NaN included)."""
    A = np.eye(n, dtype=np.float64)
    A[col, col] = value
    return A.astype(dtype)
