"""Plain CPU oracle for the Cholesky factor and its adjoint (fp64).

TEST INFRASTRUCTURE ONLY.  The test suite, the smoke check and the
benchmark's CPU-baseline leg are the only callers.  Nothing here is imported
by, or imports, the GPU library; the two share no code.  The seeded input
generators live in their own module (``workloads``) and hold none of the
method's arithmetic.

What each function computes, and the pages it follows, is stated in
``oracle.c``:

* ``potrf``            -- the factor A = L L^T, column by column
                          (jaxmg docs, "Cholesky factorization").
* ``potrf_adjoint``    -- Murray's symmetric-matrix derivative: Phi(L^T adj_L),
                          two triangular solves against L, Phi(S + S^T) into
                          the lower triangle of adj_A (Warp issue #1316,
                          resolution comment).
* ``potrf_adjoint_sweep`` -- an independent reverse sweep of the column-form
                          factorisation, used only to cross-check the formula.
* ``dot`` / ``dot_adjoint`` -- y = a.b and a_bar += y_bar b, b_bar += y_bar a
                          (Warp issue #1374, description and repro).
* ``potrf_upper`` / ``potrf_adjoint_upper`` -- the upper-factor form A = U^T U
                          (U = L^T of the same matrix, upper triangle of A
                          read) and its adjoint (G^T into the upper triangle).
* ``zpotrf`` / ``zpotrf_adjoint`` -- the Hermitian complex factor A = L L^H
                          and its adjoint (the same formula with conjugate
                          transposes; the diagonal's real part in Phi).
* ``potrs``            -- X = (L L^T)^{-1} B by forward and back substitution
                          against L (the solve the factor is returned for,
                          jaxmg docs, "Cholesky factorization"; the two
                          triangular solves of Warp issue #1316).
* ``potrs_adjoint``    -- adj_B = (L L^T)^{-1} adj_X and
                          adj_L = -tril((adj_B X^T + X adj_B^T) L).

Every array argument is a NumPy array; inputs of any float dtype are promoted
to fp64 exactly (float32 -> float64 is exact).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

_lib = None


def build(force: bool = True) -> str:
    """Compile ``oracle.c`` with gcc (fp64, no FMA contraction, OpenMP)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp"
        cmd = ["gcc", "-O2", "-std=c11", "-fopenmp", "-ffp-contract=off", "-fno-fast-math",
               "-fPIC", "-shared", _SRC, "-o", tmp, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    if _lib is None:
        if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
            build(force=True)
        _load_path(_LIB)
    return _lib


def _load_path(path: str):
    global _lib
    lib = ctypes.CDLL(path)
    i64, i32, dp, ip = ctypes.c_int64, ctypes.c_int32, ctypes.c_void_p, ctypes.c_void_p
    lib.oracle_potrf.restype = i32
    lib.oracle_potrf.argtypes = [i64, dp, i64, dp, i64]
    for name in ("oracle_potrf_adjoint", "oracle_potrf_adjoint_sweep"):
        f = getattr(lib, name)
        f.restype = i32
        f.argtypes = [i64, dp, i64, dp, i64, dp, i64, i32]
    lib.oracle_potrf_batched.restype = None
    lib.oracle_potrf_batched.argtypes = [i64, i64, dp, i64, i64, dp, i64, i64, ip]
    lib.oracle_potrf_adjoint_batched.restype = i32
    lib.oracle_potrf_adjoint_batched.argtypes = [i64, i64, dp, i64, i64, dp, i64, i64,
                                                 dp, i64, i64, i32]
    lib.oracle_potrf_upper.restype = i32
    lib.oracle_potrf_upper.argtypes = [i64, dp, i64, dp, i64]
    lib.oracle_potrf_adjoint_upper.restype = i32
    lib.oracle_potrf_adjoint_upper.argtypes = [i64, dp, i64, dp, i64, dp, i64, i32]
    lib.oracle_potrs.restype = None
    lib.oracle_potrs.argtypes = [i64, i64, dp, i64, dp, i64, dp, i64]
    lib.oracle_potrs_adjoint.restype = i32
    lib.oracle_potrs_adjoint.argtypes = [i64, i64, dp, i64, dp, i64, dp, i64, dp, i64, dp, i64, i32]
    lib.oracle_dot.restype = ctypes.c_double
    lib.oracle_dot.argtypes = [i64, dp, dp]
    lib.oracle_dot_adjoint.restype = None
    lib.oracle_dot_adjoint.argtypes = [i64, dp, dp, ctypes.c_double, dp, dp]
    lib.oracle_zpotrf.restype = i32
    lib.oracle_zpotrf.argtypes = [i64, dp, i64, dp, i64]
    lib.oracle_zpotrf_adjoint.restype = i32
    lib.oracle_zpotrf_adjoint.argtypes = [i64, dp, i64, dp, i64, dp, i64, i32]
    lib.oracle_sum.restype = ctypes.c_double
    lib.oracle_sum.argtypes = [i64, dp]
    lib.oracle_sum_adjoint.restype = None
    lib.oracle_sum_adjoint.argtypes = [i64, ctypes.c_double, dp]
    lib.oracle_max_threads.restype = i32
    lib.oracle_max_threads.argtypes = []
    _lib = lib
    return _lib


class _use_library:
    """Temporarily point this module at another build of the oracle (used only
    by the mutation test, which compiles copies of ``oracle.c`` with a planted
    mistake to show that the pins catch it)."""

    def __init__(self, path: str):
        self.path = path

    def __enter__(self):
        global _lib
        self.saved = _load()
        _lib = None
        _load_path(self.path)
        return self

    def __exit__(self, *exc):
        global _lib
        _lib = self.saved
        return False


def _f64(x) -> np.ndarray:
    return np.ascontiguousarray(np.asarray(x, dtype=np.float64))


def _ptr(a: np.ndarray):
    return ctypes.c_void_p(a.ctypes.data)


def max_threads() -> int:
    """OpenMP threads the oracle's parallel loops may use."""
    return int(_load().oracle_max_threads())


def potrf(A):
    """Return ``(L, info)`` for one square matrix (or ``(L[b], info[b])`` for a
    stacked ``[batch, n, n]`` array).  Only the lower triangle of A is read; L's
    strict upper triangle is zero."""
    A = _f64(A)
    lib = _load()
    if A.ndim == 2:
        n = A.shape[0]
        assert A.shape == (n, n)
        L = np.zeros_like(A)
        info = int(lib.oracle_potrf(n, _ptr(A), n, _ptr(L), n))
        return L, info
    assert A.ndim == 3 and A.shape[1] == A.shape[2]
    batch, n = A.shape[0], A.shape[1]
    L = np.zeros_like(A)
    info = np.zeros(batch, dtype=np.int32)
    lib.oracle_potrf_batched(n, batch, _ptr(A), n, n * n, _ptr(L), n, n * n, _ptr(info))
    return L, info


def potrf_adjoint(L, adjL, adjA=None, accumulate: bool = True, method: str = "formula"):
    """Adjoint of the factorisation.  Returns adj_A with its lower triangle
    incremented by (``accumulate``) or set to (otherwise) G = Phi(S + S^T);
    the strict upper triangle of adj_A is returned unchanged (zero if adj_A
    was not given).  ``method`` is "formula" (the pages' two-solve form) or
    "sweep" (the independent cross-check)."""
    L = _f64(L)
    adjL = _f64(adjL)
    out = np.zeros_like(L) if adjA is None else _f64(adjA).copy()
    lib = _load()
    if L.ndim == 2:
        n = L.shape[0]
        fn = lib.oracle_potrf_adjoint if method == "formula" else lib.oracle_potrf_adjoint_sweep
        rc = fn(n, _ptr(L), n, _ptr(adjL), n, _ptr(out), n, 1 if accumulate else 0)
    else:
        assert method == "formula"
        batch, n = L.shape[0], L.shape[1]
        rc = lib.oracle_potrf_adjoint_batched(n, batch, _ptr(L), n, n * n, _ptr(adjL), n, n * n,
                                              _ptr(out), n, n * n, 1 if accumulate else 0)
    if rc != 0:
        raise MemoryError("oracle adjoint could not allocate its scratch matrices")
    return out


def dot(a, b) -> float:
    a, b = _f64(a), _f64(b)
    assert a.shape == b.shape and a.ndim == 1
    return float(_load().oracle_dot(a.size, _ptr(a), _ptr(b)))


def dot_adjoint(a, b, ybar: float):
    """Return (a_bar, b_bar) for y = a.b given y_bar, starting from zero."""
    a, b = _f64(a), _f64(b)
    abar = np.zeros_like(a)
    bbar = np.zeros_like(b)
    _load().oracle_dot_adjoint(a.size, _ptr(a), _ptr(b), float(ybar), _ptr(abar), _ptr(bbar))
    return abar, bbar


def _rhs(B, n):
    B = _f64(B)
    vec = B.ndim == 1
    B2 = B.reshape(n, 1) if vec else B
    assert B2.shape[0] == n
    return np.ascontiguousarray(B2), vec


def potrs(L, B):
    """X = (L L^T)^{-1} B for one lower factor L (n x n) and B (n or n x nrhs),
    or for stacked ``[batch, n, n]`` / ``[batch, n, nrhs]`` arrays.  Only the
    lower triangle of L is read."""
    L = _f64(L)
    lib = _load()
    if L.ndim == 3:
        B = _f64(B)
        return np.stack([potrs(L[b], B[b]) for b in range(L.shape[0])])
    n = L.shape[0]
    B2, vec = _rhs(B, n)
    X = np.zeros_like(B2)
    nrhs = B2.shape[1]
    lib.oracle_potrs(n, nrhs, _ptr(L), n, _ptr(B2), nrhs, _ptr(X), nrhs)
    return X.reshape(-1) if vec else X


def potrs_adjoint(L, X, adjX, adjL=None, accumulate: bool = True):
    """Adjoint of X = potrs(L, B): returns ``(adj_B, adj_L)`` with adj_B =
    (L L^T)^{-1} adj_X and the lower triangle of adj_L incremented by
    (``accumulate``) or set to (otherwise) -tril((adj_B X^T + X adj_B^T) L);
    adj_L's strict upper triangle is returned unchanged (zero if not given).
    Stacked ``[batch, ...]`` arrays are handled element by element."""
    L = _f64(L)
    lib = _load()
    if L.ndim == 3:
        X, adjX = _f64(X), _f64(adjX)
        outs = [potrs_adjoint(L[b], X[b], adjX[b], None if adjL is None else _f64(adjL)[b], accumulate)
                for b in range(L.shape[0])]
        return np.stack([o[0] for o in outs]), np.stack([o[1] for o in outs])
    n = L.shape[0]
    X2, vec = _rhs(X, n)
    aX2, _ = _rhs(adjX, n)
    nrhs = X2.shape[1]
    assert aX2.shape == X2.shape
    adjB = np.zeros_like(X2)
    out = np.zeros_like(L) if adjL is None else _f64(adjL).copy()
    rc = lib.oracle_potrs_adjoint(n, nrhs, _ptr(L), n, _ptr(X2), nrhs, _ptr(aX2), nrhs, _ptr(adjB), nrhs,
                                  _ptr(out), n, 1 if accumulate else 0)
    if rc != 0:
        raise MemoryError("oracle potrs adjoint could not allocate its scratch matrix")
    return (adjB.reshape(-1) if vec else adjB), out


def potrf_upper(A):
    """Return ``(U, info)``: A = U^T U from A's upper triangle (stacked
    ``[batch, n, n]`` arrays element by element); U's strict lower triangle is
    zero."""
    A = _f64(A)
    lib = _load()
    if A.ndim == 3:
        outs = [potrf_upper(A[b]) for b in range(A.shape[0])]
        return np.stack([o[0] for o in outs]), np.array([o[1] for o in outs], dtype=np.int32)
    n = A.shape[0]
    U = np.zeros_like(A)
    info = int(lib.oracle_potrf_upper(n, _ptr(A), n, _ptr(U), n))
    if info < 0:
        raise MemoryError("oracle upper factor could not allocate its scratch matrices")
    return U, info


def potrf_adjoint_upper(U, adjU, adjA=None, accumulate: bool = True):
    """Adjoint of the upper form: upper(adj_A) += (or =) G^T; the strict lower
    triangle of adj_A is returned unchanged (zero if not given)."""
    U = _f64(U)
    adjU = _f64(adjU)
    out = np.zeros_like(U) if adjA is None else _f64(adjA).copy()
    lib = _load()
    if U.ndim == 3:
        for b in range(U.shape[0]):
            out[b] = potrf_adjoint_upper(U[b], adjU[b], out[b], accumulate)
        return out
    n = U.shape[0]
    rc = lib.oracle_potrf_adjoint_upper(n, _ptr(U), n, _ptr(adjU), n, _ptr(out), n, 1 if accumulate else 0)
    if rc != 0:
        raise MemoryError("oracle upper adjoint could not allocate its scratch matrices")
    return out


def wsum(a) -> float:
    """y = sum_k a_k (ascending order)."""
    a = _f64(a)
    assert a.ndim == 1
    return float(_load().oracle_sum(a.size, _ptr(a)))


def wsum_adjoint(n: int, ybar: float):
    """a_bar for y = sum a given y_bar, starting from zero."""
    abar = np.zeros(n)
    _load().oracle_sum_adjoint(n, float(ybar), _ptr(abar))
    return abar


def _c128(x) -> np.ndarray:
    return np.ascontiguousarray(np.asarray(x, dtype=np.complex128))


def zpotrf(A):
    """Return ``(L, info)``, A = L L^H (complex128; stacked arrays element by
    element).  Only the lower triangle of A is read."""
    A = _c128(A)
    if A.ndim == 3:
        outs = [zpotrf(A[b]) for b in range(A.shape[0])]
        return np.stack([o[0] for o in outs]), np.array([o[1] for o in outs], dtype=np.int32)
    n = A.shape[0]
    L = np.zeros_like(A)
    info = int(_load().oracle_zpotrf(n, _ptr(A), n, _ptr(L), n))
    return L, info


def zpotrf_adjoint(L, adjL, adjA=None, accumulate: bool = True):
    """Adjoint of the Hermitian factor: lower(adj_A) += (or =) G, gradients as
    d/dRe + i d/dIm; the strict upper triangle of adj_A is returned unchanged."""
    L = _c128(L)
    adjL = _c128(adjL)
    out = np.zeros_like(L) if adjA is None else _c128(adjA).copy()
    if L.ndim == 3:
        for b in range(L.shape[0]):
            out[b] = zpotrf_adjoint(L[b], adjL[b], out[b], accumulate)
        return out
    n = L.shape[0]
    rc = _load().oracle_zpotrf_adjoint(n, _ptr(L), n, _ptr(adjL), n, _ptr(out), n, 1 if accumulate else 0)
    if rc != 0:
        raise MemoryError("oracle complex adjoint could not allocate its scratch matrices")
    return out
