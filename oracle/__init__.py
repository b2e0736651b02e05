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
    lib.oracle_dot.restype = ctypes.c_double
    lib.oracle_dot.argtypes = [i64, dp, dp]
    lib.oracle_dot_adjoint.restype = None
    lib.oracle_dot_adjoint.argtypes = [i64, dp, dp, ctypes.c_double, dp, dp]
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
