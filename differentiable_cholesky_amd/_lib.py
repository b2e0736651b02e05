"""ctypes binding of libchol (``include/libchol.h``).

Argument marshalling only: every step of the computation runs in the HIP
kernels behind the C-ABI.  The functions named like the C entry points take
torch tensors that live on a ROCm device and pass their device pointers,
leading dimensions and the current torch stream.  There is no CPU fallback:
if the library is missing or fails to load, importing this module raises.
"""
from __future__ import annotations

import ctypes
import os
import re

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libchol.so")
HEADER = os.path.join(os.path.dirname(HERE), "include", "libchol.h")

CHOL_F32, CHOL_F64, CHOL_C64, CHOL_C128 = 0, 1, 2, 3
CHOL_OK, CHOL_ERR_INVALID_VALUE, CHOL_ERR_NOT_SUPPORTED, CHOL_ERR_WORKSPACE, CHOL_ERR_HIP = range(5)
SMALL_MAX_N = 64
MAX_NB = 128
NOALLOC_MAX_N = 1024


class CholError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(msg)
        self.status = status


def _hip_runtimes() -> set[str]:
    """Files of the HIP runtime mapped into this process (Linux)."""
    try:
        with open("/proc/self/maps") as f:
            return {ln.split()[-1] for ln in f if "libamdhip64" in ln}
    except OSError:  # pragma: no cover - not Linux
        return set()


def _load() -> ctypes.CDLL:
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"libchol.so not built at {LIB_PATH}; run `python differentiable_cholesky_amd/build.py`")
    # The tensors and streams handed to the library belong to torch's HIP
    # runtime, so the library must run on that same runtime.  torch ships its
    # own copy; loading torch first makes the dynamic loader bind libchol.so to
    # it instead of mapping a second runtime that owns no device state.
    import torch  # noqa: F401
    lib = ctypes.CDLL(LIB_PATH)
    runtimes = _hip_runtimes()
    if len(runtimes) > 1:
        raise ImportError("libchol.so and torch are bound to different HIP runtimes: " + ", ".join(sorted(runtimes)))
    i64, i32, vp, sz = ctypes.c_int64, ctypes.c_int, ctypes.c_void_p, ctypes.c_size_t
    st = ctypes.c_int
    lib.chol_potrf.restype = st
    lib.chol_potrf.argtypes = [i32, i64, vp, i64, vp, i64, vp, i64, vp]
    lib.chol_potrf_batched.restype = st
    lib.chol_potrf_batched.argtypes = [i32, i64, i64, vp, i64, i64, vp, i64, i64, vp, vp]
    lib.chol_potrf_adjoint.restype = st
    lib.chol_potrf_adjoint.argtypes = [i32, i64, vp, i64, vp, i64, vp, i64, i32, i64, vp, sz, vp]
    lib.chol_potrf_adjoint_workspace_size.restype = st
    lib.chol_potrf_adjoint_workspace_size.argtypes = [i32, i64, i64, i32, i32, ctypes.POINTER(sz)]
    lib.chol_potrf_adjoint_noalloc.restype = st
    lib.chol_potrf_adjoint_noalloc.argtypes = [i32, i64, vp, i64, vp, i64, vp, i64, i32, i64, vp]
    lib.chol_potrf_adjoint_batched.restype = st
    lib.chol_potrf_adjoint_batched.argtypes = [i32, i64, i64, vp, i64, i64, vp, i64, i64, vp, i64, i64, i32, vp]
    lib.chol_hbm_stream.restype = st
    lib.chol_hbm_stream.argtypes = [ctypes.c_int, vp, vp, sz, vp]
    lib.chol_wave_dot_fwd_adj.restype = st
    lib.chol_wave_dot_fwd_adj.argtypes = [i32, i64, vp, vp, vp, vp, vp, vp, i32, vp]
    lib.chol_status_string.restype = ctypes.c_char_p
    lib.chol_status_string.argtypes = [st]
    lib.chol_init.restype = st
    lib.chol_init.argtypes = []
    lib.chol_abi_version.restype = ctypes.c_int
    lib.chol_abi_version.argtypes = []
    lib.chol_potrf_plan.restype = ctypes.c_int64
    lib.chol_potrf_plan.argtypes = [i64, i64, ctypes.c_int, i64, ctypes.POINTER(ctypes.c_int64), i64]
    lib.chol_last_hip_error.restype = ctypes.c_int
    lib.chol_last_hip_error.argtypes = []
    lib.chol_last_hip_error_string.restype = ctypes.c_char_p
    lib.chol_last_hip_error_string.argtypes = []
    lib.chol_profile_start.restype = st
    lib.chol_profile_start.argtypes = [ctypes.c_uint32]
    lib.chol_profile_stop.restype = st
    lib.chol_profile_stop.argtypes = [ctypes.c_int32, vp, vp, vp]
    lib.chol_potrf_hermitian.restype = st
    lib.chol_potrf_hermitian.argtypes = [i32, i64, vp, i64, vp, i64, vp, i64, vp, sz, vp]
    lib.chol_potrf_hermitian_batched.restype = st
    lib.chol_potrf_hermitian_batched.argtypes = [i32, i64, i64, vp, i64, i64, vp, i64, i64, vp, vp, sz, vp]
    lib.chol_potrf_adjoint_hermitian.restype = st
    lib.chol_potrf_adjoint_hermitian.argtypes = [i32, i64, vp, i64, vp, i64, vp, i64, i32, i64, vp, sz, vp]
    lib.chol_potrf_adjoint_hermitian_batched.restype = st
    lib.chol_potrf_adjoint_hermitian_batched.argtypes = [i32, i64, i64, vp, i64, i64, vp, i64, i64, vp, i64, i64,
                                                         i32, vp, sz, vp]
    lib.chol_potrf_hermitian_workspace_size.restype = st
    lib.chol_potrf_hermitian_workspace_size.argtypes = [i32, i64, i64, i64, i32, ctypes.POINTER(sz)]
    lib.chol_wave_sum_fwd_adj.restype = st
    lib.chol_wave_sum_fwd_adj.argtypes = [i32, i64, vp, vp, vp, vp, i32, vp]
    lib.chol_potrf_upper.restype = st
    lib.chol_potrf_upper.argtypes = [i32, i64, vp, i64, vp, i64, vp, i64, vp]
    lib.chol_potrf_upper_batched.restype = st
    lib.chol_potrf_upper_batched.argtypes = [i32, i64, i64, vp, i64, i64, vp, i64, i64, vp, vp]
    lib.chol_potrf_adjoint_upper.restype = st
    lib.chol_potrf_adjoint_upper.argtypes = [i32, i64, vp, i64, vp, i64, vp, i64, i32, i64, vp, sz, vp]
    lib.chol_potrf_adjoint_upper_batched.restype = st
    lib.chol_potrf_adjoint_upper_batched.argtypes = [i32, i64, i64, vp, i64, i64, vp, i64, i64, vp, i64, i64, i32,
                                                     vp, sz, vp]
    lib.chol_potrf_adjoint_upper_workspace_size.restype = st
    lib.chol_potrf_adjoint_upper_workspace_size.argtypes = [i32, i64, i64, i64, ctypes.POINTER(sz)]
    lib.chol_potrs.restype = st
    lib.chol_potrs.argtypes = [i32, i64, i64, vp, i64, vp, i64, vp, i64, i64, vp, sz, vp]
    lib.chol_potrs_workspace_size.restype = st
    lib.chol_potrs_workspace_size.argtypes = [i32, i64, i64, i64, ctypes.POINTER(sz)]
    lib.chol_potrs_batched.restype = st
    lib.chol_potrs_batched.argtypes = [i32, i64, i64, i64, vp, i64, i64, vp, i64, i64, vp, i64, i64, vp]
    lib.chol_potrs_adjoint.restype = st
    lib.chol_potrs_adjoint.argtypes = [i32, i64, i64, vp, i64, vp, i64, vp, i64, vp, i64, vp, i64, i32, i64,
                                       vp, sz, vp]
    lib.chol_potrs_adjoint_workspace_size.restype = st
    lib.chol_potrs_adjoint_workspace_size.argtypes = [i32, i64, i64, i64, ctypes.POINTER(sz)]
    lib.chol_potrs_adjoint_batched.restype = st
    lib.chol_potrs_adjoint_batched.argtypes = [i32, i64, i64, i64, vp, i64, i64, vp, i64, i64, vp, i64, i64,
                                               vp, i64, i64, vp, i64, i64, i32, vp]
    return lib


lib = _load()


def header_entry_points() -> list[str]:
    """Names of the functions ``include/libchol.h`` declares."""
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(chol_[a-z_]+)\s*\(", text)))


def status_string(status: int) -> str:
    return lib.chol_status_string(status).decode()


def _check(status: int):
    if status != CHOL_OK:
        msg = status_string(status)
        if status == CHOL_ERR_HIP:
            msg += f" (HIP error {lib.chol_last_hip_error()}: {lib.chol_last_hip_error_string().decode()})"
        raise CholError(status, msg)


# --------------------------------------------------------------- tensors ----

def _torch():
    import torch
    return torch


def _dtype_code(t) -> int:
    torch = _torch()
    if t.dtype == torch.float32:
        return CHOL_F32
    if t.dtype == torch.float64:
        return CHOL_F64
    raise TypeError(f"libchol handles float32 and float64, got {t.dtype}")


def _mat(t, name: str):
    """(pointer, ld) of a 2-D row-major device matrix (last stride 1)."""
    if t.dim() != 2 or t.shape[0] != t.shape[1]:
        raise ValueError(f"{name} must be a square 2-D tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must live on the GPU")
    if t.shape[1] > 1 and t.stride(1) != 1:
        raise ValueError(f"{name} must have unit column stride")
    return ctypes.c_void_p(t.data_ptr()), max(int(t.stride(0)), int(t.shape[0]), 1)


def _bat(t, name: str):
    """(pointer, ld, stride) of a [batch, n, n] row-major device array."""
    if t.dim() != 3 or t.shape[1] != t.shape[2]:
        raise ValueError(f"{name} must be [batch, n, n]")
    if not t.is_cuda:
        raise ValueError(f"{name} must live on the GPU")
    if t.shape[2] > 1 and t.stride(2) != 1:
        raise ValueError(f"{name} must have unit column stride")
    n = int(t.shape[1])
    ld = max(int(t.stride(1)), n, 1)
    stride = int(t.stride(0)) if t.shape[0] > 1 else ld * n
    return ctypes.c_void_p(t.data_ptr()), ld, stride


def _stream(stream=None):
    torch = _torch()
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def chol_potrf(A, L=None, info=None, nb: int = 0, stream=None):
    """Factor one SPD matrix: returns (L, info).  ``L`` may be ``A`` (in place)."""
    torch = _torch()
    if L is None:
        L = torch.empty_like(A)
    if info is None:
        info = torch.empty(1, dtype=torch.int32, device=A.device)
    pa, lda = _mat(A, "A")
    pl, ldl = _mat(L, "L")
    _check(lib.chol_potrf(_dtype_code(A), A.shape[0], pa, lda, pl, ldl, ctypes.c_void_p(info.data_ptr()),
                          nb, _stream(stream)))
    return L, info


def chol_potrf_batched(A, L=None, info=None, stream=None):
    """Factor [batch, n, n] SPD matrices (n <= 64): returns (L, info[batch])."""
    torch = _torch()
    if L is None:
        L = torch.empty_like(A)
    if info is None:
        info = torch.empty(A.shape[0], dtype=torch.int32, device=A.device)
    pa, lda, sa = _bat(A, "A")
    pl, ldl, sl = _bat(L, "L")
    _check(lib.chol_potrf_batched(_dtype_code(A), A.shape[1], A.shape[0], pa, lda, sa, pl, ldl, sl,
                                  ctypes.c_void_p(info.data_ptr()), _stream(stream)))
    return L, info


def chol_potrf_adjoint_workspace_size(dtype_code: int, n: int, nb: int = 0, accumulate: bool = True,
                                      in_place: bool = False) -> int:
    out = ctypes.c_size_t(0)
    _check(lib.chol_potrf_adjoint_workspace_size(dtype_code, n, nb, 1 if accumulate else 0,
                                                 1 if in_place else 0, ctypes.byref(out)))
    return int(out.value)


def chol_potrf_adjoint(L, adjL, adjA=None, accumulate: bool = True, nb: int = 0, workspace=None,
                       stream=None):
    """Adjoint of the factor: lower(adjA) += G (or = G).  Returns adjA.
    ``adjA`` may be ``adjL`` when ``accumulate`` is False."""
    torch = _torch()
    if adjA is None:
        adjA = torch.zeros_like(L)
    pl, ldl = _mat(L, "L")
    pb, ldb = _mat(adjL, "adjL")
    pa, lda = _mat(adjA, "adjA")
    code = _dtype_code(L)
    n = L.shape[0]
    need = chol_potrf_adjoint_workspace_size(code, n, nb, accumulate, adjA.data_ptr() == adjL.data_ptr())
    if workspace is None and need:
        workspace = torch.empty(need, dtype=torch.uint8, device=L.device)
    wptr = ctypes.c_void_p(workspace.data_ptr() if workspace is not None else 0)
    wbytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _check(lib.chol_potrf_adjoint(code, n, pl, ldl, pb, ldb, pa, lda, 1 if accumulate else 0, nb, wptr,
                                  wbytes, _stream(stream)))
    return adjA


def chol_potrf_adjoint_noalloc(L, adjL, adjA, accumulate: bool = True, nb: int = 0, stream=None):
    """chol_potrf_adjoint without a workspace (n <= CHOL_NOALLOC_MAX_N): the
    library's static device array serves as workspace.  adjA must be given."""
    pl, ldl = _mat(L, "L")
    pb, ldb = _mat(adjL, "adjL")
    pa, lda = _mat(adjA, "adjA")
    _check(lib.chol_potrf_adjoint_noalloc(_dtype_code(L), L.shape[0], pl, ldl, pb, ldb, pa, lda,
                                          1 if accumulate else 0, nb, _stream(stream)))
    return adjA


def chol_potrf_adjoint_batched(L, adjL, adjA=None, accumulate: bool = True, stream=None):
    torch = _torch()
    if adjA is None:
        adjA = torch.zeros_like(L)
    pl, ldl, sl = _bat(L, "L")
    pb, ldb, sb = _bat(adjL, "adjL")
    pa, lda, sa = _bat(adjA, "adjA")
    _check(lib.chol_potrf_adjoint_batched(_dtype_code(L), L.shape[1], L.shape[0], pl, ldl, sl, pb, ldb, sb,
                                          pa, lda, sa, 1 if accumulate else 0, _stream(stream)))
    return adjA


def _cdtype_code(t) -> int:
    torch = _torch()
    if t.dtype == torch.complex64:
        return CHOL_C64
    if t.dtype == torch.complex128:
        return CHOL_C128
    raise TypeError(f"the Hermitian factor takes complex64 or complex128, got {t.dtype}")


def chol_potrf_hermitian_workspace_size(dtype_code: int, n: int, batch: int = 1, nb: int = 0,
                                        adjoint: bool = False) -> int:
    out = ctypes.c_size_t(0)
    _check(lib.chol_potrf_hermitian_workspace_size(dtype_code, n, batch, nb, 1 if adjoint else 0, ctypes.byref(out)))
    return int(out.value)


def chol_potrf_hermitian(A, L=None, info=None, nb: int = 0, workspace=None, stream=None):
    """Hermitian complex factor A = L L^H: returns (L, info); ``L`` may be ``A``."""
    torch = _torch()
    if L is None:
        L = torch.empty_like(A)
    if info is None:
        info = torch.empty(1, dtype=torch.int32, device=A.device)
    pa, lda = _mat(A, "A")
    pl, ldl = _mat(L, "L")
    code = _cdtype_code(A)
    n = A.shape[0]
    _, wptr, wbytes = _workspace(chol_potrf_hermitian_workspace_size(code, n, 1, nb), A.device, workspace)
    _check(lib.chol_potrf_hermitian(code, n, pa, lda, pl, ldl, ctypes.c_void_p(info.data_ptr()), nb, wptr, wbytes,
                                    _stream(stream)))
    return L, info


def chol_potrf_hermitian_batched(A, L=None, info=None, workspace=None, stream=None):
    torch = _torch()
    if L is None:
        L = torch.empty_like(A)
    if info is None:
        info = torch.empty(A.shape[0], dtype=torch.int32, device=A.device)
    pa, lda, sa = _bat(A, "A")
    pl, ldl, sl = _bat(L, "L")
    code = _cdtype_code(A)
    n, batch = A.shape[1], A.shape[0]
    _, wptr, wbytes = _workspace(chol_potrf_hermitian_workspace_size(code, n, batch, 0), A.device, workspace)
    _check(lib.chol_potrf_hermitian_batched(code, n, batch, pa, lda, sa, pl, ldl, sl,
                                            ctypes.c_void_p(info.data_ptr()), wptr, wbytes, _stream(stream)))
    return L, info


def chol_potrf_adjoint_hermitian(L, adjL, adjA=None, accumulate: bool = True, nb: int = 0, workspace=None,
                                 stream=None):
    """Adjoint of the Hermitian factor: lower(adjA) += (or =) G.  Returns adjA."""
    torch = _torch()
    if adjA is None:
        adjA = torch.zeros_like(L)
    pl, ldl = _mat(L, "L")
    pg, ldg = _mat(adjL, "adjL")
    pa, lda = _mat(adjA, "adjA")
    code = _cdtype_code(L)
    n = L.shape[0]
    _, wptr, wbytes = _workspace(chol_potrf_hermitian_workspace_size(code, n, 1, nb, True), L.device, workspace)
    _check(lib.chol_potrf_adjoint_hermitian(code, n, pl, ldl, pg, ldg, pa, lda, 1 if accumulate else 0, nb, wptr,
                                            wbytes, _stream(stream)))
    return adjA


def chol_potrf_adjoint_hermitian_batched(L, adjL, adjA=None, accumulate: bool = True, workspace=None,
                                         stream=None):
    torch = _torch()
    if adjA is None:
        adjA = torch.zeros_like(L)
    pl, ldl, sl = _bat(L, "L")
    pg, ldg, sg = _bat(adjL, "adjL")
    pa, lda, sa = _bat(adjA, "adjA")
    code = _cdtype_code(L)
    n, batch = L.shape[1], L.shape[0]
    _, wptr, wbytes = _workspace(chol_potrf_hermitian_workspace_size(code, n, batch, 0, True), L.device, workspace)
    _check(lib.chol_potrf_adjoint_hermitian_batched(code, n, batch, pl, ldl, sl, pg, ldg, sg, pa, lda, sa,
                                                    1 if accumulate else 0, wptr, wbytes, _stream(stream)))
    return adjA


def chol_potrf_upper(A, U=None, info=None, nb: int = 0, stream=None):
    """Upper form: returns (U, info) with A = U^T U from A's upper triangle.
    ``U`` may be ``A`` (in place)."""
    torch = _torch()
    if U is None:
        U = torch.empty_like(A)
    if info is None:
        info = torch.empty(1, dtype=torch.int32, device=A.device)
    pa, lda = _mat(A, "A")
    pu, ldu = _mat(U, "U")
    _check(lib.chol_potrf_upper(_dtype_code(A), A.shape[0], pa, lda, pu, ldu, ctypes.c_void_p(info.data_ptr()),
                                nb, _stream(stream)))
    return U, info


def chol_potrf_upper_batched(A, U=None, info=None, stream=None):
    torch = _torch()
    if U is None:
        U = torch.empty_like(A)
    if info is None:
        info = torch.empty(A.shape[0], dtype=torch.int32, device=A.device)
    pa, lda, sa = _bat(A, "A")
    pu, ldu, su = _bat(U, "U")
    _check(lib.chol_potrf_upper_batched(_dtype_code(A), A.shape[1], A.shape[0], pa, lda, sa, pu, ldu, su,
                                        ctypes.c_void_p(info.data_ptr()), _stream(stream)))
    return U, info


def chol_potrf_adjoint_upper_workspace_size(dtype_code: int, n: int, batch: int = 1, nb: int = 0) -> int:
    out = ctypes.c_size_t(0)
    _check(lib.chol_potrf_adjoint_upper_workspace_size(dtype_code, n, batch, nb, ctypes.byref(out)))
    return int(out.value)


def chol_potrf_adjoint_upper(U, adjU, adjA=None, accumulate: bool = True, nb: int = 0, workspace=None,
                             stream=None):
    """Adjoint of the upper form: upper(adjA) += (or =) G^T.  Returns adjA."""
    torch = _torch()
    if adjA is None:
        adjA = torch.zeros_like(U)
    pu, ldu = _mat(U, "U")
    pg, ldg = _mat(adjU, "adjU")
    pa, lda = _mat(adjA, "adjA")
    code = _dtype_code(U)
    n = U.shape[0]
    _, wptr, wbytes = _workspace(chol_potrf_adjoint_upper_workspace_size(code, n, 1, nb), U.device, workspace)
    _check(lib.chol_potrf_adjoint_upper(code, n, pu, ldu, pg, ldg, pa, lda, 1 if accumulate else 0, nb, wptr,
                                        wbytes, _stream(stream)))
    return adjA


def chol_potrf_adjoint_upper_batched(U, adjU, adjA=None, accumulate: bool = True, workspace=None, stream=None):
    torch = _torch()
    if adjA is None:
        adjA = torch.zeros_like(U)
    pu, ldu, su = _bat(U, "U")
    pg, ldg, sg = _bat(adjU, "adjU")
    pa, lda, sa = _bat(adjA, "adjA")
    code = _dtype_code(U)
    n, batch = U.shape[1], U.shape[0]
    _, wptr, wbytes = _workspace(chol_potrf_adjoint_upper_workspace_size(code, n, batch, 0), U.device, workspace)
    _check(lib.chol_potrf_adjoint_upper_batched(code, n, batch, pu, ldu, su, pg, ldg, sg, pa, lda, sa,
                                                1 if accumulate else 0, wptr, wbytes, _stream(stream)))
    return adjA


def _rhs(t, name: str, n: int):
    """(pointer, ld, nrhs) of an n x nrhs row-major device matrix (a 1-D tensor
    of n entries is one column)."""
    if not t.is_cuda:
        raise ValueError(f"{name} must live on the GPU")
    if t.dim() == 1:
        if t.shape[0] != n or (n > 1 and t.stride(0) != 1):
            raise ValueError(f"{name} must hold {n} contiguous entries")
        return ctypes.c_void_p(t.data_ptr()), 1, 1
    if t.dim() != 2 or t.shape[0] != n:
        raise ValueError(f"{name} must be [n, nrhs] with n = {n}")
    if t.shape[1] > 1 and t.stride(1) != 1:
        raise ValueError(f"{name} must have unit column stride")
    return ctypes.c_void_p(t.data_ptr()), max(int(t.stride(0)), int(t.shape[1]), 1), int(t.shape[1])


def _rhs_bat(t, name: str, n: int):
    """(pointer, ld, stride, nrhs) of a [batch, n, nrhs] row-major device array."""
    if not t.is_cuda:
        raise ValueError(f"{name} must live on the GPU")
    if t.dim() != 3 or t.shape[1] != n:
        raise ValueError(f"{name} must be [batch, n, nrhs] with n = {n}")
    if t.shape[2] > 1 and t.stride(2) != 1:
        raise ValueError(f"{name} must have unit column stride")
    nrhs = int(t.shape[2])
    ld = max(int(t.stride(1)), nrhs, 1)
    stride = int(t.stride(0)) if t.shape[0] > 1 else ld * n
    return ctypes.c_void_p(t.data_ptr()), ld, stride, nrhs


def _workspace(need: int, device, workspace):
    torch = _torch()
    if workspace is None and need:
        workspace = torch.empty(need, dtype=torch.uint8, device=device)
    wptr = ctypes.c_void_p(workspace.data_ptr() if workspace is not None else 0)
    wbytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    return workspace, wptr, wbytes


def chol_potrs_workspace_size(dtype_code: int, n: int, nrhs: int, nb: int = 0) -> int:
    out = ctypes.c_size_t(0)
    _check(lib.chol_potrs_workspace_size(dtype_code, n, nrhs, nb, ctypes.byref(out)))
    return int(out.value)


def chol_potrs(L, B, X=None, nb: int = 0, workspace=None, stream=None):
    """X = (L L^T)^{-1} B (B: [n] or [n, nrhs]); ``X`` may be ``B`` (in place)."""
    torch = _torch()
    if X is None:
        X = torch.empty_like(B)
    pl, ldl = _mat(L, "L")
    n = L.shape[0]
    pb, ldb, nrhs = _rhs(B, "B", n)
    px, ldx, nx = _rhs(X, "X", n)
    if nx != nrhs:
        raise ValueError("X and B must have the same shape")
    code = _dtype_code(L)
    _, wptr, wbytes = _workspace(chol_potrs_workspace_size(code, n, nrhs, nb), L.device, workspace)
    _check(lib.chol_potrs(code, n, nrhs, pl, ldl, pb, ldb, px, ldx, nb, wptr, wbytes, _stream(stream)))
    return X


def chol_potrs_batched(L, B, X=None, stream=None):
    """X[b] = (L[b] L[b]^T)^{-1} B[b] for [batch, n, n] L and [batch, n, nrhs] B (n <= 64)."""
    torch = _torch()
    if X is None:
        X = torch.empty_like(B)
    pl, ldl, sl = _bat(L, "L")
    n = L.shape[1]
    pb, ldb, sb, nrhs = _rhs_bat(B, "B", n)
    px, ldx, sx, _ = _rhs_bat(X, "X", n)
    _check(lib.chol_potrs_batched(_dtype_code(L), n, nrhs, L.shape[0], pl, ldl, sl, pb, ldb, sb, px, ldx, sx,
                                  _stream(stream)))
    return X


def chol_potrs_adjoint_workspace_size(dtype_code: int, n: int, nrhs: int, nb: int = 0) -> int:
    out = ctypes.c_size_t(0)
    _check(lib.chol_potrs_adjoint_workspace_size(dtype_code, n, nrhs, nb, ctypes.byref(out)))
    return int(out.value)


def chol_potrs_adjoint(L, X, adjX, adjB=None, adjL=None, accumulate: bool = True, nb: int = 0, workspace=None,
                       stream=None):
    """Adjoint of X = chol_potrs(L, B): returns (adjB, adjL) with adjB =
    (L L^T)^{-1} adjX (``adjB`` may be ``adjX``) and lower(adjL) += (or =)
    -tril((adjB X^T + X adjB^T) L)."""
    torch = _torch()
    if adjB is None:
        adjB = torch.empty_like(adjX)
    if adjL is None:
        adjL = torch.zeros_like(L)
    pl, ldl = _mat(L, "L")
    n = L.shape[0]
    px, ldx, nrhs = _rhs(X, "X", n)
    pa, lda, na = _rhs(adjX, "adjX", n)
    pb, ldb, nb_ = _rhs(adjB, "adjB", n)
    if na != nrhs or nb_ != nrhs:
        raise ValueError("X, adjX and adjB must have the same shape")
    pg, ldg = _mat(adjL, "adjL")
    code = _dtype_code(L)
    _, wptr, wbytes = _workspace(chol_potrs_adjoint_workspace_size(code, n, nrhs, nb), L.device, workspace)
    _check(lib.chol_potrs_adjoint(code, n, nrhs, pl, ldl, px, ldx, pa, lda, pb, ldb, pg, ldg,
                                  1 if accumulate else 0, nb, wptr, wbytes, _stream(stream)))
    return adjB, adjL


def chol_potrs_adjoint_batched(L, X, adjX, adjB=None, adjL=None, accumulate: bool = True, stream=None):
    """Batched chol_potrs_adjoint (n <= 64): returns (adjB, adjL)."""
    torch = _torch()
    if adjB is None:
        adjB = torch.empty_like(adjX)
    if adjL is None:
        adjL = torch.zeros_like(L)
    pl, ldl, sl = _bat(L, "L")
    n = L.shape[1]
    px, ldx, sx, nrhs = _rhs_bat(X, "X", n)
    pa, lda, sa, _ = _rhs_bat(adjX, "adjX", n)
    pb, ldb, sb, _ = _rhs_bat(adjB, "adjB", n)
    pg, ldg, sg = _bat(adjL, "adjL")
    _check(lib.chol_potrs_adjoint_batched(_dtype_code(L), n, nrhs, L.shape[0], pl, ldl, sl, px, ldx, sx, pa, lda,
                                          sa, pb, ldb, sb, pg, ldg, sg, 1 if accumulate else 0, _stream(stream)))
    return adjB, adjL


def chol_wave_dot_fwd_adj(a, b, ybar, abar=None, bbar=None, staging: int = 0, stream=None):
    """Returns (y, abar, bbar) of the one-lane-result dot product kernel."""
    torch = _torch()
    y = torch.empty(1, dtype=a.dtype, device=a.device)
    if abar is None:
        abar = torch.zeros_like(a)
    if bbar is None:
        bbar = torch.zeros_like(b)
    p = lambda t: ctypes.c_void_p(t.data_ptr())
    _check(lib.chol_wave_dot_fwd_adj(_dtype_code(a), a.numel(), p(a), p(b), p(y), p(ybar), p(abar), p(bbar),
                                     staging, _stream(stream)))
    return y, abar, bbar


def chol_wave_sum_fwd_adj(a, ybar, abar=None, staging: int = 0, stream=None):
    """Returns (y, abar) of the one-lane-result sum kernel."""
    torch = _torch()
    y = torch.empty(1, dtype=a.dtype, device=a.device)
    if abar is None:
        abar = torch.zeros_like(a)
    p = lambda t: ctypes.c_void_p(t.data_ptr())
    _check(lib.chol_wave_sum_fwd_adj(_dtype_code(a), a.numel(), p(a), p(y), p(ybar), p(abar), staging,
                                     _stream(stream)))
    return y, abar


HBM_READ_SINK_FLOATS = 2048 * 256


def chol_hbm_stream(mode: int, src, dst, nbytes: int, stream=None) -> None:
    """Diagnostic streaming kernel: 0 read src, 1 write dst, 2 copy src to dst."""
    p = lambda t: ctypes.c_void_p(t.data_ptr() if t is not None else 0)
    _check(lib.chol_hbm_stream(mode, p(src), p(dst), nbytes, _stream(stream)))


def chol_status_string(status: int) -> str:
    return status_string(status)


PLAN_FIELDS = ("kind", "stream", "k", "c", "w", "f", "np", "t0", "tn", "slot")


# block slots of the persistent trailing-update grid on a 256-CU MI355X
# (two blocks per CU on all but 16 CUs)
PLAN_SLOTS_MI355X = 480


def chol_potrf_plan(n: int, nb: int = 0, copy: bool = True, slots: int = PLAN_SLOTS_MI355X):
    """The blocked factorisation's schedule for an n x n matrix (host only, no
    GPU call): an int64 array with one row per operation, columns PLAN_FIELDS."""
    import numpy as np
    count = lib.chol_potrf_plan(n, nb, int(bool(copy)), slots, None, 0)
    if count < 0:
        raise CholError(CHOL_ERR_INVALID_VALUE, f"chol_potrf_plan: invalid n={n}, nb={nb} or slots={slots}")
    out = np.zeros((count, len(PLAN_FIELDS)), dtype=np.int64)
    if count:
        got = lib.chol_potrf_plan(n, nb, int(bool(copy)), slots,
                                  out.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)), count)
        assert got == count
    return out


def chol_init() -> None:
    """One-time set-up on the current device (kernels loaded, library streams
    created); optional, the first call does it otherwise."""
    _check(lib.chol_init())


def chol_abi_version() -> int:
    return int(lib.chol_abi_version())


def chol_last_hip_error() -> int:
    return int(lib.chol_last_hip_error())


def chol_last_hip_error_string() -> str:
    return lib.chol_last_hip_error_string().decode()
