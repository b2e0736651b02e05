"""The C-ABI boundary on the CPU: the library loads, exports every entry point
the header declares, and rejects bad arguments on the host before launching
anything.  No call here reaches a kernel launch."""
import ctypes

import pytest

dc = pytest.importorskip("differentiable_cholesky_amd")
from differentiable_cholesky_amd import _lib  # noqa: E402

lib = _lib.lib
F32, F64 = _lib.CHOL_F32, _lib.CHOL_F64
OK, INVALID, NOTSUP, WS = (_lib.CHOL_OK, _lib.CHOL_ERR_INVALID_VALUE, _lib.CHOL_ERR_NOT_SUPPORTED,
                           _lib.CHOL_ERR_WORKSPACE)

# fake, never dereferenced device addresses (every call below fails validation first)
P1 = ctypes.c_void_p(0x10000000)
P2 = ctypes.c_void_p(0x20000000)
P3 = ctypes.c_void_p(0x30000000)
NUL = ctypes.c_void_p(0)


def test_abi_version():
    assert lib.chol_abi_version() == 1


def test_every_declared_entry_point_is_exported():
    names = _lib.header_entry_points()
    assert set(names) >= {"chol_potrf", "chol_potrf_batched", "chol_potrf_adjoint",
                          "chol_potrf_adjoint_batched", "chol_potrf_adjoint_workspace_size",
                          "chol_status_string", "chol_abi_version", "chol_wave_dot_fwd_adj"}
    for n in names:
        assert hasattr(lib, n), n


def test_status_strings():
    for s in range(5):
        assert lib.chol_status_string(s).startswith(b"CHOL_")
    assert b"unknown" in lib.chol_status_string(99)


@pytest.mark.parametrize("args,expect", [
    ((7, 10, P1, 10, P2, 10, NUL, 0, NUL), INVALID),          # bad dtype
    ((F64, -1, P1, 10, P2, 10, NUL, 0, NUL), INVALID),        # n < 0
    ((F64, 0, NUL, 0, NUL, 0, NUL, 0, NUL), OK),              # empty: no-op
    ((F64, 10, NUL, 10, P2, 10, NUL, 0, NUL), INVALID),       # null A
    ((F64, 10, P1, 10, NUL, 10, NUL, 0, NUL), INVALID),       # null L
    ((F64, 10, P1, 9, P2, 10, NUL, 0, NUL), INVALID),         # lda < n
    ((F64, 10, P1, 10, P2, 9, NUL, 0, NUL), INVALID),         # ldl < n
    ((F64, 100, P1, 100, P2, 100, NUL, -1, NUL), INVALID),    # nb < 0
    ((F64, 100, P1, 100, P2, 100, NUL, 129, NUL), INVALID),   # nb > max
    ((F64, 1000, P1, 1000, P2, 1000, NUL, 256, NUL), INVALID),  # nb = 256: tiles stop at 128
    ((F64, 10, P1, 10, ctypes.c_void_p(0x10000000 + 8), 10, NUL, 0, NUL), INVALID),  # partial overlap
    ((F64, 10, P1, 10, P1, 12, NUL, 0, NUL), INVALID),        # same buffer, different ld
    ((F64, 10, P1, 10, P2, 10, ctypes.c_void_p(0x20000000 + 16), 0, NUL), INVALID),  # info inside L
])
def test_potrf_argument_errors(args, expect):
    assert lib.chol_potrf(*args) == expect


@pytest.mark.parametrize("args,expect", [
    ((F32, 65, 4, P1, 65, 65 * 65, P2, 65, 65 * 65, NUL, NUL), NOTSUP),     # n > 64
    ((F32, 8, -1, P1, 8, 64, P2, 8, 64, NUL, NUL), INVALID),                 # batch < 0
    ((F32, 8, 0, NUL, 8, 64, NUL, 8, 64, NUL, NUL), OK),                     # empty batch
    ((F32, 8, 4, P1, 8, 63, P2, 8, 64, NUL, NUL), INVALID),                  # strideA < ld*n
    ((F32, 8, 4, P1, 8, 64, P2, 7, 64, NUL, NUL), INVALID),                  # ldl < n
    ((F32, 8, 4, P1, 8, 64, ctypes.c_void_p(0x10000000 + 4 * 100), 8, 64, NUL, NUL), INVALID),  # overlap
    ((F32, 8, 4, P1, 8, 64, P1, 8, 72, NUL, NUL), INVALID),                  # in place, different stride
])
def test_batched_argument_errors(args, expect):
    assert lib.chol_potrf_batched(*args) == expect


def _ws(dt, n, nb, acc, inplace):
    out = ctypes.c_size_t(123)
    st = lib.chol_potrf_adjoint_workspace_size(dt, n, nb, acc, inplace, ctypes.byref(out))
    return st, out.value


def test_workspace_size_query():
    assert _ws(F64, 64, 0, 1, 0) == (OK, 0)
    st, b = _ws(F64, 1000, 0, 1, 0)
    assert st == OK and b >= 1000 * 1000 * 8
    st, b0 = _ws(F64, 1000, 0, 0, 0)
    assert st == OK and 0 < b0 and b - b0 >= 1000 * 1000 * 8   # the n x n gradient copy
    st, b1 = _ws(F64, 1000, 0, 0, 1)
    assert st == OK and b1 == b0
    assert _ws(F64, 1000, 0, 1, 1)[0] == INVALID              # in place needs accumulate == 0
    assert _ws(F32, 1000, 200, 1, 0)[0] == INVALID            # nb too large
    assert lib.chol_potrf_adjoint_workspace_size(F64, 10, 0, 1, 0, None) == INVALID


def test_adjoint_argument_errors():
    n = 1000
    # in place with accumulate
    assert lib.chol_potrf_adjoint(F64, n, P1, n, P2, n, P2, n, 1, 0, P3, 1 << 40, NUL) == INVALID
    # adjA overlapping L
    assert lib.chol_potrf_adjoint(F64, n, P1, n, P2, n, ctypes.c_void_p(0x10000000 + 8 * 5), n, 0, 0, P3,
                                  1 << 40, NUL) == INVALID
    # missing / small workspace
    assert lib.chol_potrf_adjoint(F64, n, P1, n, P2, n, P3, n, 1, 0, NUL, 0, NUL) == WS
    st, need = _ws(F64, n, 0, 1, 0)
    big = ctypes.c_void_p(0x7000000000)
    assert lib.chol_potrf_adjoint(F64, n, P1, n, P2, n, P3, n, 1, 0, big, need - 1, NUL) == WS
    # workspace overlapping an operand
    assert lib.chol_potrf_adjoint(F64, n, P1, n, P2, n, P3, n, 1, 0, P2, need, NUL) == INVALID
    # bad ld / null
    assert lib.chol_potrf_adjoint(F64, n, P1, n - 1, P2, n, P3, n, 1, 0, big, need, NUL) == INVALID
    assert lib.chol_potrf_adjoint(F64, n, NUL, n, P2, n, P3, n, 1, 0, big, need, NUL) == INVALID
    assert lib.chol_potrf_adjoint(F64, 0, NUL, 0, NUL, 0, NUL, 0, 1, 0, NUL, 0, NUL) == OK


def test_adjoint_batched_argument_errors():
    assert lib.chol_potrf_adjoint_batched(F32, 65, 2, P1, 65, 65 * 65, P2, 65, 65 * 65, P3, 65, 65 * 65, 1,
                                          NUL) == NOTSUP
    assert lib.chol_potrf_adjoint_batched(F32, 8, 2, P1, 8, 64, P2, 8, 64, P2, 8, 64, 1, NUL) == INVALID
    assert lib.chol_potrf_adjoint_batched(F32, 8, 2, P1, 8, 64, P2, 8, 64, ctypes.c_void_p(0x10000000 + 40),
                                          8, 64, 0, NUL) == INVALID
    assert lib.chol_potrf_adjoint_batched(F32, 8, 0, NUL, 8, 64, NUL, 8, 64, NUL, 8, 64, 1, NUL) == OK


def test_wave_dot_argument_errors():
    assert lib.chol_wave_dot_fwd_adj(F32, 65, P1, P2, P3, P1, P2, P3, 0, NUL) == INVALID
    assert lib.chol_wave_dot_fwd_adj(F32, 16, P1, P2, P3, P1, P2, P3, 2, NUL) == INVALID
    assert lib.chol_wave_dot_fwd_adj(F32, 16, NUL, P2, P3, P1, P2, P3, 0, NUL) == INVALID


def test_binding_rejects_cpu_tensors():
    torch = pytest.importorskip("torch")
    A = torch.eye(4, dtype=torch.float64)
    with pytest.raises(ValueError):
        dc.chol_potrf(A, L=A.clone(), info=torch.zeros(1, dtype=torch.int32))


def test_library_binds_to_torch_hip_runtime():
    # importing the package with no earlier torch import must still leave one
    # HIP runtime in the process: the one torch's tensors and streams live in
    import subprocess
    import sys
    root = _lib.HERE.rsplit("/", 1)[0]
    code = ("import sys; sys.path.insert(0, %r); import differentiable_cholesky_amd as d; "
            "print(len(d._lib._hip_runtimes()))" % root)
    out = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, timeout=300)
    assert out.returncode == 0, out.stderr
    assert out.stdout.strip().splitlines()[-1] == "1"


def test_init_reports_hip_failure_without_a_device():
    # chol_init is the one-time set-up; with no device visible it must fail
    # with CHOL_ERR_HIP (and a recorded HIP error), never crash
    torch = pytest.importorskip("torch")
    if torch.cuda.is_available():
        pytest.skip("a GPU is visible")
    assert lib.chol_init() == _lib.CHOL_ERR_HIP
    assert lib.chol_last_hip_error() != 0


def test_noalloc_adjoint_argument_errors():
    # the allocation-free adjoint validates like chol_potrf_adjoint and
    # rejects sizes beyond its static workspace before launching anything
    n = _lib.NOALLOC_MAX_N
    f = lib.chol_potrf_adjoint_noalloc
    assert f(F64, n + 1, P1, n + 1, P2, n + 1, P3, n + 1, 1, 0, NUL) == NOTSUP
    assert f(F64, n, P1, n, P2, n, P2, n, 1, 0, NUL) == INVALID          # in place with accumulate
    assert f(F64, n, NUL, n, P2, n, P3, n, 1, 0, NUL) == INVALID
    assert f(F64, n, P1, n, P2, n, P3, n, 1, 129, NUL) == INVALID      # nb too large
    assert f(F64, 0, NUL, 0, NUL, 0, NUL, 0, 1, 0, NUL) == OK


def test_hbm_stream_argument_errors():
    f = lib.chol_hbm_stream
    assert f(3, P1, P2, 1 << 20, NUL) == INVALID                       # unknown mode
    assert f(2, P1, P2, (1 << 20) + 8, NUL) == INVALID                 # not a multiple of 16
    assert f(2, P1, ctypes.c_void_p(0x10000000 + 64), 1 << 20, NUL) == INVALID   # overlapping copy
    assert f(0, NUL, P2, 1 << 20, NUL) == INVALID                      # read without a source
    assert f(2, P1, P2, 0, NUL) == OK


def test_potrs_argument_errors():
    n = 100
    big = ctypes.c_void_p(0x7000000000)
    ws = ctypes.c_size_t(0)
    assert lib.chol_potrs_workspace_size(F64, n, 3, 0, ctypes.byref(ws)) == OK and ws.value > 0
    assert lib.chol_potrs_workspace_size(F64, 64, 3, 0, ctypes.byref(ws)) == OK and ws.value == 0
    assert lib.chol_potrs_workspace_size(F64, n, 3, 129, ctypes.byref(ws)) == INVALID
    need = ctypes.c_size_t(0)
    lib.chol_potrs_workspace_size(F64, n, 3, 0, ctypes.byref(need))
    need = need.value
    # empty problems are no-ops
    assert lib.chol_potrs(F64, 0, 3, NUL, 1, NUL, 3, NUL, 3, 0, NUL, 0, NUL) == OK
    assert lib.chol_potrs(F64, n, 0, NUL, n, NUL, 1, NUL, 1, 0, NUL, 0, NUL) == OK
    # bad dtype / sizes / leading dimensions / nulls
    assert lib.chol_potrs(7, n, 3, P1, n, P2, 3, P3, 3, 0, big, need, NUL) == INVALID
    assert lib.chol_potrs(F64, -1, 3, P1, n, P2, 3, P3, 3, 0, big, need, NUL) == INVALID
    assert lib.chol_potrs(F64, n, -1, P1, n, P2, 3, P3, 3, 0, big, need, NUL) == INVALID
    assert lib.chol_potrs(F64, n, 3, P1, n - 1, P2, 3, P3, 3, 0, big, need, NUL) == INVALID
    assert lib.chol_potrs(F64, n, 3, P1, n, P2, 2, P3, 3, 0, big, need, NUL) == INVALID
    assert lib.chol_potrs(F64, n, 3, P1, n, P2, 3, P3, 2, 0, big, need, NUL) == INVALID
    assert lib.chol_potrs(F64, n, 3, NUL, n, P2, 3, P3, 3, 0, big, need, NUL) == INVALID
    assert lib.chol_potrs(F64, n, 3, P1, n, P2, 3, P3, 3, 129, big, need, NUL) == INVALID
    # X partly over B, X over L, in place with another ld
    assert lib.chol_potrs(F64, n, 3, P1, n, P2, 3, ctypes.c_void_p(0x20000000 + 8), 3, 0, big, need, NUL) == INVALID
    assert lib.chol_potrs(F64, n, 3, P1, n, P2, 3, ctypes.c_void_p(0x10000000 + 80), 3, 0, big, need,
                          NUL) == INVALID
    assert lib.chol_potrs(F64, n, 3, P1, n, P2, 3, P2, 4, 0, big, need, NUL) == INVALID
    # workspace missing, short, or over an operand
    assert lib.chol_potrs(F64, n, 3, P1, n, P2, 3, P3, 3, 0, NUL, 0, NUL) == WS
    assert lib.chol_potrs(F64, n, 3, P1, n, P2, 3, P3, 3, 0, big, need - 1, NUL) == WS
    assert lib.chol_potrs(F64, n, 3, P1, n, P2, 3, P3, 3, 0, P1, need, NUL) == INVALID
    # batched: n > 64 not supported, stride too small, overlap
    assert lib.chol_potrs_batched(F32, 65, 1, 2, P1, 65, 65 * 65, P2, 1, 65, P3, 1, 65, NUL) == NOTSUP
    assert lib.chol_potrs_batched(F32, 8, 2, 2, P1, 8, 63, P2, 2, 16, P3, 2, 16, NUL) == INVALID
    assert lib.chol_potrs_batched(F32, 8, 2, 2, P1, 8, 64, P2, 2, 15, P3, 2, 16, NUL) == INVALID
    assert lib.chol_potrs_batched(F32, 8, 2, 2, P1, 8, 64, P2, 2, 16, ctypes.c_void_p(0x20000000 + 4), 2, 16,
                                  NUL) == INVALID
    assert lib.chol_potrs_batched(F32, 8, 2, 0, NUL, 8, 64, NUL, 2, 16, NUL, 2, 16, NUL) == OK


def test_potrs_adjoint_argument_errors():
    n, r = 100, 3
    big = ctypes.c_void_p(0x7000000000)
    need = ctypes.c_size_t(0)
    assert lib.chol_potrs_adjoint_workspace_size(F64, n, r, 0, ctypes.byref(need)) == OK and need.value > 0
    need = need.value
    P4 = ctypes.c_void_p(0x40000000)
    P5 = ctypes.c_void_p(0x50000000)
    ok = (F64, n, r, P1, n, P2, r, P3, r, P4, r, P5, n, 1, 0, big, need, NUL)
    assert lib.chol_potrs_adjoint(*ok[:-3], NUL, 0, NUL) == WS
    # adj_B may be adj_X (same ld), not X; adj_L must stay apart from every operand
    assert lib.chol_potrs_adjoint(F64, n, r, P1, n, P2, r, P3, r, P3, r + 1, P5, n, 1, 0, big, need, NUL) == INVALID
    assert lib.chol_potrs_adjoint(F64, n, r, P1, n, P2, r, P3, r, P2, r, P5, n, 1, 0, big, need, NUL) == INVALID
    assert lib.chol_potrs_adjoint(F64, n, r, P1, n, P2, r, P3, r, P4, r, P1, n, 1, 0, big, need, NUL) == INVALID
    assert lib.chol_potrs_adjoint(F64, n, r, P1, n, P2, r, P3, r, P4, r, P4, n, 1, 0, big, need, NUL) == INVALID
    assert lib.chol_potrs_adjoint(F64, n, r, P1, n, P2, r, P3, r, P4, r, P5, n - 1, 1, 0, big, need, NUL) == INVALID
    assert lib.chol_potrs_adjoint(F64, n, r, P1, n, NUL, r, P3, r, P4, r, P5, n, 1, 0, big, need, NUL) == INVALID
    assert lib.chol_potrs_adjoint(F64, n, r, P1, n, P2, r, P3, r, P4, r, P5, n, 1, 0, P5, need, NUL) == INVALID
    # no right-hand side: accumulate is a no-op; adj_L is still checked
    assert lib.chol_potrs_adjoint(F64, n, 0, NUL, n, NUL, 1, NUL, 1, NUL, 1, P5, n, 1, 0, NUL, 0, NUL) == OK
    assert lib.chol_potrs_adjoint(F64, n, 0, NUL, n, NUL, 1, NUL, 1, NUL, 1, NUL, n, 0, 0, NUL, 0, NUL) == INVALID
    assert lib.chol_potrs_adjoint_batched(F64, 65, r, 2, P1, 65, 65 * 65, P2, r, 65 * r, P3, r, 65 * r, P4, r,
                                          65 * r, P5, 65, 65 * 65, 1, NUL) == NOTSUP


def test_upper_argument_errors():
    n = 100
    big = ctypes.c_void_p(0x7000000000)
    assert lib.chol_potrf_upper(F64, 0, NUL, 0, NUL, 0, NUL, 0, NUL) == OK
    assert lib.chol_potrf_upper(F64, n, NUL, n, P2, n, NUL, 0, NUL) == INVALID
    assert lib.chol_potrf_upper(F64, n, P1, n - 1, P2, n, NUL, 0, NUL) == INVALID
    assert lib.chol_potrf_upper(F64, n, P1, n, ctypes.c_void_p(0x10000000 + 8), n, NUL, 0, NUL) == INVALID
    assert lib.chol_potrf_upper(F64, n, P1, n, P2, n, NUL, 129, NUL) == INVALID
    assert lib.chol_potrf_upper_batched(F32, 65, 2, P1, 65, 65 * 65, P2, 65, 65 * 65, NUL, NUL) == NOTSUP
    assert lib.chol_potrf_upper_batched(F32, 8, 2, P1, 8, 63, P2, 8, 64, NUL, NUL) == INVALID
    ws = ctypes.c_size_t(0)
    assert lib.chol_potrf_adjoint_upper_workspace_size(F64, n, 1, 0, ctypes.byref(ws)) == OK
    need = ws.value
    assert need >= 2 * n * n * 8
    assert lib.chol_potrf_adjoint_upper_workspace_size(F64, n, 2, 0, ctypes.byref(ws)) == NOTSUP
    assert lib.chol_potrf_adjoint_upper_workspace_size(F32, 32, 3, 0, ctypes.byref(ws)) == OK
    assert ws.value >= 2 * 3 * 32 * 32 * 4
    assert lib.chol_potrf_adjoint_upper(F64, n, P1, n, P2, n, P3, n, 1, 0, NUL, 0, NUL) == WS
    assert lib.chol_potrf_adjoint_upper(F64, n, P1, n, P2, n, P3, n, 1, 0, big, need - 1, NUL) == WS
    assert lib.chol_potrf_adjoint_upper(F64, n, P1, n, P2, n, P3, n, 1, 0, P3, need, NUL) == INVALID
    # adj_A over U, or partly over adj_U
    assert lib.chol_potrf_adjoint_upper(F64, n, P1, n, P2, n, P1, n, 1, 0, big, need, NUL) == INVALID
    assert lib.chol_potrf_adjoint_upper(F64, n, P1, n, P2, n, ctypes.c_void_p(0x20000000 + 8), n, 1, 0, big, need,
                                        NUL) == INVALID
    assert lib.chol_potrf_adjoint_upper_batched(F32, 65, 2, P1, 65, 65 * 65, P2, 65, 65 * 65, P3, 65, 65 * 65, 1,
                                                big, 1 << 30, NUL) == NOTSUP


def test_wave_sum_argument_errors():
    assert lib.chol_wave_sum_fwd_adj(F32, 65, P1, P2, P3, P1, 0, NUL) == INVALID
    assert lib.chol_wave_sum_fwd_adj(F32, 16, P1, P2, P3, P1, 2, NUL) == INVALID
    assert lib.chol_wave_sum_fwd_adj(F32, 16, NUL, P2, P3, P1, 0, NUL) == INVALID
    assert lib.chol_wave_sum_fwd_adj(7, 16, P1, P2, P3, P1, 0, NUL) == INVALID


def test_hermitian_argument_errors():
    C64, C128 = _lib.CHOL_C64, _lib.CHOL_C128
    n = 100
    big = ctypes.c_void_p(0x7000000000)
    ws = ctypes.c_size_t(0)
    assert lib.chol_potrf_hermitian_workspace_size(C128, n, 1, 0, 0, ctypes.byref(ws)) == OK
    assert ws.value >= 4 * n * n * 8
    need = ws.value
    assert lib.chol_potrf_hermitian_workspace_size(C128, n, 1, 0, 1, ctypes.byref(ws)) == OK
    assert ws.value >= 2 * 4 * n * n * 8
    need_adj = ws.value
    assert lib.chol_potrf_hermitian_workspace_size(F64, n, 1, 0, 0, ctypes.byref(ws)) == INVALID
    assert lib.chol_potrf_hermitian_workspace_size(C64, 33, 2, 0, 0, ctypes.byref(ws)) == NOTSUP
    # real dtypes are rejected by the Hermitian entry points and complex ones by the real ones
    assert lib.chol_potrf_hermitian(F64, n, P1, n, P2, n, NUL, 0, big, need, NUL) == INVALID
    assert lib.chol_potrf(C128, n, P1, n, P2, n, NUL, 0, NUL) == INVALID
    assert lib.chol_potrf_hermitian(C128, 0, NUL, 0, NUL, 0, NUL, 0, NUL, 0, NUL) == OK
    assert lib.chol_potrf_hermitian(C128, n, P1, n, P2, n, NUL, 0, NUL, 0, NUL) == WS
    assert lib.chol_potrf_hermitian(C128, n, P1, n, P2, n, NUL, 0, big, need - 1, NUL) == WS
    assert lib.chol_potrf_hermitian(C128, n, P1, n - 1, P2, n, NUL, 0, big, need, NUL) == INVALID
    # L partly over A (complex elements are 16 bytes), workspace over an operand
    assert lib.chol_potrf_hermitian(C128, n, P1, n, ctypes.c_void_p(0x10000000 + 16), n, NUL, 0, big, need,
                                    NUL) == INVALID
    assert lib.chol_potrf_hermitian(C128, n, P1, n, P2, n, NUL, 0, P2, need, NUL) == INVALID
    assert lib.chol_potrf_hermitian_batched(C64, 33, 2, P1, 33, 33 * 33, P2, 33, 33 * 33, NUL, big, 1 << 30,
                                            NUL) == NOTSUP
    # adjoint: adjA over L, missing workspace
    assert lib.chol_potrf_adjoint_hermitian(C128, n, P1, n, P2, n, P1, n, 1, 0, big, need_adj, NUL) == INVALID
    assert lib.chol_potrf_adjoint_hermitian(C128, n, P1, n, P2, n, P3, n, 1, 0, NUL, 0, NUL) == WS
    assert lib.chol_potrf_adjoint_hermitian_batched(C64, 33, 2, P1, 33, 33 * 33, P2, 33, 33 * 33, P3, 33, 33 * 33,
                                                    1, big, 1 << 30, NUL) == NOTSUP
