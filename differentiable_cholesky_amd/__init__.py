"""libchol: Cholesky factor A = L L^T and its reverse-mode adjoint on AMD MI355X.

The computation lives in hand-written HIP kernels behind the C-ABI declared in
``include/libchol.h``; this package only binds that library (``_lib``) and
builds it (``build``).  Importing the package loads ``libchol.so`` and fails
loudly if it has not been built.
"""
from ._lib import (  # noqa: F401
    CHOL_C64,
    CHOL_C128,
    CHOL_F32,
    CHOL_F64,
    CholError,
    MAX_NB,
    SMALL_MAX_N,
    chol_abi_version,
    chol_hbm_stream,
    chol_init,
    chol_potrf,
    chol_potrf_adjoint,
    chol_potrf_adjoint_batched,
    chol_potrf_adjoint_hermitian,
    chol_potrf_adjoint_hermitian_batched,
    chol_potrf_adjoint_noalloc,
    chol_potrf_adjoint_workspace_size,
    chol_potrf_batched,
    chol_potrf_hermitian,
    chol_potrf_hermitian_batched,
    chol_potrf_hermitian_workspace_size,
    chol_potrf_adjoint_upper,
    chol_potrf_adjoint_upper_batched,
    chol_potrf_adjoint_upper_workspace_size,
    chol_potrf_plan,
    chol_potrf_upper,
    chol_potrf_upper_batched,
    chol_potrs,
    chol_potrs_adjoint,
    chol_potrs_adjoint_batched,
    chol_potrs_adjoint_workspace_size,
    chol_potrs_batched,
    chol_potrs_workspace_size,
    chol_status_string,
    chol_wave_dot_fwd_adj,
    chol_wave_sum_fwd_adj,
    header_entry_points,
    lib,
)
