/*
 * libchol -- Cholesky factorisation A = L L^T of symmetric positive-definite
 * matrices and its reverse-mode adjoint, on one AMD Instinct MI355X (gfx950).
 *
 * What is computed (sources: the pages this library follows):
 *   - jaxmg documentation, "Cholesky factorization" (potrf example): the
 *     factor is the lower-triangular L with A = L L^T; no solve is performed;
 *     the example validates against an expected factor whose strict upper
 *     triangle is zero; its input may be donated so the factor overwrites it
 *     ("Common setup", "Compute the factor" and the donation warning), and the
 *     lower-level entry returns a status next to the factor ("Advanced:
 *     control the outer jax.jit"); the tile size T_A is a parameter.
 *   - Warp issue #1316, "[REQ] Add adjoint for out-of-place tile Cholesky
 *     factorization", resolution comment: the adjoint is Murray's (2016)
 *     symmetric-matrix derivative -- form Phi(L^T adj_L), apply two triangular
 *     solves against L, and accumulate into the lower triangle of the gradient
 *     of A.
 *
 * Conventions shared by every entry point
 *   - Row-major storage: element (i, j) of a matrix with leading dimension ld
 *     is at p[i * ld + j].  Batched arrays add stride * b for element b.
 *   - "Lower" means i >= j.  Only the lower triangle of A and of adj_L is read.
 *     L's strict upper triangle is written as zero.  adj_A's strict upper
 *     triangle is never written.
 *   - Phi(X) is the lower triangle of X with its diagonal halved.  The adjoint
 *     written to adj_A is G = Phi(S + S^T), S = L^{-T} Phi(L^T adj_L) L^{-1}:
 *     the exact gradient with respect to the lower entries the factorisation
 *     reads (for f(A) = <adj_L, chol(A)>, G_ij = df/dA_ij for i >= j).
 *   - dtype selects fp32 or fp64 for every floating-point array of the call.
 *   - All data pointers are DEVICE pointers owned by the caller.  The library
 *     keeps no reference after a call returns and allocates no device memory
 *     in these calls (the blocked adjoint takes a caller workspace).  What it
 *     keeps per device: two streams and six events, created on the first
 *     blocked call (n > CHOL_SMALL_MAX_N) on that device, and, in the device
 *     memory of its own code object (loaded with the library's kernels), a
 *     256-byte array of work counters and two CHOL_MAX_NB x CHOL_MAX_NB fp64
 *     slots for the forward's diagonal-tile inverses.  If the one-time set-up
 *     fails, the call returns CHOL_ERR_HIP and the next blocked call retries.
 *   - Calls are asynchronous on `stream` (a hipStream_t passed as void*; NULL
 *     is the null stream).  Nothing is synchronised with the host.  A
 *     blocked call runs on the library's two streams, joined to `stream` by
 *     events at entry and exit, so it is ordered on `stream` like one kernel.
 *   - Numerical failure is not an error code: info[b] is set on the device to
 *     0 on success, else to 1 + the first column j whose pivot
 *     d = A_jj - sum_k L_jk^2 fails d > 0 (NaN fails); the factor's columns
 *     >= j are then unspecified.  The adjoint does not check its inputs.
 *   - Argument errors are detected on the host before anything is launched:
 *     n < 0, batch < 0, ld < max(1, n), a batch stride smaller than ld * n,
 *     a NULL data pointer with n > 0 (and batch > 0), an unknown dtype, an
 *     out-of-range tile size, or input and output buffers that overlap without
 *     being exactly the same buffer with the same leading dimension and stride.
 *     These return CHOL_ERR_INVALID_VALUE and launch nothing.  A HIP launch
 *     failure returns CHOL_ERR_HIP.  n == 0 or batch == 0 is a no-op.
 *   - Thread safety: calls from several host threads are safe; calls that share
 *     output buffers or a workspace on concurrent streams race on that memory.
 *     Blocked calls on one device share the library's streams and device
 *     buffers, so they run one after another (never overlapping each other).
 */
#ifndef LIBCHOL_H
#define LIBCHOL_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define LIBCHOL_ABI_VERSION 1

/* Largest matrix edge handled by the batched small-tile kernels. */
#define CHOL_SMALL_MAX_N 64
/* Largest tile of the blocked factorisation (the page's T_A).  A diagonal tile
 * is factored and inverted by one 256-thread workgroup in registers, and every
 * product runs on 128 x 128 output tiles.  Larger tiles are not offered: the
 * trailing update already contracts four tile columns (512) at a time, which
 * gives the data reuse a larger tile would, while a larger diagonal tile would
 * lengthen the serial chain of diagonal factors that the updates hide. */
#define CHOL_MAX_NB 128

/* Real types for every entry point; the complex types (interleaved real and
 * imaginary parts, complex64 = 2 x fp32, complex128 = 2 x fp64) only for the
 * chol_potrf_hermitian* family. */
typedef enum { CHOL_F32 = 0, CHOL_F64 = 1, CHOL_C64 = 2, CHOL_C128 = 3 } chol_dtype;

typedef enum {
    CHOL_OK = 0,
    CHOL_ERR_INVALID_VALUE = 1,
    CHOL_ERR_NOT_SUPPORTED = 2,
    CHOL_ERR_WORKSPACE = 3,
    CHOL_ERR_HIP = 4
} chol_status;

/*
 * chol_potrf -- factor one n x n SPD matrix.
 *   A      [in]  device, n x n, leading dimension lda; lower triangle read.
 *   L      [out] device, n x n, leading dimension ldl.  L == A with ldl == lda
 *                factors in place (the jaxmg "donated input" case) and gives
 *                bitwise the same L as the out-of-place call.
 *   info   [out] device int32[1], or NULL if not wanted.
 *   nb     tile size of the blocked algorithm (the page's T_A): 0 picks the
 *          default (128); otherwise 1 <= nb <= CHOL_MAX_NB.  Matrices with
 *          n <= CHOL_SMALL_MAX_N use the small-tile kernel and ignore nb.
 * For n > CHOL_SMALL_MAX_N the call runs the blocked right-looking
 * factorisation: per tile column a diagonal factor in LDS, a panel solve, and
 * a lower-triangular trailing update on the matrix cores.
 */
chol_status chol_potrf(chol_dtype dtype, int64_t n,
                       const void *A, int64_t lda,
                       void *L, int64_t ldl,
                       int32_t *info, int64_t nb, void *stream);

/*
 * chol_potrf_batched -- factor `batch` independent n x n SPD matrices,
 * n <= CHOL_SMALL_MAX_N (larger n returns CHOL_ERR_NOT_SUPPORTED).
 * Matrix b is at A + b * strideA (elements); likewise for L.  L == A with equal
 * ld and stride is in place.  info: device int32[batch] or NULL.
 * (Warp issue #1316 resolution comment: one tile Cholesky per block, loaded,
 * factored and stored.)
 */
chol_status chol_potrf_batched(chol_dtype dtype, int64_t n, int64_t batch,
                               const void *A, int64_t lda, int64_t strideA,
                               void *L, int64_t ldl, int64_t strideL,
                               int32_t *info, void *stream);

/*
 * chol_potrf_adjoint -- reverse-mode adjoint of chol_potrf for one matrix.
 *   L      [in]  device, the factor (lower triangle read; diagonal must be
 *                nonzero).
 *   adjL   [in]  device, the upstream gradient dLoss/dL; lower triangle read.
 *   adjA   [in/out] device; its lower triangle receives G:
 *                accumulate != 0 : lower(adjA) += G   (gradient-buffer semantics)
 *                accumulate == 0 : lower(adjA)  = G
 *                adjA == adjL (same ld) is allowed only with accumulate == 0;
 *                adj_L is then overwritten with G.
 *   nb     tile size (0 = default 128, else 1..CHOL_MAX_NB); ignored for
 *          n <= CHOL_SMALL_MAX_N.
 *   workspace, workspace_bytes: device scratch of at least the size
 *          chol_potrf_adjoint_workspace_size reports for the same arguments
 *          (NULL / 0 allowed when it reports 0).  Too small returns
 *          CHOL_ERR_WORKSPACE.
 * The blocked form walks the tile columns in reverse order: the adjoint of the
 * trailing update (a symmetric product on the matrix cores), the adjoint of
 * the panel solve, and the formula above on each diagonal tile.
 */
chol_status chol_potrf_adjoint(chol_dtype dtype, int64_t n,
                               const void *L, int64_t ldl,
                               const void *adjL, int64_t ldal,
                               void *adjA, int64_t ldaa,
                               int accumulate, int64_t nb,
                               void *workspace, size_t workspace_bytes,
                               void *stream);

/* Bytes of workspace chol_potrf_adjoint needs for these arguments.
 * in_place != 0 means adjA == adjL. */
chol_status chol_potrf_adjoint_workspace_size(chol_dtype dtype, int64_t n, int64_t nb,
                                              int accumulate, int in_place,
                                              size_t *bytes);

/*
 * chol_potrf_adjoint_noalloc -- chol_potrf_adjoint for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation): the same arguments without the
 * workspace, and the same result (G in the lower triangle of adjA, added with
 * accumulate != 0; adjA == adjL allowed with accumulate == 0).
 *   n      <= CHOL_NOALLOC_MAX_N; larger n returns CHOL_ERR_NOT_SUPPORTED
 *          before anything is launched.
 * The workspace is a device array of CHOL_NOALLOC_SCRATCH_BYTES inside the
 * library's code object (one per device, held until the process ends); the
 * call allocates nothing and creates nothing: its kernels run on `stream`
 * alone (no library stream or event), in the order of the blocked adjoint,
 * with the split count of the large products capped so that the workspace
 * fits.  The array keeps the last call's contents; every value a call reads
 * from it is written by that call first.  Calls on one device share the
 * array and a work counter, so calls that overlap on one GPU (concurrent
 * streams, or concurrent with another chol_potrf_adjoint_noalloc call) race;
 * calls ordered on one stream, or synchronised, do not.  The device address
 * of the array is looked up once per device (by chol_init, or the first
 * call); argument errors as for chol_potrf_adjoint.
 */
#define CHOL_NOALLOC_MAX_N 1024
#define CHOL_NOALLOC_SCRATCH_BYTES (16u << 20)
chol_status chol_potrf_adjoint_noalloc(chol_dtype dtype, int64_t n,
                                       const void *L, int64_t ldl,
                                       const void *adjL, int64_t ldal,
                                       void *adjA, int64_t ldaa,
                                       int accumulate, int64_t nb,
                                       void *stream);

/*
 * chol_potrf_adjoint_batched -- adjoint for `batch` independent matrices,
 * n <= CHOL_SMALL_MAX_N, no workspace.  Strides and in-place rules as in
 * chol_potrf_batched / chol_potrf_adjoint; lower(adjA[b]) receives G_b (added
 * with accumulate != 0).  (Warp issue #1316, resolution comment: the tile
 * Cholesky's adjoint forms Phi(L^T adj_L), applies two triangular solves
 * against L and accumulates into the lower triangle of A's gradient; here one
 * matrix per group of lanes, every matrix of the batch in one launch.)
 */
chol_status chol_potrf_adjoint_batched(chol_dtype dtype, int64_t n, int64_t batch,
                                       const void *L, int64_t ldl, int64_t strideL,
                                       const void *adjL, int64_t ldal, int64_t strideAL,
                                       void *adjA, int64_t ldaa, int64_t strideAA,
                                       int accumulate, void *stream);

/*
 * Upper-factor form (uplo = U): A = U^T U with U upper triangular and positive
 * diagonal, reading only the upper triangle of A; U's strict lower triangle is
 * written as zero.  This is the row-major image of a column-major caller's
 * lower factor: U = L^T for the lower factor L of the same matrix (jaxmg
 * documentation, "Cholesky factorization": the factor of a symmetric
 * positive-definite matrix is unique), so these calls run the lower-form
 * kernels on transposed triangles: A's upper triangle is transposed into the
 * output's lower triangle (in place when U == A), factored there in place,
 * and transposed back (zeros below).  info as chol_potrf (column j of U is
 * row j of L).
 */
chol_status chol_potrf_upper(chol_dtype dtype, int64_t n,
                             const void *A, int64_t lda,
                             void *U, int64_t ldu,
                             int32_t *info, int64_t nb, void *stream);

/* chol_potrf_upper for `batch` matrices, n <= CHOL_SMALL_MAX_N (strides and
 * in-place rules as chol_potrf_batched). */
chol_status chol_potrf_upper_batched(chol_dtype dtype, int64_t n, int64_t batch,
                                     const void *A, int64_t lda, int64_t strideA,
                                     void *U, int64_t ldu, int64_t strideU,
                                     int32_t *info, void *stream);

/*
 * chol_potrf_adjoint_upper -- adjoint of the upper form.  With L = U^T and
 * adj_L = adj_U^T, the gradient with respect to A's upper entries is G^T, G
 * the lower-form adjoint (Warp issue #1316, resolution comment; see
 * chol_potrf_adjoint).  Only the upper triangles of U and adj_U are read;
 * upper(adjA) += G^T (accumulate != 0) or = G^T; adjA's strict lower triangle
 * is not touched.  adjA may be adjU itself (same ld), with either accumulate
 * (adj_U is copied into the workspace first); it must not overlap U.
 * workspace: at least chol_potrf_adjoint_upper_workspace_size(dtype, n, 1,
 * nb) bytes: the transposed copies of U and adj_U (2 n^2 elements) and, for
 * n > CHOL_SMALL_MAX_N, the lower-form adjoint's workspace.
 */
chol_status chol_potrf_adjoint_upper(chol_dtype dtype, int64_t n,
                                     const void *U, int64_t ldu,
                                     const void *adjU, int64_t ldau,
                                     void *adjA, int64_t ldaa,
                                     int accumulate, int64_t nb,
                                     void *workspace, size_t workspace_bytes,
                                     void *stream);

/* chol_potrf_adjoint_upper for `batch` matrices, n <= CHOL_SMALL_MAX_N; the
 * workspace holds 2 * batch * n^2 elements. */
chol_status chol_potrf_adjoint_upper_batched(chol_dtype dtype, int64_t n, int64_t batch,
                                             const void *U, int64_t ldu, int64_t strideU,
                                             const void *adjU, int64_t ldau, int64_t strideAU,
                                             void *adjA, int64_t ldaa, int64_t strideAA,
                                             int accumulate,
                                             void *workspace, size_t workspace_bytes,
                                             void *stream);

/* Bytes of workspace the upper adjoint needs for `batch` matrices (batch > 1
 * only with n <= CHOL_SMALL_MAX_N; larger n returns CHOL_ERR_NOT_SUPPORTED). */
chol_status chol_potrf_adjoint_upper_workspace_size(chol_dtype dtype, int64_t n, int64_t batch, int64_t nb,
                                                    size_t *bytes);

/*
 * Hermitian complex factor A = L L^H (jaxmg documentation, "Cholesky
 * factorization": the factor of a symmetric or Hermitian positive-definite
 * matrix) and its adjoint, dtype CHOL_C64 or CHOL_C128.  Complex arrays hold
 * interleaved (re, im) pairs; leading dimensions and strides count complex
 * elements.  Only the lower triangle of A is read, and of its diagonal only
 * the real part; L has a real positive diagonal and zeros above it.
 * Gradients are taken as d/dRe + i d/dIm.  The adjoint is the real one with
 * conjugate transposes: M = L^H tril(adj_L), Phi keeps the lower triangle
 * and the real part of the diagonal halved, S = L^{-H} Phi(M) L^{-1}, and
 * G_ij = S_ij + conj(S_ji) below the diagonal, G_ii = Re S_ii (so the
 * imaginary part of adj_L's diagonal does not enter).
 * Both run the real kernels on the real embedding: each entry x + iy becomes
 * the 2 x 2 block [[x, -y], [y, x]], the Hermitian A a symmetric 2n x 2n
 * matrix whose real factor is the embedding of L (read back from the first
 * column of each block), and the adjoint folds the real gradient of the
 * embedding's lower entries back onto the complex ones.  This costs twice
 * the flops of a native complex factor.
 *   workspace  device scratch of chol_potrf_hermitian_workspace_size bytes
 *              (adjoint = 0 for the factor, 1 for the adjoint): the 2n x 2n
 *              embeddings (4 n^2 reals per matrix, twice for the adjoint) and,
 *              for 2n > CHOL_SMALL_MAX_N, the real adjoint's workspace.  It
 *              must not overlap the operands.
 *   L == A (same ld and stride) factors in place; adjA may be adjL (it is
 *   read into the workspace first), with either accumulate; adjA must not
 *   overlap L.  lower(adjA) += G (accumulate != 0) or = G.
 * info as chol_potrf, in complex columns.  The batched forms take n <= 32
 * (the embedding's 2n <= CHOL_SMALL_MAX_N); larger n returns
 * CHOL_ERR_NOT_SUPPORTED.
 */
chol_status chol_potrf_hermitian(chol_dtype dtype, int64_t n,
                                 const void *A, int64_t lda,
                                 void *L, int64_t ldl,
                                 int32_t *info, int64_t nb,
                                 void *workspace, size_t workspace_bytes, void *stream);

chol_status chol_potrf_hermitian_batched(chol_dtype dtype, int64_t n, int64_t batch,
                                         const void *A, int64_t lda, int64_t strideA,
                                         void *L, int64_t ldl, int64_t strideL,
                                         int32_t *info,
                                         void *workspace, size_t workspace_bytes, void *stream);

chol_status chol_potrf_adjoint_hermitian(chol_dtype dtype, int64_t n,
                                         const void *L, int64_t ldl,
                                         const void *adjL, int64_t ldal,
                                         void *adjA, int64_t ldaa,
                                         int accumulate, int64_t nb,
                                         void *workspace, size_t workspace_bytes, void *stream);

chol_status chol_potrf_adjoint_hermitian_batched(chol_dtype dtype, int64_t n, int64_t batch,
                                                 const void *L, int64_t ldl, int64_t strideL,
                                                 const void *adjL, int64_t ldal, int64_t strideAL,
                                                 void *adjA, int64_t ldaa, int64_t strideAA,
                                                 int accumulate,
                                                 void *workspace, size_t workspace_bytes, void *stream);

/* Workspace bytes of the Hermitian factor (adjoint == 0) or its adjoint
 * (adjoint != 0) for `batch` matrices. */
chol_status chol_potrf_hermitian_workspace_size(chol_dtype dtype, int64_t n, int64_t batch, int64_t nb,
                                                int adjoint, size_t *bytes);

/*
 * chol_potrs -- solve with the factor: X = A^{-1} B for A = L L^T, given the
 * lower factor L (for example from chol_potrf).  The factor is returned
 * without a solve (jaxmg documentation, "Cholesky factorization", opening
 * paragraph); this is the solve it is computed for, made of the two
 * triangular solves against L that Warp issue #1316's resolution comment
 * names: L Y = B by forward substitution, then L^T X = Y.
 *   L      [in]  device, n x n, leading dimension ldl; lower triangle read.
 *   B      [in]  device, n x nrhs, leading dimension ldb >= max(1, nrhs).
 *   X      [out] device, n x nrhs, leading dimension ldx >= max(1, nrhs).
 *                X == B with ldx == ldb solves in place; otherwise X must
 *                overlap neither B nor L.
 *   nb     tile size of the blocked solve (0 = 128, else 1..CHOL_MAX_NB);
 *          ignored for n <= CHOL_SMALL_MAX_N.
 *   workspace, workspace_bytes: device scratch of at least the size
 *          chol_potrs_workspace_size reports (0 for n <= CHOL_SMALL_MAX_N);
 *          too small returns CHOL_ERR_WORKSPACE.  It must not overlap L, B or X.
 * n <= CHOL_SMALL_MAX_N: one wavefront per matrix, substitution row by row.
 * Larger n: the inverses of the diagonal tiles are formed in the workspace,
 * then both solves run tile by tile as matrix-core products (each diagonal
 * block as a product with its inverse, each off-diagonal block as an update).
 * There is no failure status: a zero or non-finite diagonal entry of L gives
 * non-finite entries in X.  nrhs == 0 is a no-op.
 */
chol_status chol_potrs(chol_dtype dtype, int64_t n, int64_t nrhs,
                       const void *L, int64_t ldl,
                       const void *B, int64_t ldb,
                       void *X, int64_t ldx, int64_t nb,
                       void *workspace, size_t workspace_bytes, void *stream);

/* Bytes of workspace chol_potrs needs (n x nb tile inverses for n >
 * CHOL_SMALL_MAX_N, else 0). */
chol_status chol_potrs_workspace_size(chol_dtype dtype, int64_t n, int64_t nrhs, int64_t nb, size_t *bytes);

/*
 * chol_potrs_batched -- chol_potrs for `batch` independent systems, n <=
 * CHOL_SMALL_MAX_N (larger n returns CHOL_ERR_NOT_SUPPORTED), no workspace.
 * System b uses L + b * strideL, B + b * strideB and X + b * strideX
 * (elements); in place as in chol_potrs (equal ld and stride).
 */
chol_status chol_potrs_batched(chol_dtype dtype, int64_t n, int64_t nrhs, int64_t batch,
                               const void *L, int64_t ldl, int64_t strideL,
                               const void *B, int64_t ldb, int64_t strideB,
                               void *X, int64_t ldx, int64_t strideX, void *stream);

/*
 * chol_potrs_adjoint -- reverse-mode adjoint of X = chol_potrs(L, B).  With
 * A = L L^T, dX = -A^{-1} dA X and dA = dL L^T + L dL^T, so
 *   adj_B = A^{-1} adj_X                        (the same two solves)
 *   adj_L = -tril((adj_B X^T + X adj_B^T) L)    (gradient for the lower entries of L)
 *   L      [in]  device, the factor (lower triangle read).
 *   X      [in]  device, n x nrhs, the solve's result.
 *   adjX   [in]  device, n x nrhs, dLoss/dX.
 *   adjB   [out] device, n x nrhs: written with adj_B (it may be adjX itself,
 *                same ld; it must not overlap X or adjL).
 *   adjL   [in/out] device, n x n; its lower triangle receives adj_L:
 *                accumulate != 0: lower(adjL) += adj_L; == 0: lower(adjL) = adj_L.
 *                The strict upper triangle is not touched.  adjL must not
 *                overlap L, X, adjX or adjB.
 *   nb, workspace, workspace_bytes: as chol_potrs, with the size from
 *          chol_potrs_adjoint_workspace_size.
 * The adj_L term is formed as tril(S P + X Q) with S = adj_B, P = X^T L and
 * Q = S^T L: for n <= CHOL_SMALL_MAX_N one wavefront per matrix; for larger n
 * [Q; P] = [S | X]^T tril(L) as one split-contraction product and
 * lower(adj_L) -= [X | S] [Q; P] as one lower-only product of depth 2 nrhs.
 */
chol_status chol_potrs_adjoint(chol_dtype dtype, int64_t n, int64_t nrhs,
                               const void *L, int64_t ldl,
                               const void *X, int64_t ldx,
                               const void *adjX, int64_t ldax,
                               void *adjB, int64_t ldab,
                               void *adjL, int64_t ldal,
                               int accumulate, int64_t nb,
                               void *workspace, size_t workspace_bytes, void *stream);

/* Bytes of workspace chol_potrs_adjoint needs (0 for n <= CHOL_SMALL_MAX_N). */
chol_status chol_potrs_adjoint_workspace_size(chol_dtype dtype, int64_t n, int64_t nrhs, int64_t nb,
                                              size_t *bytes);

/*
 * chol_potrs_adjoint_batched -- chol_potrs_adjoint for `batch` independent
 * systems, n <= CHOL_SMALL_MAX_N (larger n returns CHOL_ERR_NOT_SUPPORTED),
 * no workspace; per-array strides as in chol_potrs_batched.
 */
chol_status chol_potrs_adjoint_batched(chol_dtype dtype, int64_t n, int64_t nrhs, int64_t batch,
                                       const void *L, int64_t ldl, int64_t strideL,
                                       const void *X, int64_t ldx, int64_t strideX,
                                       const void *adjX, int64_t ldax, int64_t strideAX,
                                       void *adjB, int64_t ldab, int64_t strideAB,
                                       void *adjL, int64_t ldal, int64_t strideAL,
                                       int accumulate, void *stream);

/*
 * chol_wave_dot_fwd_adj -- diagnostic kernel for the reduction/broadcast
 * pattern the small-tile kernels rely on (Warp issue #1374, "adj_tile_dot is
 * missing a block-wide broadcast of adj_ret": a dot product whose result only
 * one lane writes must still hand the upstream gradient to every lane in the
 * reverse pass).  One 64-lane wavefront loads a and b (n <= 64 elements each,
 * fp32 or fp64), reduces y = a.b, and only lane 0 writes y[0].  In the
 * reverse pass only lane 0 reads ybar[0]; it is broadcast to every lane,
 * which then writes abar[k] += ybar*b[k] and bbar[k] += ybar*a[k] for the
 * elements it owns.  `staging` 0 keeps a and b in registers, 1 stages them
 * through LDS.
 */
chol_status chol_wave_dot_fwd_adj(chol_dtype dtype, int64_t n,
                                  const void *a, const void *b, void *y,
                                  const void *ybar, void *abar, void *bbar,
                                  int staging, void *stream);

/*
 * chol_wave_sum_fwd_adj -- the same ownership pattern for the sum reduction
 * (Warp issue #1374 holds up the tile_sum adjoint as the model: it broadcasts
 * the upstream gradient from one thread through shared scratch).  One
 * wavefront loads a (n <= 64), reduces y = sum_k a_k, and only lane 0 writes
 * y[0]; in the reverse pass only lane 0 reads ybar[0], which is published to
 * every lane before abar[k] += ybar.  staging as chol_wave_dot_fwd_adj.
 */
chol_status chol_wave_sum_fwd_adj(chol_dtype dtype, int64_t n, const void *a, void *y,
                                  const void *ybar, void *abar, int staging, void *stream);

/*
 * chol_hbm_stream -- diagnostic: plain streaming kernels that measure the
 * device-memory ceiling the bandwidth-bound kernels are compared with.
 *   mode 0  read `bytes` from src (dst receives CHOL_HBM_READ_SINK_FLOATS
 *           floats of per-thread sums, so that no load is dropped);
 *   mode 1  write `bytes` to dst;
 *   mode 2  copy `bytes` from src to dst (disjoint).
 * bytes must be a multiple of 16 and the pointers 16-byte aligned device
 * pointers; otherwise CHOL_ERR_INVALID_VALUE.  Asynchronous on `stream`.
 */
#define CHOL_HBM_READ_SINK_FLOATS (2048 * 256)
chol_status chol_hbm_stream(int mode, const void *src, void *dst, size_t bytes, void *stream);

/*
 * Timing hook (diagnostics; used by the benchmark for per-kernel rooflines).
 * chol_profile_start(mask) clears previous records and turns timing on for
 * later calls in this process: each launch of a kernel family i below with
 * bit i set in `mask` is then bracketed by a pair of HIP events recorded on
 * the stream it runs on (CHOL_PROFILE_ALL selects every family).  Timing only
 * the families of interest keeps the event records out of the others' path.
 * chol_profile_stop() turns timing off, waits for the recorded events, and
 * writes, for family i < max_ids, the number of launches count[i], their summed
 * duration ms[i] and their summed algorithmic work work[i] (flops for the
 * matrix-core and tile kernels, bytes for the bandwidth-bound ones; the unit of
 * each family is given below).  Arrays are host memory owned by the caller.
 * Returns CHOL_ERR_HIP if an event could not be read.  While timing is on,
 * launches from several host threads are recorded together.
 */
typedef enum {
    CHOL_K_SMALL_FACTOR = 0,     /* batched small-tile factor; bytes: 2 * n(n+1)/2 * elem per matrix */
    CHOL_K_SMALL_ADJOINT = 1,    /* batched small-tile adjoint; bytes: (3 or 4) * n(n+1)/2 * elem */
    CHOL_K_DIAG_FACTOR = 2,      /* blocked: factor of a diagonal tile; flops: kb^3 / 3 */
    CHOL_K_DIAG_INVERSE = 3,     /* blocked: inverse of diagonal tiles; flops: kb^3 / 3 per tile */
    CHOL_K_PANEL_SOLVE = 4,      /* blocked: L_ik = W_ik L_kk^-T; flops: m * kb^2 */
    CHOL_K_TRAILING_UPDATE = 5,  /* blocked: lower trailing update; flops: m (m + 1) kb */
    CHOL_K_ADJ_TRAILING = 6,     /* adjoint: split partials of Sym(Wb22) L_panel; flops: 2 m^2 kb */
    CHOL_K_ADJ_PANEL = 7,        /* adjoint: X = Wb_panel L_kk^-1; flops: m * kb^2 */
    CHOL_K_ADJ_DIAG_UPDATE = 8,  /* adjoint: split partials of X^T L_panel; flops: 2 m kb^2 */
    CHOL_K_ADJ_DIAG = 9,         /* adjoint of the factor on a diagonal tile; flops: 2 kb^3 / 3 */
    CHOL_K_ELEMENTWISE = 10,     /* triangle copies, zeroing, accumulation; bytes moved */
    CHOL_K_REDUCE = 11,          /* sums of split partial products into their target; bytes moved */
    CHOL_K_SOLVE = 12,           /* chol_potrs*, and the solve inside chol_potrs_adjoint*, whole
                                    calls; flops: 2 n^2 nrhs per matrix */
    CHOL_K_SOLVE_ADJOINT = 13,   /* the adj_L term of chol_potrs_adjoint*; flops: 4 n^2 nrhs per matrix */
    CHOL_K_COUNT = 14
} chol_kernel_family;

#define CHOL_PROFILE_ALL 0xffffffffu
chol_status chol_profile_start(uint32_t mask);
chol_status chol_profile_stop(int32_t max_ids, int64_t *count, double *ms, double *work);

/*
 * chol_init -- one-time set-up of the library on the current device: loads its
 * kernels (and with them the device buffers of its code object, listed under
 * "What it keeps per device" above) and creates its two streams and events.
 * Optional: the first call on a device does the same on its own; calling
 * chol_init first keeps that one-time device-memory use and latency out of
 * the first factorisation.  Idempotent and thread-safe.  Returns CHOL_ERR_HIP
 * if a HIP call fails (the set-up is retried by the next call).
 */
chol_status chol_init(void);

/* Human-readable name of a status code (static string, never NULL). */
const char *chol_status_string(chol_status status);

/* LIBCHOL_ABI_VERSION of the loaded library. */
int chol_abi_version(void);

/*
 * chol_potrf_plan -- the schedule chol_potrf's blocked path (n >
 * CHOL_SMALL_MAX_N) enqueues for an n x n matrix with tile size nb, so that it
 * can be checked on the host.  It is the right-looking factorisation of the
 * page's blocked algorithm with the trailing update deferred to groups of
 * panels.  Host only: calls no GPU function.
 *   ops  [out] host, cap rows of CHOL_PLAN_FIELDS int64 each (may be NULL if
 *              cap == 0), one row per operation in enqueue order:
 *     kind    0 copy the lower part of columns 0 .. w-1 of A into L (chain
 *               stream); the columns right of them are brought over by the
 *               first kind-4 operations, which read A (slot 1)
 *             1 factor diagonal tile k (chain stream, or wide where no
 *               far-triangle part runs beside it); slot >= 0: its inverse
 *               is written whole into inverse slot `slot`
 *             2 panel solve of tile column k below its diagonal tile (wide
 *               stream), reading inverse slot `slot`
 *             3 lower part of W[c:, c:c+w] -= Q[c:] Q[c:c+w]^T with Q the
 *               tile columns f .. f+np-1 of L (wide)
 *             4 the lower 128 x 128 tiles t0 .. t0+tn-1 (row-major) of the
 *               trailing triangle W[c:, c:] -= Q Q^T, same Q (wide); slot 1:
 *               W's values are read from A (the tiles' first update, in
 *               place of their copy), -1: from L
 *             5 `stream` waits for every operation enqueued so far on the
 *               other stream
 *             6 clear the strict upper triangle of L (chain)
 *     stream  0 chain, 1 wide;  then k, c, w, f, np, t0, tn, slot (element
 *             offsets and counts; unused fields 0, unused slot -1)
 *   copy nonzero when A and L are different buffers.
 *   slots  block slots of the persistent grid that takes the tiles of the
 *          kind-4 operations: each group's far triangle is cut at multiples
 *          of it, so that only one of the group's launches ends in a partly
 *          filled round of tiles (0: equal parts).  chol_potrf uses two
 *          blocks per CU on all but 16 CUs of the device (480 on a 256-CU
 *          MI355X), or on all of them with 64 CUs or fewer.
 * Returns the number of operations (rows beyond cap are not written), or -1
 * for n < 0, slots < 0 or nb outside 0 .. CHOL_MAX_NB (0 picks 128).
 */
#define CHOL_PLAN_FIELDS 10
int64_t chol_potrf_plan(int64_t n, int64_t nb, int copy, int64_t slots, int64_t *ops, int64_t cap);

/* Diagnostics: the hipError_t code (0 if none so far) of the HIP call whose
 * failure made the most recent call return CHOL_ERR_HIP, process-wide, and
 * HIP's description of it (static string, never NULL). */
int chol_last_hip_error(void);
const char *chol_last_hip_error_string(void);

#ifdef __cplusplus
}
#endif

#endif /* LIBCHOL_H */
