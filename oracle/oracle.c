/*
 * oracle.c -- plain, unblocked, fp64 CPU reference for the Cholesky factor and
 * its reverse-mode adjoint.
 *
 * THIS IS TEST INFRASTRUCTURE, NOT PART OF THE PRODUCT.  Only the test suite,
 * the smoke check and the benchmark's CPU-baseline leg may load it.  It shares
 * no source, header, table or helper with the GPU library, and the GPU library
 * never calls it.
 *
 * Sources (the pages these functions follow):
 *   [jaxmg-potrf]  jaxmg documentation, "Cholesky factorization" (potrf example):
 *                  the factor is the lower-triangular L with A = L L^T for a
 *                  symmetric positive-definite A; no solve is performed; the
 *                  example's validation compares against an expected factor whose
 *                  strict upper triangle is zero.
 *   [warp-1316]    Warp issue #1316, "[REQ] Add adjoint for out-of-place tile
 *                  Cholesky factorization", resolution comment: the adjoint is
 *                  Murray's (2016) symmetric-matrix derivative -- form
 *                  Phi(L^T adj_L), apply two triangular solves against L, and
 *                  accumulate the result into the lower triangle of adj_A.
 *   [warp-1374]    Warp issue #1374, "adj_tile_dot is missing a block-wide
 *                  broadcast of adj_ret", description and repro: the dot product
 *                  y = sum_k a_k b_k and its adjoint a_bar += y_bar * b.
 *
 * Conventions (readings where the pages are silent):
 *   - row-major storage; element (i, j) of a matrix with leading dimension ld
 *     is at p[i * ld + j];
 *   - only the lower triangle (i >= j) of A and of adj_L is read;
 *   - L's strict upper triangle is written as zero;
 *   - Phi(X) = lower triangle of X with the diagonal halved (Murray's Phi; the
 *     pages name Phi without defining it -- the N = 1 case pins it);
 *   - the adjoint written into adj_A is G = Phi(S + S^T) with
 *     S = L^{-T} Phi(L^T tril(adj_L)) L^{-1}: the gradient with respect to the
 *     lower entries the factorisation reads;
 *   - info = 0 on success, else 1 + the first column j whose pivot d fails
 *     d > 0 (NaN fails too).  On failure the factor's columns >= j are left
 *     unspecified.
 *   - arithmetic is IEEE fp64 with no FMA contraction (built with
 *     -ffp-contract=off), sums in ascending index order, correctly rounded
 *     sqrt and division.
 *
 * OpenMP is used only to split independent rows, columns or batch elements
 * over threads; every element is still computed by one plain loop.
 */
#include <complex.h>
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define AT(p, ld, i, j) ((p)[(int64_t)(i) * (ld) + (j)])

/* Forward factor, column by column [jaxmg-potrf]:
 *   d      = A_jj - sum_{k<j} L_jk^2 ;  fail unless d > 0
 *   L_jj   = sqrt(d)
 *   L_ij   = (A_ij - sum_{k<j} L_ik L_jk) / L_jj   for i > j
 * L and A must not overlap. */
int32_t oracle_potrf(int64_t n, const double *A, int64_t lda, double *L, int64_t ldl)
{
    for (int64_t i = 0; i < n; ++i)
        for (int64_t j = i + 1; j < n; ++j)
            AT(L, ldl, i, j) = 0.0;
    for (int64_t j = 0; j < n; ++j) {
        double d = AT(A, lda, j, j);
        for (int64_t k = 0; k < j; ++k)
            d -= AT(L, ldl, j, k) * AT(L, ldl, j, k);
        if (!(d > 0.0))
            return (int32_t)(j + 1);
        const double ljj = sqrt(d);
        AT(L, ldl, j, j) = ljj;
#pragma omp parallel for schedule(static) if (n - j > 512)
        for (int64_t i = j + 1; i < n; ++i) {
            double s = AT(A, lda, i, j);
            for (int64_t k = 0; k < j; ++k)
                s -= AT(L, ldl, i, k) * AT(L, ldl, j, k);
            AT(L, ldl, i, j) = s / ljj;
        }
    }
    return 0;
}

/* Adjoint by the formula of [warp-1316] (Murray's symmetric-matrix derivative):
 *   M = L^T tril(adj_L)              (only its lower triangle is used)
 *   P = Phi(M)
 *   X = L^{-T} P                     (first triangular solve, with L^T)
 *   S = X L^{-1}                     (second triangular solve, with L, from the right)
 *   G = Phi(S + S^T)
 *   lower(adj_A) += G   (accumulate != 0)   or   lower(adj_A) = G   (accumulate == 0)
 * The strict upper triangle of adj_A is not touched.  Returns 0, or -1 if the
 * scratch allocation fails. */
int32_t oracle_potrf_adjoint(int64_t n, const double *L, int64_t ldl,
                             const double *adjL, int64_t ldal,
                             double *adjA, int64_t ldaa, int32_t accumulate)
{
    if (n <= 0)
        return 0;
    const size_t nn = (size_t)n * (size_t)n;
    double *M = (double *)calloc(nn, sizeof(double)); /* becomes P, then X's right-hand side */
    double *X = (double *)calloc(nn, sizeof(double));
    double *S = (double *)calloc(nn, sizeof(double));
    if (!M || !X || !S) {
        free(M); free(X); free(S);
        return -1;
    }

    /* M_ij = sum_{k >= i} L_ki adjL_kj  for i >= j (L_ki = 0 for k < i; adjL read for k >= j only). */
#pragma omp parallel for schedule(dynamic, 16) if (n > 64)
    for (int64_t i = 0; i < n; ++i) {
        double *mrow = M + (size_t)i * n;
        for (int64_t k = i; k < n; ++k) {
            const double lki = AT(L, ldl, k, i);
            for (int64_t j = 0; j <= i; ++j)
                mrow[j] += lki * AT(adjL, ldal, k, j);
        }
    }

    /* P = Phi(M): halve the diagonal; the strict upper triangle of M is already zero. */
    for (int64_t i = 0; i < n; ++i)
        M[(size_t)i * n + i] *= 0.5;

    /* X = L^{-T} P, i.e. L^T X = P, by back substitution over rows:
     *   X_i,: = R_i,: / L_ii ;  R_t,: -= L_it X_i,:  for t < i   (i = n-1 .. 0)
     * R starts as P (held in M).  Columns of the right-hand side are independent:
     * OpenMP splits them into blocks. */
    const int64_t cb = 64;
#pragma omp parallel for schedule(dynamic, 1) if (n > 64)
    for (int64_t c0 = 0; c0 < n; c0 += cb) {
        const int64_t c1 = (c0 + cb < n) ? c0 + cb : n;
        for (int64_t i = n - 1; i >= 0; --i) {
            const double lii = AT(L, ldl, i, i);
            double *ri = M + (size_t)i * n;
            double *xi = X + (size_t)i * n;
            for (int64_t c = c0; c < c1; ++c)
                xi[c] = ri[c] / lii;
            for (int64_t t = 0; t < i; ++t) {
                const double lit = AT(L, ldl, i, t);
                double *rt = M + (size_t)t * n;
                for (int64_t c = c0; c < c1; ++c)
                    rt[c] -= lit * xi[c];
            }
        }
    }

    /* S = X L^{-1}, i.e. S L = X, row by row from the right:
     *   S_rj = R_rj / L_jj ;  R_rk -= S_rj L_jk  for k < j   (j = n-1 .. 0)
     * R starts as X (overwritten in place: X is not needed afterwards). */
#pragma omp parallel for schedule(static) if (n > 64)
    for (int64_t r = 0; r < n; ++r) {
        double *rr = X + (size_t)r * n;
        double *sr = S + (size_t)r * n;
        for (int64_t j = n - 1; j >= 0; --j) {
            const double srj = rr[j] / AT(L, ldl, j, j);
            sr[j] = srj;
            for (int64_t k = 0; k < j; ++k)
                rr[k] -= srj * AT(L, ldl, j, k);
        }
    }

    /* G = Phi(S + S^T):  G_ij = S_ij + S_ji (i > j),  G_ii = S_ii. */
#pragma omp parallel for schedule(static) if (n > 64)
    for (int64_t i = 0; i < n; ++i) {
        for (int64_t j = 0; j <= i; ++j) {
            const double g = (i == j) ? S[(size_t)i * n + i]
                                      : S[(size_t)i * n + j] + S[(size_t)j * n + i];
            if (accumulate)
                AT(adjA, ldaa, i, j) += g;
            else
                AT(adjA, ldaa, i, j) = g;
        }
    }
    free(M); free(X); free(S);
    return 0;
}

/* Second, independent adjoint used only to cross-check the formula above:
 * the reverse sweep of the column-form factorisation.  Forward step j computes
 *   d = sqrt(A_jj - r.r),   c = (A[j+1:, j] - B r) / d,
 * with r = L[j, :j], B = L[j+1:, :j], c = L[j+1:, j].  Walking j from n-1 down
 * to 0 and differentiating those two lines gives, on the running adjoint Abar
 * (which starts as tril(adj_L) and ends as the gradient G):
 *   dbar -= c.cbar / d;  cbar /= d;  rbar -= B^T cbar;  Bbar -= cbar r^T;
 *   rbar -= (dbar / d) r;  dbar /= 2 d.
 * Writes G into the lower triangle of adj_A (accumulate as above). */
int32_t oracle_potrf_adjoint_sweep(int64_t n, const double *L, int64_t ldl,
                                   const double *adjL, int64_t ldal,
                                   double *adjA, int64_t ldaa, int32_t accumulate)
{
    if (n <= 0)
        return 0;
    double *G = (double *)calloc((size_t)n * (size_t)n, sizeof(double));
    if (!G)
        return -1;
    for (int64_t i = 0; i < n; ++i)
        for (int64_t j = 0; j <= i; ++j)
            G[(size_t)i * n + j] = AT(adjL, ldal, i, j);

    for (int64_t j = n - 1; j >= 0; --j) {
        const double d = AT(L, ldl, j, j);
        double dbar = G[(size_t)j * n + j];
        for (int64_t i = j + 1; i < n; ++i)
            dbar -= AT(L, ldl, i, j) * G[(size_t)i * n + j] / d;
        for (int64_t i = j + 1; i < n; ++i)
            G[(size_t)i * n + j] /= d;
        for (int64_t i = j + 1; i < n; ++i) {
            const double cbar = G[(size_t)i * n + j];
            for (int64_t k = 0; k < j; ++k) {
                G[(size_t)j * n + k] -= AT(L, ldl, i, k) * cbar;  /* rbar -= B^T cbar */
                G[(size_t)i * n + k] -= cbar * AT(L, ldl, j, k);  /* Bbar -= cbar r^T */
            }
        }
        for (int64_t k = 0; k < j; ++k)
            G[(size_t)j * n + k] -= (dbar / d) * AT(L, ldl, j, k);
        G[(size_t)j * n + j] = dbar / (2.0 * d);
    }

    for (int64_t i = 0; i < n; ++i)
        for (int64_t j = 0; j <= i; ++j) {
            if (accumulate)
                AT(adjA, ldaa, i, j) += G[(size_t)i * n + j];
            else
                AT(adjA, ldaa, i, j) = G[(size_t)i * n + j];
        }
    free(G);
    return 0;
}

/* Batched forms: the single-matrix functions above applied to each element of a
 * strided batch; batch elements are independent and split over threads. */
void oracle_potrf_batched(int64_t n, int64_t batch,
                          const double *A, int64_t lda, int64_t strideA,
                          double *L, int64_t ldl, int64_t strideL, int32_t *info)
{
#pragma omp parallel for schedule(static) if (batch > 1)
    for (int64_t b = 0; b < batch; ++b) {
        const int32_t r = oracle_potrf(n, A + b * strideA, lda, L + b * strideL, ldl);
        if (info)
            info[b] = r;
    }
}

int32_t oracle_potrf_adjoint_batched(int64_t n, int64_t batch,
                                     const double *L, int64_t ldl, int64_t strideL,
                                     const double *adjL, int64_t ldal, int64_t strideAL,
                                     double *adjA, int64_t ldaa, int64_t strideAA,
                                     int32_t accumulate)
{
    int32_t bad = 0;
#pragma omp parallel for schedule(static) reduction(| : bad) if (batch > 1)
    for (int64_t b = 0; b < batch; ++b)
        bad |= oracle_potrf_adjoint(n, L + b * strideL, ldl, adjL + b * strideAL, ldal,
                                    adjA + b * strideAA, ldaa, accumulate) != 0;
    return bad ? -1 : 0;
}

/* Upper-factor form (uplo = U, the layout a column-major caller's lower
 * factor has in row-major memory): A = U^T U with U upper triangular and
 * positive diagonal, reading only the upper triangle of A.  By uniqueness of
 * the factor, U = L^T for the lower factor L of the same symmetric matrix, so
 * this is the lower factorisation [jaxmg-potrf] applied to A^T (whose lower
 * triangle is A's upper triangle) and written back transposed.  U's strict
 * lower triangle is written as zero.  Returns info as oracle_potrf.  A and U
 * must not overlap. */
int32_t oracle_potrf_upper(int64_t n, const double *A, int64_t lda, double *U, int64_t ldu)
{
    if (n <= 0)
        return 0;
    double *At = (double *)malloc((size_t)n * (size_t)n * sizeof(double));
    double *L = (double *)malloc((size_t)n * (size_t)n * sizeof(double));
    if (!At || !L) {
        free(At); free(L);
        return -1;
    }
    for (int64_t i = 0; i < n; ++i)
        for (int64_t j = 0; j <= i; ++j)
            At[(size_t)i * n + j] = AT(A, lda, j, i);       /* lower of A^T = upper of A */
    const int32_t info = oracle_potrf(n, At, n, L, n);
    for (int64_t i = 0; i < n; ++i)
        for (int64_t j = 0; j < n; ++j)
            AT(U, ldu, i, j) = (j >= i) ? L[(size_t)j * n + i] : 0.0;
    free(At); free(L);
    return info;
}

/* Adjoint of the upper form: with U = L^T and adj_L = adj_U^T, the gradient
 * with respect to A's upper entries is G^T, G the lower-form adjoint
 * [warp-1316] of (L, adj_L).  Only the upper triangles of U and adj_U are
 * read; upper(adj_A) += G^T (accumulate != 0) or = G^T; the strict lower
 * triangle of adj_A is not touched. */
int32_t oracle_potrf_adjoint_upper(int64_t n, const double *U, int64_t ldu,
                                   const double *adjU, int64_t ldau,
                                   double *adjA, int64_t ldaa, int32_t accumulate)
{
    if (n <= 0)
        return 0;
    const size_t nn = (size_t)n * (size_t)n;
    double *L = (double *)calloc(nn, sizeof(double));
    double *aL = (double *)calloc(nn, sizeof(double));
    double *G = (double *)calloc(nn, sizeof(double));
    if (!L || !aL || !G) {
        free(L); free(aL); free(G);
        return -1;
    }
    for (int64_t i = 0; i < n; ++i)
        for (int64_t j = 0; j <= i; ++j) {
            L[(size_t)i * n + j] = AT(U, ldu, j, i);
            aL[(size_t)i * n + j] = AT(adjU, ldau, j, i);
        }
    int32_t rc = oracle_potrf_adjoint(n, L, n, aL, n, G, n, 0);
    if (rc == 0)
        for (int64_t i = 0; i < n; ++i)
            for (int64_t j = i; j < n; ++j) {
                const double g = G[(size_t)j * n + i];
                double *dst = &AT(adjA, ldaa, i, j);
                *dst = accumulate ? *dst + g : g;
            }
    free(L); free(aL); free(G);
    return rc;
}

/* Hermitian complex factor A = L L^H [jaxmg-potrf: the factor of a symmetric
 * or Hermitian positive-definite matrix], column by column, complex128 stored
 * as (re, im) pairs, row-major, leading dimensions in complex elements:
 *   d      = Re(A_jj) - sum_{k<j} |L_jk|^2 ;  fail unless d > 0
 *   L_jj   = sqrt(d)                               (real)
 *   L_ij   = (A_ij - sum_{k<j} L_ik conj(L_jk)) / L_jj   for i > j
 * Only the lower triangle of A is read; the imaginary part of its diagonal is
 * ignored (a Hermitian matrix has a real diagonal).  L's strict upper
 * triangle is written as zero.  info as oracle_potrf. */
#define ZAT(p, ld, i, j) ((p)[(int64_t)(i) * (ld) + (j)])
int32_t oracle_zpotrf(int64_t n, const double complex *A, int64_t lda, double complex *L, int64_t ldl)
{
    for (int64_t i = 0; i < n; ++i)
        for (int64_t j = i + 1; j < n; ++j)
            ZAT(L, ldl, i, j) = 0.0;
    for (int64_t j = 0; j < n; ++j) {
        double d = creal(ZAT(A, lda, j, j));
        for (int64_t k = 0; k < j; ++k) {
            const double complex l = ZAT(L, ldl, j, k);
            d -= creal(l) * creal(l) + cimag(l) * cimag(l);
        }
        if (!(d > 0.0))
            return (int32_t)(j + 1);
        const double djj = sqrt(d);
        ZAT(L, ldl, j, j) = djj;
#pragma omp parallel for schedule(static) if (n - j > 256)
        for (int64_t i = j + 1; i < n; ++i) {
            double complex s = ZAT(A, lda, i, j);
            for (int64_t k = 0; k < j; ++k)
                s -= ZAT(L, ldl, i, k) * conj(ZAT(L, ldl, j, k));
            ZAT(L, ldl, i, j) = CMPLX(creal(s) / djj, cimag(s) / djj);
        }
    }
    return 0;
}

/* Its adjoint: the formula of [warp-1316] with conjugate transposes.  With
 * gradients taken as adj_X = dloss/dRe(X) + i dloss/dIm(X):
 *   M = L^H tril(adj_L)                  (lower triangle used)
 *   P = Phi(M)      Phi: lower triangle, diagonal -> Re(diagonal) / 2
 *   X = L^{-H} P    (back substitution with L^H)
 *   S = X L^{-1}    (solve with L from the right)
 *   G = Phi(S + S^H):  G_ij = S_ij + conj(S_ji) (i > j),  G_ii = Re(S_ii)
 *   lower(adj_A) += G (accumulate != 0) or = G.
 * G is the gradient with respect to the entries the factor reads: Re and Im
 * of A_ij below the diagonal, and the real diagonal. */
int32_t oracle_zpotrf_adjoint(int64_t n, const double complex *L, int64_t ldl,
                              const double complex *adjL, int64_t ldal,
                              double complex *adjA, int64_t ldaa, int32_t accumulate)
{
    if (n <= 0)
        return 0;
    const size_t nn = (size_t)n * (size_t)n;
    double complex *M = (double complex *)calloc(nn, sizeof(double complex));
    double complex *X = (double complex *)calloc(nn, sizeof(double complex));
    double complex *S = (double complex *)calloc(nn, sizeof(double complex));
    if (!M || !X || !S) {
        free(M); free(X); free(S);
        return -1;
    }
    /* M_ij = sum_{k >= i} conj(L_ki) adjL_kj for i >= j */
#pragma omp parallel for schedule(dynamic, 16) if (n > 64)
    for (int64_t i = 0; i < n; ++i)
        for (int64_t k = i; k < n; ++k) {
            const double complex lki = conj(ZAT(L, ldl, k, i));
            for (int64_t j = 0; j <= i; ++j)
                M[(size_t)i * n + j] += lki * ZAT(adjL, ldal, k, j);
        }
    for (int64_t i = 0; i < n; ++i)
        M[(size_t)i * n + i] = 0.5 * creal(M[(size_t)i * n + i]);
    /* X = L^{-H} P:  X_i = (P_i - sum_{t > i} conj(L_ti) X_t) / L_ii, i = n-1 .. 0 */
    for (int64_t i = n - 1; i >= 0; --i) {
        const double lii = creal(ZAT(L, ldl, i, i));
        for (int64_t c = 0; c < n; ++c) {
            double complex s = M[(size_t)i * n + c];
            for (int64_t t = i + 1; t < n; ++t)
                s -= conj(ZAT(L, ldl, t, i)) * X[(size_t)t * n + c];
            X[(size_t)i * n + c] = CMPLX(creal(s) / lii, cimag(s) / lii);
        }
    }
    /* S = X L^{-1}:  S_rj = (X_rj - sum_{k > j} S_rk L_kj) / L_jj, j = n-1 .. 0 */
#pragma omp parallel for schedule(static) if (n > 64)
    for (int64_t r = 0; r < n; ++r)
        for (int64_t j = n - 1; j >= 0; --j) {
            double complex s = X[(size_t)r * n + j];
            for (int64_t k = j + 1; k < n; ++k)
                s -= S[(size_t)r * n + k] * ZAT(L, ldl, k, j);
            const double ljj = creal(ZAT(L, ldl, j, j));
            S[(size_t)r * n + j] = CMPLX(creal(s) / ljj, cimag(s) / ljj);
        }
    for (int64_t i = 0; i < n; ++i)
        for (int64_t j = 0; j <= i; ++j) {
            const double complex g = (i == j) ? (double complex)creal(S[(size_t)i * n + i])
                                              : S[(size_t)i * n + j] + conj(S[(size_t)j * n + i]);
            double complex *dst = &ZAT(adjA, ldaa, i, j);
            *dst = accumulate ? *dst + g : g;
        }
    free(M); free(X); free(S);
    return 0;
}

/* Solve with the factor: X = A^{-1} B for A = L L^T, B and X n x nrhs
 * (row-major, leading dimensions ldb, ldx).  The factor is returned without a
 * solve [jaxmg-potrf]; this is the solve it is computed for, written as the
 * two triangular solves against L that [warp-1316] names for the adjoint:
 *   L Y = B     forward substitution:  Y_i = (B_i - sum_{k<i} L_ik Y_k) / L_ii
 *   L^T X = Y   back substitution:     X_i = (Y_i - sum_{k>i} L_ki X_k) / L_ii
 * (rows i; each right-hand-side column on its own).  Only the lower triangle of
 * L is read.  X may be B itself (then B is overwritten); otherwise they must
 * not overlap. */
void oracle_potrs(int64_t n, int64_t nrhs, const double *L, int64_t ldl,
                  const double *B, int64_t ldb, double *X, int64_t ldx)
{
    if (n <= 0 || nrhs <= 0)
        return;
    if (X != B)
        for (int64_t i = 0; i < n; ++i)
            for (int64_t c = 0; c < nrhs; ++c)
                AT(X, ldx, i, c) = AT(B, ldb, i, c);
#pragma omp parallel for schedule(static) if (nrhs > 1 && n * nrhs > 4096)
    for (int64_t c = 0; c < nrhs; ++c) {
        for (int64_t i = 0; i < n; ++i) {
            double s = AT(X, ldx, i, c);
            for (int64_t k = 0; k < i; ++k)
                s -= AT(L, ldl, i, k) * AT(X, ldx, k, c);
            AT(X, ldx, i, c) = s / AT(L, ldl, i, i);
        }
        for (int64_t i = n - 1; i >= 0; --i) {
            double s = AT(X, ldx, i, c);
            for (int64_t k = i + 1; k < n; ++k)
                s -= AT(L, ldl, k, i) * AT(X, ldx, k, c);
            AT(X, ldx, i, c) = s / AT(L, ldl, i, i);
        }
    }
}

/* Adjoint of X = (L L^T)^{-1} B, given adj_X (reverse mode).  With A = L L^T,
 * dX = -A^{-1} dA X and dA = dL L^T + L dL^T, so for any adj_X
 *   <adj_X, dX> = <adj_B, dB> - <(adj_B X^T + X adj_B^T) L, dL>,
 *   adj_B = A^{-1} adj_X                     (the same two triangular solves)
 * and the gradient with respect to the lower entries of L is
 *   adj_L = -tril((adj_B X^T + X adj_B^T) L).
 * adj_B is written (it may be adj_X itself); lower(adj_L) += adj_L
 * (accumulate != 0) or = adj_L (accumulate == 0); the strict upper triangle of
 * adj_L is not touched.  Returns 0, or -1 if the scratch allocation fails. */
int32_t oracle_potrs_adjoint(int64_t n, int64_t nrhs, const double *L, int64_t ldl,
                             const double *X, int64_t ldx, const double *adjX, int64_t ldax,
                             double *adjB, int64_t ldab, double *adjL, int64_t ldal,
                             int32_t accumulate)
{
    if (n <= 0)
        return 0;
    oracle_potrs(n, nrhs, L, ldl, adjX, ldax, adjB, ldab);
    double *W = (double *)calloc((size_t)n * (size_t)n, sizeof(double));
    if (!W)
        return -1;
    /* W = adj_B X^T + X adj_B^T */
#pragma omp parallel for schedule(static) if (n > 64)
    for (int64_t i = 0; i < n; ++i)
        for (int64_t k = 0; k < n; ++k) {
            double w = 0.0;
            for (int64_t c = 0; c < nrhs; ++c)
                w += AT(adjB, ldab, i, c) * AT(X, ldx, k, c) + AT(X, ldx, i, c) * AT(adjB, ldab, k, c);
            W[(size_t)i * n + k] = w;
        }
    /* adj_L_ij = -sum_{k >= j} W_ik L_kj  for i >= j */
#pragma omp parallel for schedule(static) if (n > 64)
    for (int64_t i = 0; i < n; ++i)
        for (int64_t j = 0; j <= i; ++j) {
            double g = 0.0;
            for (int64_t k = j; k < n; ++k)
                g += W[(size_t)i * n + k] * AT(L, ldl, k, j);
            if (accumulate)
                AT(adjL, ldal, i, j) -= g;
            else
                AT(adjL, ldal, i, j) = -g;
        }
    free(W);
    return 0;
}

/* Dot product and its adjoint [warp-1374]:
 *   y = sum_k a_k b_k ;   a_bar_k += y_bar b_k ;   b_bar_k += y_bar a_k. */
double oracle_dot(int64_t n, const double *a, const double *b)
{
    double y = 0.0;
    for (int64_t k = 0; k < n; ++k)
        y += a[k] * b[k];
    return y;
}

void oracle_dot_adjoint(int64_t n, const double *a, const double *b, double ybar,
                        double *abar, double *bbar)
{
    for (int64_t k = 0; k < n; ++k) {
        abar[k] += ybar * b[k];
        bbar[k] += ybar * a[k];
    }
}

/* Sum and its adjoint (the tile_sum reduction [warp-1374] names as the model
 * for broadcasting the upstream gradient):
 *   y = sum_k a_k ;   a_bar_k += y_bar. */
double oracle_sum(int64_t n, const double *a)
{
    double y = 0.0;
    for (int64_t k = 0; k < n; ++k)
        y += a[k];
    return y;
}

void oracle_sum_adjoint(int64_t n, double ybar, double *abar)
{
    for (int64_t k = 0; k < n; ++k)
        abar[k] += ybar;
}

int32_t oracle_max_threads(void)
{
#ifdef _OPENMP
    extern int omp_get_max_threads(void);
    return (int32_t)omp_get_max_threads();
#else
    return 1;
#endif
}
