// Blocked family: right-looking tiled factorisation for large n and its
// reverse-order adjoint.
//
// What is computed (see the page citations in small.hip and libchol.h):
// the factor of jaxmg's "Cholesky factorization" page with tile size T_A
// (here nb), and Murray's adjoint from Warp issue #1316.  The tiled forms
// below are the plain block versions of those definitions.
//
// Forward, with W := lower(A) and tile columns k = 0 .. K-1
// (k0 = k*nb, kb = tile width, r0 = k0 + kb, m = n - r0 rows below):
//   L_kk = chol(W_kk)                       diagonal tile, registers + LDS
//   L_ik = W_ik L_kk^{-T}        (i > k)    panel solve: product with the
//                                           explicit inverse on the matrix cores
//   W_ij -= L_ik L_jk^T    (i >= j > k)     lower trailing update, matrix cores
// Reverse, with Wb := tril(adj_L) and k = K-1 .. 0:
//   Wb_ik -= sum_{j>k} Sym(Wb)_ij L_jk      adjoint of the trailing update;
//                                           Sym(Wb) = Wb + Wb^T with Wb lower
//                                           (diagonal doubled)
//   X_ik = Wb_ik L_kk^{-1};  Wb_ik := X_ik  adjoint of the panel solve
//   Wb_kk -= tril(sum_{i>k} X_ik^T L_ik)
//   Wb_kk := adjoint of chol on the tile   the tile formula (small.hip), applied
//                                           recursively on 64-wide sub-tiles
// and at the end Wb holds G.
#include <algorithm>
#include <cmath>

#include "common.hpp"
#include "gemm.hpp"
#include "profile.hpp"

namespace chol {

template <typename T>
chol_status diag_potrf(int n, T *W, int64_t ld, int32_t *info, int info_mode, int64_t info_base,
                       hipStream_t st);
template <typename T>
chol_status small_potrf_adjoint(int n, int64_t batch, const T *L, int64_t ldl, int64_t sL,
                                const T *adjL, int64_t ldal, int64_t sAL, T *adjA, int64_t ldaa,
                                int64_t sAA, int accumulate, hipStream_t st);

// ------------------------------------------------------------ elementwise ----
enum { TRI_COPY_LOWER = 0, TRI_ZERO_UPPER = 1, TRI_ADD_LOWER = 2 };

// 32 x 32 element tiles; a block covers one tile with 256 threads.
template <typename T, int MODE>
__global__ void __launch_bounds__(256)
k_tri(int64_t n, const T *src, int64_t lds, T *dst, int64_t ldd)
{
    const int64_t i0 = (int64_t)blockIdx.y * 32, j0 = (int64_t)blockIdx.x * 32;
    if (MODE == TRI_ZERO_UPPER ? (j0 + 31 <= i0) : (j0 > i0 + 31))
        return;
    const int tj = threadIdx.x % 32, ti = threadIdx.x / 32;
    for (int r = ti; r < 32; r += 8) {
        const int64_t i = i0 + r, j = j0 + tj;
        if (i >= n || j >= n)
            continue;
        if (MODE == TRI_COPY_LOWER) {
            if (j <= i)
                dst[i * ldd + j] = src[i * lds + j];
        } else if (MODE == TRI_ZERO_UPPER) {
            if (j > i)
                dst[i * ldd + j] = T(0);
        } else {
            if (j <= i)
                dst[i * ldd + j] += src[i * lds + j];
        }
    }
}

template <typename T, int MODE>
static chol_status tri_op(int64_t n, const T *src, int64_t lds, T *dst, int64_t ldd, hipStream_t st)
{
    const double tri = (double)n * (n + 1) / 2, es = (double)sizeof(T);
    const double bytes = MODE == TRI_COPY_LOWER ? 2 * tri * es
                       : MODE == TRI_ZERO_UPPER ? ((double)n * n - tri) * es : 3 * tri * es;
    prof::Scope ps(CHOL_K_ELEMENTWISE, st, bytes);
    const unsigned t = (unsigned)((n + 31) / 32);
    hipLaunchKernelGGL((k_tri<T, MODE>), dim3(t, t), dim3(256), 0, st, n, src, lds, dst, ldd);
    CHOL_LAUNCH_CHECK();
    return CHOL_OK;
}

// ------------------------------------------------------ triangular inverse ----
// Inverse X = L^{-1} of lower-triangular kb x kb tiles (kb <= 128) placed on
// the diagonal of W every `step` rows: tile t starts at W + t*step*(ld+1).
// One 256-thread block per tile; L in LDS, X spread over a 16 x 16 lane grid
// (8 x 8 entries per lane).  Row i of X: X_i = R_i / L_ii, then
// R_t -= L_ti X_i for t > i (R starts as the identity).
//   out_mode 0: strict lower of X written transposed into the tile's strict
//               upper triangle in W (the factor's upper triangle is free
//               scratch until it is zeroed at the end).
//   out_mode 1: X (lower) written to ws + t*ws_stride with leading dim ws_ld.
template <typename T>
__global__ void __launch_bounds__(256)
k_trinv(int64_t n_total, int nb, int64_t tile0, int64_t step, T *W, int64_t ld, int out_mode, T *ws,
        int64_t ws_stride, int64_t ws_ld)
{
    constexpr int G = 16, E = 8, NP = 128, LP = NP + 1;
    __shared__ T ls[NP * LP];
    __shared__ T bc[2 * NP];
    const int tid = threadIdx.x, lr = tid / G, lc = tid % G;
    const int64_t k0 = tile0 + (int64_t)blockIdx.x * step;
    const int kb = (int)std::min<int64_t>(nb, n_total - k0);
    const T *Lkk = W + k0 * ld + k0;
    for (int idx = tid; idx < NP * NP; idx += 256) {
        const int i = idx / NP, k = idx % NP;
        T v = (i == k) ? T(1) : T(0);
        if (i < kb && k <= i)
            v = Lkk[(int64_t)i * ld + k];
        ls[i * LP + k] = v;
    }
    T x[E][E];
#pragma unroll
    for (int a = 0; a < E; ++a)
#pragma unroll
        for (int b = 0; b <= a; ++b)
            x[a][b] = (lr + G * a == lc + G * b) ? T(1) : T(0);
    __syncthreads();

#pragma unroll
    for (int ib = 0; ib < E; ++ib) {
#pragma unroll 1
        for (int ir = 0; ir < G; ++ir) {
            const int i = ib * G + ir;
            T *cb = bc + (i & 1) * NP;
            if (lr == ir) {
                const T rinv = drcp(ls[i * LP + i]);
#pragma unroll
                for (int b = 0; b <= ib; ++b) {
                    x[ib][b] *= rinv;
                    cb[lc * E + b] = x[ib][b];
                }
            }
            __syncthreads();
            T w[E];
#pragma unroll
            for (int b = 0; b <= ib; ++b)
                w[b] = cb[lc * E + b];
#pragma unroll
            for (int a = ib; a < E; ++a) {
                T u = ls[(lr + G * a) * LP + i];   // L_ti, t = lr + G a
                if (a == ib && lr <= ir)
                    u = T(0);
#pragma unroll
                for (int b = 0; b <= ib; ++b)
                    x[a][b] -= u * w[b];
            }
        }
    }

#pragma unroll
    for (int a = 0; a < E; ++a)
#pragma unroll
        for (int b = 0; b <= a; ++b) {
            const int i = lr + G * a, j = lc + G * b;
            if (i >= kb || j > i)
                continue;
            if (out_mode == 0) {
                if (i > j)
                    W[(k0 + j) * ld + k0 + i] = x[a][b];
            } else {
                ws[(int64_t)blockIdx.x * ws_stride + (int64_t)i * ws_ld + j] = x[a][b];
            }
        }
}

// C_lower(n x n) -= sum_s part[s] (lower entries only)
template <typename T>
__global__ void __launch_bounds__(256)
k_splitk_reduce_lower(int n, int splits, const T *part, T *c, int64_t ldc)
{
    const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (idx >= (int64_t)n * n)
        return;
    const int r = (int)(idx / n), col = (int)(idx % n);
    if (col > r)
        return;
    T s = T(0);
    for (int q = 0; q < splits; ++q)
        s += part[(int64_t)q * n * n + idx];
    c[(int64_t)r * ldc + col] -= s;
}

// C(M x N) -= sum_s part[s] (all entries), part row-major M x N per split
template <typename T>
__global__ void __launch_bounds__(256)
k_splitk_reduce(int M, int N, int splits, const T *part, T *c, int64_t ldc)
{
    const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
    const int64_t tot = (int64_t)M * N;
    if (idx >= tot)
        return;
    const int r = (int)(idx / N), col = (int)(idx % N);
    T s = T(0);
    for (int q = 0; q < splits; ++q)
        s += part[(int64_t)q * tot + idx];
    c[(int64_t)r * ldc + col] -= s;
}

// Split of a long contraction so that about two blocks per CU are busy.
static inline int split_count(int64_t tiles, int64_t K, int max_splits)
{
    int s = (int)std::min<int64_t>(max_splits, std::max<int64_t>(1, (512 + tiles - 1) / tiles));
    s = (int)std::min<int64_t>(s, std::max<int64_t>(1, K / 256));
    return s;
}
static inline int split_chunk(int64_t K, int splits)
{
    int c = (int)((K + splits - 1) / splits);
    return (c + 15) / 16 * 16;
}

// ------------------------------------------------------------- forward ----
template <typename T>
chol_status blocked_potrf(int64_t n, const T *A, int64_t lda, T *L, int64_t ldl, int32_t *info, int nb,
                          hipStream_t st)
{
    chol_status s;
    if (A != L) {
        if ((s = tri_op<T, TRI_COPY_LOWER>(n, A, lda, L, ldl, st)) != CHOL_OK)
            return s;
    }
    const int64_t K = (n + nb - 1) / nb;
    for (int64_t k = 0; k < K; ++k) {
        const int64_t k0 = k * nb;
        const int kb = (int)std::min<int64_t>(nb, n - k0);
        const int64_t r0 = k0 + kb, m = n - r0;
        T *Wkk = L + k0 * ldl + k0;
        const double kb3 = (double)kb * kb * kb;
        {
            prof::Scope ps(CHOL_K_DIAG_FACTOR, st, kb3 / 3);
            if ((s = diag_potrf<T>(kb, Wkk, ldl, info, k == 0 ? 1 : 2, k0, st)) != CHOL_OK)
                return s;
        }
        if (m == 0)
            break;
        // inverse of L_kk, transposed into the tile's strict upper triangle
        {
            prof::Scope ps(CHOL_K_DIAG_INVERSE, st, kb3 / 3);
            hipLaunchKernelGGL((k_trinv<T>), dim3(1), dim3(256), 0, st, n, nb, k0, (int64_t)nb, L, ldl, 0,
                               (T *)nullptr, (int64_t)0, (int64_t)0);
            CHOL_LAUNCH_CHECK();
        }
        // panel: L_ik = W_ik * Linv^T  (in place; one block spans the full panel width)
        {
            GemmArgs<T> p{};
            p.M = (int)m; p.N = kb; p.K = kb;
            p.a = L + r0 * ldl + k0; p.lda = ldl;
            p.b = Wkk; p.ldb = ldl;
            p.c = L + r0 * ldl + k0; p.ldc = ldl;
            prof::Scope ps(CHOL_K_PANEL_SOLVE, st, (double)m * kb * kb);
            if ((s = gemm<T, OP_MK, OP_KM_INVT, C_STORE>(p, 1, st)) != CHOL_OK)
                return s;
        }
        // trailing: W22 lower -= P P^T
        {
            GemmArgs<T> p{};
            p.M = (int)m; p.N = (int)m; p.K = kb;
            p.a = L + r0 * ldl + k0; p.lda = ldl;
            p.b = L + r0 * ldl + k0; p.ldb = ldl;
            p.c = L + r0 * ldl + r0; p.ldc = ldl;
            p.tri = 1;
            prof::Scope ps(CHOL_K_TRAILING_UPDATE, st, (double)m * (m + 1) * kb);
            if ((s = gemm<T, OP_MK, OP_MK, C_SUB_LOWER>(p, 1, st)) != CHOL_OK)
                return s;
        }
    }
    return tri_op<T, TRI_ZERO_UPPER>(n, nullptr, 0, L, ldl, st);
}

// ------------------------------------------------------------- adjoint ----
// Workspace layout (bytes, each part 256-aligned):
//   [Wb : n*n]  (absent when the gradient is formed directly in adj_A)
//   [inv: K * nb * nb]   inverses of the diagonal tiles of L
//   [part: SPLITS * nb * nb]  split-K partial products
static inline size_t align256(size_t x) { return (x + 255) & ~size_t(255); }
static const int ADJ_SPLIT_MAX = 64;     // splits of the tile-sized product Wb_kk -= tril(X^T L)
static const int R1_SPLIT_MAX = 8;       // splits of the panel product Wb_panel -= Sym(Wb22) L

size_t blocked_adjoint_workspace(int64_t n, int nb, size_t esize, bool need_wb)
{
    const int64_t K = (n + nb - 1) / nb;
    size_t s = 0;
    if (need_wb)
        s += align256((size_t)n * n * esize);
    s += align256((size_t)K * nb * nb * esize);
    s += align256(std::max((size_t)ADJ_SPLIT_MAX * nb * nb, (size_t)R1_SPLIT_MAX * n * nb) * esize);
    return s;
}

// Adjoint of chol on one kb x kb diagonal tile, in place on Wb (lower):
// the blocked reverse steps again with 64-wide sub-tiles, the 64-edge tile
// kernel at the leaves.  inv holds L^{-1} of this tile (its diagonal
// sub-blocks are the sub-tiles' inverses).
template <typename T>
static chol_status diag_adjoint(int kb, const T *L, int64_t ldl, T *Wb, int64_t ldw, const T *inv,
                                int64_t ldi, hipStream_t st)
{
    if (kb <= 64)
        return small_potrf_adjoint<T>(kb, 1, L, ldl, 0, Wb, ldw, 0, Wb, ldw, 0, 0, st);
    chol_status s;
    const int h = 64, m = kb - h;
    // lower sub-tile first (reverse order)
    if ((s = diag_adjoint<T>(m, L + (int64_t)h * ldl + h, ldl, Wb + (int64_t)h * ldw + h, ldw,
                             inv + (int64_t)h * ldi + h, ldi, st)) != CHOL_OK)
        return s;
    GemmArgs<T> p{};
    // Wb10 -= Sym(Wb11) L10
    p.M = m; p.N = h; p.K = m;
    p.a = Wb + (int64_t)h * ldw + h; p.lda = ldw;
    p.b = L + (int64_t)h * ldl; p.ldb = ldl;
    p.c = Wb + (int64_t)h * ldw; p.ldc = ldw;
    if ((s = gemm<T, OP_SYM, OP_KM, C_SUB>(p, 1, st)) != CHOL_OK)
        return s;
    // X = Wb10 L00^{-1}  (in place: one block spans the full width)
    p = GemmArgs<T>{};
    p.M = m; p.N = h; p.K = h;
    p.a = Wb + (int64_t)h * ldw; p.lda = ldw;
    p.b = inv; p.ldb = ldi;
    p.c = Wb + (int64_t)h * ldw; p.ldc = ldw;
    if ((s = gemm<T, OP_MK, OP_KM_LOWER, C_STORE>(p, 1, st)) != CHOL_OK)
        return s;
    // Wb00 -= tril(X^T L10)
    p = GemmArgs<T>{};
    p.M = h; p.N = h; p.K = m;
    p.a = Wb + (int64_t)h * ldw; p.lda = ldw;
    p.b = L + (int64_t)h * ldl; p.ldb = ldl;
    p.c = Wb; p.ldc = ldw;
    if ((s = gemm<T, OP_KM, OP_KM, C_SUB_LOWER>(p, 1, st)) != CHOL_OK)
        return s;
    return diag_adjoint<T>(h, L, ldl, Wb, ldw, inv, ldi, st);
}

template <typename T>
chol_status blocked_adjoint(int64_t n, const T *L, int64_t ldl, const T *adjL, int64_t ldal, T *adjA,
                            int64_t ldaa, int accumulate, int nb, void *ws, hipStream_t st)
{
    chol_status s;
    const int64_t K = (n + nb - 1) / nb;
    const bool need_wb = accumulate != 0;
    char *w = (char *)ws;
    T *Wb;
    int64_t ldw;
    if (need_wb) {
        Wb = (T *)w;
        ldw = n;
        w += align256((size_t)n * n * sizeof(T));
    } else {
        Wb = adjA;
        ldw = ldaa;
    }
    T *inv = (T *)w;
    w += align256((size_t)K * nb * nb * sizeof(T));
    T *part = (T *)w;

    if ((const T *)Wb != adjL) {
        if ((s = tri_op<T, TRI_COPY_LOWER>(n, adjL, ldal, Wb, ldw, st)) != CHOL_OK)
            return s;
    }
    // inverses of every diagonal tile, all at once
    {
        prof::Scope ps(CHOL_K_DIAG_INVERSE, st, (double)K * nb * nb * nb / 3);
        hipLaunchKernelGGL((k_trinv<T>), dim3((unsigned)K), dim3(256), 0, st, n, nb, (int64_t)0, (int64_t)nb,
                           const_cast<T *>(L), ldl, 1, inv, (int64_t)nb * nb, (int64_t)nb);
        CHOL_LAUNCH_CHECK();
    }

    for (int64_t k = K - 1; k >= 0; --k) {
        const int64_t k0 = k * nb;
        const int kb = (int)std::min<int64_t>(nb, n - k0);
        const int64_t r0 = k0 + kb, m = n - r0;
        const T *Lkk = L + k0 * ldl + k0;
        T *Wkk = Wb + k0 * ldw + k0;
        const T *invk = inv + k * nb * nb;
        if (m > 0) {
            GemmArgs<T> p{};
            // R1: Wb_panel -= Sym(Wb22) L_panel, the contraction over m split
            // into partial products reduced in a fixed order
            p.M = (int)m; p.N = kb; p.K = (int)m;
            p.a = Wb + r0 * ldw + r0; p.lda = ldw;
            p.b = L + r0 * ldl + k0; p.ldb = ldl;
            p.c = Wb + r0 * ldw + k0; p.ldc = ldw;
            {
                prof::Scope ps(CHOL_K_ADJ_TRAILING, st, 2.0 * m * m * kb);
                const int64_t tiles = ((m + 127) / 128) * ((kb + 127) / 128);
                const int splits = split_count(tiles, m, R1_SPLIT_MAX);
                p.kchunk = split_chunk(m, splits);
                const int used = (int)((m + p.kchunk - 1) / p.kchunk);
                p.part = part;
                if ((s = gemm<T, OP_SYM, OP_KM, C_PARTIAL>(p, used, st)) != CHOL_OK)
                    return s;
                const int64_t tot = m * kb;
                hipLaunchKernelGGL((k_splitk_reduce<T>), dim3((unsigned)((tot + 255) / 256)), dim3(256), 0, st,
                                   (int)m, kb, used, (const T *)part, p.c, ldw);
                CHOL_LAUNCH_CHECK();
            }
            // R2a: X = Wb_panel L_kk^{-1} (in place, full panel width per block)
            p = GemmArgs<T>{};
            p.M = (int)m; p.N = kb; p.K = kb;
            p.a = Wb + r0 * ldw + k0; p.lda = ldw;
            p.b = invk; p.ldb = nb;
            p.c = Wb + r0 * ldw + k0; p.ldc = ldw;
            {
                prof::Scope ps(CHOL_K_ADJ_PANEL, st, (double)m * kb * kb);
                if ((s = gemm<T, OP_MK, OP_KM_LOWER, C_STORE>(p, 1, st)) != CHOL_OK)
                    return s;
            }
            // R2b: Wb_kk -= tril(X^T L_panel), split over the m rows
            p = GemmArgs<T>{};
            p.M = kb; p.N = kb; p.K = (int)m;
            p.a = Wb + r0 * ldw + k0; p.lda = ldw;
            p.b = L + r0 * ldl + k0; p.ldb = ldl;
            prof::Scope ps(CHOL_K_ADJ_DIAG_UPDATE, st, (double)m * kb * (kb + 1));
            int splits = (int)std::min<int64_t>(ADJ_SPLIT_MAX, (m + 511) / 512);
            if (splits <= 1) {
                p.c = Wkk; p.ldc = ldw;
                if ((s = gemm<T, OP_KM, OP_KM, C_SUB_LOWER>(p, 1, st)) != CHOL_OK)
                    return s;
            } else {
                int chunk = (int)((m + splits - 1) / splits);
                chunk = (chunk + 15) / 16 * 16;
                splits = (int)((m + chunk - 1) / chunk);
                p.kchunk = chunk;
                p.part = part;
                if ((s = gemm<T, OP_KM, OP_KM, C_PARTIAL>(p, splits, st)) != CHOL_OK)
                    return s;
                const int64_t tot = (int64_t)kb * kb;
                hipLaunchKernelGGL((k_splitk_reduce_lower<T>), dim3((unsigned)((tot + 255) / 256)), dim3(256),
                                   0, st, kb, splits, (const T *)part, Wkk, ldw);
                CHOL_LAUNCH_CHECK();
            }
        }
        // R3: the tile adjoint on the diagonal
        {
            prof::Scope ps(CHOL_K_ADJ_DIAG, st, 2.0 * kb * kb * kb / 3);
            if ((s = diag_adjoint<T>(kb, Lkk, ldl, Wkk, ldw, invk, nb, st)) != CHOL_OK)
                return s;
        }
    }
    if (need_wb)
        return tri_op<T, TRI_ADD_LOWER>(n, Wb, ldw, adjA, ldaa, st);
    return CHOL_OK;
}

#define CHOL_INST(T)                                                                                     \
    template chol_status blocked_potrf<T>(int64_t, const T *, int64_t, T *, int64_t, int32_t *, int,     \
                                          hipStream_t);                                                  \
    template chol_status blocked_adjoint<T>(int64_t, const T *, int64_t, const T *, int64_t, T *, int64_t, \
                                            int, int, void *, hipStream_t);
CHOL_INST(float)
CHOL_INST(double)
#undef CHOL_INST

} // namespace chol
