// Small-tile family: one n <= 64 matrix (or a diagonal tile of the blocked
// path, up to 128) per group of G*G lanes, held in registers.
//
// What is computed:
//  * factor   -- jaxmg documentation, "Cholesky factorization": the lower
//                factor L of A = L L^T, strict upper triangle written as zero.
//                Warp issue #1316 (resolution comment) shows the same
//                load -> tile factor -> store shape with one tile per block.
//  * adjoint  -- Warp issue #1316, resolution comment: Murray's
//                symmetric-matrix derivative.  With M = L^T tril(adj_L),
//                P = Phi(M), the adjoint is G = Phi(S + S^T) with
//                S = L^{-T} P L^{-1}.  Because S + S^T = L^{-T} (P + P^T) L^{-1},
//                the kernel forms Psi = P + P^T (M's lower part mirrored; its
//                diagonal keeps M_ii) and runs the two triangular solves on Psi:
//                V = Psi L^{-1} (full), then Z = L^{-T} V, of which only the lower
//                triangle is needed (it depends only on V's lower triangle).
//                G = Phi(Z) is added to (or stored into) the lower triangle of
//                adj_A.
//  * broadcast rule -- Warp issue #1374 ("adj_tile_dot is missing a block-wide
//                broadcast of adj_ret"): a value produced or received by one
//                lane (a pivot, a solved entry, an upstream gradient) is
//                published through LDS and read back by every lane that needs
//                it before anyone uses it.
//
// Data layout.  A matrix padded to NP = G*E (padding rows/columns act as the
// identity, so the padded factor and adjoint contain the real ones) is spread
// cyclically over a G x G lane grid: lane (lr, lc) owns entries
// (lr + G*a, lc + G*b), a, b in [0, E).  Every step of the column loops then
// retires the same number of entries on every lane, and whole blocks of
// (a, b) fall out of the trailing work at compile time.  Global memory is read
// and written row-contiguously through an LDS staging tile; per-step
// broadcasts (a column of the trailing matrix, a solved row or column) go
// through a small double-buffered LDS vector.
#include "common.hpp"

namespace chol {

template <int G_, int E_> struct TileShape {
    static constexpr int G = G_;
    static constexpr int E = E_;
    static constexpr int NP = G * E;                      // padded edge
    static constexpr int LPM = G * G;                     // lanes per matrix
    static constexpr int THREADS = LPM < 64 ? 64 : LPM;   // one wavefront at least
    static constexpr int MPB = THREADS / LPM;             // matrices per block
    static constexpr int LDP = NP + G;                    // natural-layout LDS pitch
    static constexpr int MSTRIDE = NP * LDP + 16;         // per-matrix LDS region
};

// Position of column c inside a "permuted" LDS row: the E entries that lane
// column lc needs (columns lc, lc+G, ...) sit contiguously at lc*E.
template <int G, int E> __device__ __forceinline__ int perm_col(int c) { return (c % G) * E + c / G; }

// info_mode: 0 -> info[mat] = first failing column + 1 (or 0);
//            1 -> info[0] = (fail ? info_base + fail : 0)            (first tile of a blocked call)
//            2 -> if fail and info[0] == 0: info[0] = info_base + fail (later tiles)
__device__ __forceinline__ void write_info(int32_t *info, int64_t mat, int fail, int mode, int64_t base)
{
    if (!info)
        return;
    if (mode == 0)
        info[mat] = fail;
    else if (mode == 1)
        info[0] = fail ? (int32_t)(base + fail) : 0;
    else if (fail && info[0] == 0)
        info[0] = (int32_t)(base + fail);
}

// ------------------------------------------------------------------------
// Factor: right-looking column loop on register-resident tiles.
// A and L may be the same buffer (in place); each block reads all of its
// matrices before it writes any.
// ------------------------------------------------------------------------
template <typename T, int G, int E>
__global__ void __launch_bounds__((TileShape<G, E>::THREADS))
k_potrf_tile(int n, int64_t batch, const T *A, int64_t lda, int64_t sA,
             T *L, int64_t ldl, int64_t sL, int32_t *info, int info_mode, int64_t info_base)
{
    typedef TileShape<G, E> S;
    constexpr int NP = S::NP, LDP = S::LDP, MSTRIDE = S::MSTRIDE, MPB = S::MPB, THREADS = S::THREADS;
    __shared__ T stage[MPB * MSTRIDE];
    __shared__ T colbuf[2 * MPB * NP];

    const int tid = threadIdx.x;
    const int g = tid / S::LPM;
    const int lr = (tid % S::LPM) / G;
    const int lc = tid % G;
    const int64_t mat0 = (int64_t)blockIdx.x * MPB;

    // global -> LDS, row-contiguous; padding is the identity
    for (int m = 0; m < MPB; ++m) {
        const int64_t mat = mat0 + m;
        const bool mv = mat < batch;
        const T *Am = A + (mv ? mat * sA : 0);
        T *St = stage + m * MSTRIDE;
        for (int idx = tid; idx < NP * NP; idx += THREADS) {
            const int i = idx / NP, k = idx % NP;
            T v = (i == k) ? T(1) : T(0);
            if (mv && i < n && k <= i)
                v = Am[(int64_t)i * lda + k];
            St[i * LDP + k] = v;
        }
    }
    __syncthreads();

    T x[E][E];
    {
        const T *St = stage + g * MSTRIDE;
#pragma unroll
        for (int a = 0; a < E; ++a)
#pragma unroll
            for (int b = 0; b <= a; ++b)
                x[a][b] = St[(lr + G * a) * LDP + lc + G * b];
    }

    int fail = 0;
    // column j = jb*G + jr; jb selects registers (compile time), jr only lanes
#pragma unroll
    for (int jb = 0; jb < E; ++jb) {
#pragma unroll 1
        for (int jr = 0; jr < G; ++jr) {
            const int j = jb * G + jr;
            T *cb = colbuf + ((j & 1) * MPB + g) * NP;
            // owners of column j publish it (unscaled); rows lr + G*a
            if (lc == jr) {
#pragma unroll
                for (int a = jb; a < E; ++a)
                    cb[lr * E + a] = x[a][jb];
            }
            __syncthreads();
            const T d = cb[jr * E + jb];
            T u[E], v[E];
#pragma unroll
            for (int a = jb; a < E; ++a)
                u[a] = cb[lr * E + a];
#pragma unroll
            for (int b = jb; b < E; ++b)
                v[b] = cb[lc * E + b];
            if (!(d > T(0)) && fail == 0)
                fail = j + 1;
            const T sq = dsqrt(d);
            const T rs = drcp(sq);
            const T rd = rs * rs;
            // only rows / columns strictly below / right of j take part in the update
            if (lr <= jr)
                u[jb] = T(0);
            if (lc <= jr)
                v[jb] = T(0);
            if (lc == jr) {
#pragma unroll
                for (int a = jb; a < E; ++a)
                    x[a][jb] = (a == jb && lr == jr) ? sq : x[a][jb] * rs;
            }
#pragma unroll
            for (int a = jb; a < E; ++a) {
                const T ua = u[a] * rd;
#pragma unroll
                for (int b = jb; b <= a; ++b)
                    x[a][b] -= ua * v[b];
            }
        }
    }

    // registers -> LDS -> global (lower triangle and zeroed upper)
    __syncthreads();
    {
        T *St = stage + g * MSTRIDE;
#pragma unroll
        for (int a = 0; a < E; ++a)
#pragma unroll
            for (int b = 0; b <= a; ++b)
                St[(lr + G * a) * LDP + lc + G * b] = x[a][b];
    }
    __syncthreads();
    for (int m = 0; m < MPB; ++m) {
        const int64_t mat = mat0 + m;
        if (mat >= batch)
            break;
        T *Lm = L + mat * sL;
        const T *St = stage + m * MSTRIDE;
        for (int idx = tid; idx < NP * NP; idx += THREADS) {
            const int i = idx / NP, k = idx % NP;
            if (i < n && k < n)
                Lm[(int64_t)i * ldl + k] = (k <= i) ? St[i * LDP + k] : T(0);
        }
    }
    if (lr == 0 && lc == 0 && mat0 + g < batch)
        write_info(info, mat0 + g, fail, info_mode, info_base);
}

// ------------------------------------------------------------------------
// Adjoint: Psi = sym(Phi(L^T adj_L)), V = Psi L^{-1}, Z = L^{-T} V (lower),
// lower(adj_A) (+)= Phi(Z).  adj_A may be adj_L itself when accumulate == 0.
// ------------------------------------------------------------------------
template <typename T, int G, int E>
__global__ void __launch_bounds__((TileShape<G, E>::THREADS))
k_potrf_adj_tile(int n, int64_t batch, const T *L, int64_t ldl, int64_t sL,
                 const T *adjL, int64_t ldal, int64_t sAL,
                 T *adjA, int64_t ldaa, int64_t sAA, int accumulate)
{
    typedef TileShape<G, E> S;
    constexpr int NP = S::NP, LDP = S::LDP, MSTRIDE = S::MSTRIDE, MPB = S::MPB, THREADS = S::THREADS;
    constexpr int LPSTRIDE = NP * NP + 16;
    __shared__ T lp[MPB * LPSTRIDE];      // L, rows natural, columns permuted; upper = 0
    __shared__ T scr[MPB * MSTRIDE];      // adj_L (permuted), then transposes, then G
    __shared__ T bc[2 * MPB * NP];

    const int tid = threadIdx.x;
    const int g = tid / S::LPM;
    const int lr = (tid % S::LPM) / G;
    const int lc = tid % G;
    const int64_t mat0 = (int64_t)blockIdx.x * MPB;

    for (int m = 0; m < MPB; ++m) {
        const int64_t mat = mat0 + m;
        const bool mv = mat < batch;
        const T *Lm = L + (mv ? mat * sL : 0);
        const T *Bm = adjL + (mv ? mat * sAL : 0);
        T *Lp = lp + m * LPSTRIDE;
        T *Sc = scr + m * MSTRIDE;
        for (int idx = tid; idx < NP * NP; idx += THREADS) {
            const int i = idx / NP, k = idx % NP;
            T lv = (i == k) ? T(1) : T(0);
            T bv = T(0);
            if (mv && i < n && k <= i) {
                lv = Lm[(int64_t)i * ldl + k];
                bv = Bm[(int64_t)i * ldal + k];
            }
            Lp[i * NP + perm_col<G, E>(k)] = lv;
            Sc[i * LDP + perm_col<G, E>(k)] = bv;
        }
    }
    __syncthreads();

    const T *Lp = lp + g * LPSTRIDE;
    T *Sc = scr + g * MSTRIDE;

    // M = L^T tril(adj_L), lower part: M_ij = sum_k L_ki adjL_kj (k >= i >= j).
    T p[E][E];
#pragma unroll
    for (int a = 0; a < E; ++a)
#pragma unroll
        for (int b = 0; b < E; ++b)
            p[a][b] = T(0);
#pragma unroll
    for (int kb = 0; kb < E; ++kb) {
#pragma unroll 1
        for (int kr = 0; kr < G; ++kr) {
            const int k = kb * G + kr;
            T lk[E], ak[E];
#pragma unroll
            for (int a = 0; a <= kb; ++a)
                lk[a] = Lp[k * NP + lr * E + a];    // L[k][lr + G a]
#pragma unroll
            for (int b = 0; b <= kb; ++b)
                ak[b] = Sc[k * LDP + lc * E + b];   // adjL[k][lc + G b]
#pragma unroll
            for (int a = 0; a <= kb; ++a)
#pragma unroll
                for (int b = 0; b <= a; ++b)
                    p[a][b] += lk[a] * ak[b];
        }
    }

    // Psi = P + P^T: lower entries of M stay; the upper ones are M's transposed
    // lower entries; the diagonal keeps M_ii (Phi halves it, the mirror adds it back).
    __syncthreads();
#pragma unroll
    for (int a = 0; a < E; ++a)
#pragma unroll
        for (int b = 0; b <= a; ++b) {
            const int i = lr + G * a, j = lc + G * b;
            if (i >= j)
                Sc[j * LDP + i] = p[a][b];      // transposed
        }
    __syncthreads();
#pragma unroll
    for (int a = 0; a < E; ++a)
#pragma unroll
        for (int b = a; b < E; ++b) {
            const int i = lr + G * a, j = lc + G * b;
            if (i < j)
                p[a][b] = Sc[i * LDP + j];      // = M_ji
        }

    // V = Psi L^{-1}  (V L = Psi), columns j = NP-1 .. 0:
    //   V[:, j] = R[:, j] / L_jj ;  R[:, k] -= V[:, j] L_jk  (k < j)
#pragma unroll
    for (int jb = E - 1; jb >= 0; --jb) {
#pragma unroll 1
        for (int jr = G - 1; jr >= 0; --jr) {
            const int j = jb * G + jr;
            T *cb = bc + ((j & 1) * MPB + g) * NP;
            if (lc == jr) {
                const T rinv = drcp(Lp[j * NP + jr * E + jb]);
#pragma unroll
                for (int a = 0; a < E; ++a) {
                    p[a][jb] *= rinv;
                    cb[lr * E + a] = p[a][jb];
                }
            }
            __syncthreads();
            T u[E], lj[E];
#pragma unroll
            for (int a = 0; a < E; ++a)
                u[a] = cb[lr * E + a];
#pragma unroll
            for (int b = 0; b <= jb; ++b)
                lj[b] = Lp[j * NP + lc * E + b];    // L[j][lc + G b]; zero right of j
            if (lc == jr)
                lj[jb] = T(0);                      // the solved column itself
#pragma unroll
            for (int a = 0; a < E; ++a)
#pragma unroll
                for (int b = 0; b <= jb; ++b)
                    p[a][b] -= u[a] * lj[b];
        }
    }

    // Z = L^{-T} V (L^T Z = V), lower part, rows i = NP-1 .. 0:
    //   Z[i, :] = R[i, :] / L_ii ;  R[t, :] -= L_it Z[i, :]  (t < i)
#pragma unroll
    for (int ib = E - 1; ib >= 0; --ib) {
#pragma unroll 1
        for (int ir = G - 1; ir >= 0; --ir) {
            const int i = ib * G + ir;
            T *cb = bc + ((i & 1) * MPB + g) * NP;
            if (lr == ir) {
                const T rinv = drcp(Lp[i * NP + ir * E + ib]);
#pragma unroll
                for (int b = 0; b <= ib; ++b) {
                    p[ib][b] *= rinv;
                    cb[lc * E + b] = p[ib][b];
                }
            }
            __syncthreads();
            T w[E], li[E];
#pragma unroll
            for (int b = 0; b <= ib; ++b)
                w[b] = cb[lc * E + b];
#pragma unroll
            for (int a = 0; a <= ib; ++a)
                li[a] = Lp[i * NP + lr * E + a];    // L[i][lr + G a]; zero right of i
            if (lr == ir)
                li[ib] = T(0);                      // the solved row itself
#pragma unroll
            for (int a = 0; a <= ib; ++a)
#pragma unroll
                for (int b = 0; b <= a; ++b)
                    p[a][b] -= li[a] * w[b];
        }
    }

    // G = Phi(Z): halve the diagonal; stage the lower triangle and store it.
    __syncthreads();
#pragma unroll
    for (int a = 0; a < E; ++a)
#pragma unroll
        for (int b = 0; b <= a; ++b) {
            const int i = lr + G * a, j = lc + G * b;
            if (i >= j)
                Sc[i * LDP + j] = (i == j) ? p[a][b] * T(0.5) : p[a][b];
        }
    __syncthreads();
    for (int m = 0; m < MPB; ++m) {
        const int64_t mat = mat0 + m;
        if (mat >= batch)
            break;
        T *Gm = adjA + mat * sAA;
        const T *Sm = scr + m * MSTRIDE;
        for (int idx = tid; idx < NP * NP; idx += THREADS) {
            const int i = idx / NP, k = idx % NP;
            if (i < n && k <= i) {
                T *dst = Gm + (int64_t)i * ldaa + k;
                const T gv = Sm[i * LDP + k];
                *dst = accumulate ? *dst + gv : gv;
            }
        }
    }
}

// ------------------------------------------------------------------------
// Diagnostic: dot product with a one-lane result and a broadcast adjoint.
// ------------------------------------------------------------------------
template <typename T>
__global__ void __launch_bounds__(64)
k_wave_dot(int n, const T *a, const T *b, T *y, const T *ybar, T *abar, T *bbar, int staging)
{
    __shared__ T sa[64], sb[64], sy[1];
    const int l = threadIdx.x;
    T av = T(0), bv = T(0);
    if (staging) {
        sa[l] = l < n ? a[l] : T(0);
        sb[l] = l < n ? b[l] : T(0);
        __syncthreads();
        av = sa[l];
        bv = sb[l];
    } else if (l < n) {
        av = a[l];
        bv = b[l];
    }
    // forward: wavefront reduction; only lane 0 owns the result
    T s = av * bv;
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1)
        s += __shfl_xor(s, off, 64);
    if (l == 0)
        y[0] = s;
    // reverse: the upstream gradient exists on lane 0 only ...
    T yb = (l == 0) ? ybar[0] : T(0);
    // ... and is published to every lane before any lane uses it
    if (staging) {
        if (l == 0)
            sy[0] = yb;
        __syncthreads();
        yb = sy[0];
    } else {
        yb = __shfl(yb, 0, 64);
    }
    if (l < n) {
        abar[l] += yb * bv;
        bbar[l] += yb * av;
    }
}

// ------------------------------------------------------------------ hosts ----
template <typename T, int G, int E>
static chol_status launch_potrf_tile(int n, int64_t batch, const T *A, int64_t lda, int64_t sA,
                                     T *L, int64_t ldl, int64_t sL, int32_t *info, int info_mode,
                                     int64_t info_base, hipStream_t st)
{
    typedef TileShape<G, E> S;
    const int64_t blocks = (batch + S::MPB - 1) / S::MPB;
    hipLaunchKernelGGL((k_potrf_tile<T, G, E>), dim3((unsigned)blocks), dim3(S::THREADS), 0, st,
                       n, batch, A, lda, sA, L, ldl, sL, info, info_mode, info_base);
    CHOL_LAUNCH_CHECK();
    return CHOL_OK;
}

template <typename T, int G, int E>
static chol_status launch_adj_tile(int n, int64_t batch, const T *L, int64_t ldl, int64_t sL,
                                   const T *adjL, int64_t ldal, int64_t sAL, T *adjA, int64_t ldaa,
                                   int64_t sAA, int accumulate, hipStream_t st)
{
    typedef TileShape<G, E> S;
    const int64_t blocks = (batch + S::MPB - 1) / S::MPB;
    hipLaunchKernelGGL((k_potrf_adj_tile<T, G, E>), dim3((unsigned)blocks), dim3(S::THREADS), 0, st,
                       n, batch, L, ldl, sL, adjL, ldal, sAL, adjA, ldaa, sAA, accumulate);
    CHOL_LAUNCH_CHECK();
    return CHOL_OK;
}

// Batched small factor: n <= 64.
template <typename T>
chol_status small_potrf(int n, int64_t batch, const T *A, int64_t lda, int64_t sA, T *L, int64_t ldl,
                        int64_t sL, int32_t *info, int info_mode, int64_t info_base, hipStream_t st)
{
    if (n <= 4)
        return launch_potrf_tile<T, 4, 1>(n, batch, A, lda, sA, L, ldl, sL, info, info_mode, info_base, st);
    if (n <= 8)
        return launch_potrf_tile<T, 4, 2>(n, batch, A, lda, sA, L, ldl, sL, info, info_mode, info_base, st);
    if (n <= 16)
        return launch_potrf_tile<T, 4, 4>(n, batch, A, lda, sA, L, ldl, sL, info, info_mode, info_base, st);
    if (n <= 32)
        return launch_potrf_tile<T, 4, 8>(n, batch, A, lda, sA, L, ldl, sL, info, info_mode, info_base, st);
    return launch_potrf_tile<T, 8, 8>(n, batch, A, lda, sA, L, ldl, sL, info, info_mode, info_base, st);
}

// Diagonal tile of the blocked factor: n <= 128, one 256-thread block.
template <typename T>
chol_status diag_potrf(int n, T *W, int64_t ld, int32_t *info, int info_mode, int64_t info_base,
                       hipStream_t st)
{
    if (n <= 64)
        return small_potrf<T>(n, 1, W, ld, 0, W, ld, 0, info, info_mode, info_base, st);
    return launch_potrf_tile<T, 16, 8>(n, 1, W, ld, 0, W, ld, 0, info, info_mode, info_base, st);
}

template <typename T>
chol_status small_potrf_adjoint(int n, int64_t batch, const T *L, int64_t ldl, int64_t sL,
                                const T *adjL, int64_t ldal, int64_t sAL, T *adjA, int64_t ldaa,
                                int64_t sAA, int accumulate, hipStream_t st)
{
    if (n <= 4)
        return launch_adj_tile<T, 4, 1>(n, batch, L, ldl, sL, adjL, ldal, sAL, adjA, ldaa, sAA, accumulate, st);
    if (n <= 8)
        return launch_adj_tile<T, 4, 2>(n, batch, L, ldl, sL, adjL, ldal, sAL, adjA, ldaa, sAA, accumulate, st);
    if (n <= 16)
        return launch_adj_tile<T, 4, 4>(n, batch, L, ldl, sL, adjL, ldal, sAL, adjA, ldaa, sAA, accumulate, st);
    if (n <= 32)
        return launch_adj_tile<T, 4, 8>(n, batch, L, ldl, sL, adjL, ldal, sAL, adjA, ldaa, sAA, accumulate, st);
    return launch_adj_tile<T, 8, 8>(n, batch, L, ldl, sL, adjL, ldal, sAL, adjA, ldaa, sAA, accumulate, st);
}

template <typename T>
chol_status wave_dot(int n, const T *a, const T *b, T *y, const T *ybar, T *abar, T *bbar, int staging,
                     hipStream_t st)
{
    hipLaunchKernelGGL((k_wave_dot<T>), dim3(1), dim3(64), 0, st, n, a, b, y, ybar, abar, bbar, staging);
    CHOL_LAUNCH_CHECK();
    return CHOL_OK;
}

#define CHOL_INST(T)                                                                                      \
    template chol_status small_potrf<T>(int, int64_t, const T *, int64_t, int64_t, T *, int64_t, int64_t, \
                                        int32_t *, int, int64_t, hipStream_t);                            \
    template chol_status diag_potrf<T>(int, T *, int64_t, int32_t *, int, int64_t, hipStream_t);          \
    template chol_status small_potrf_adjoint<T>(int, int64_t, const T *, int64_t, int64_t, const T *,     \
                                                int64_t, int64_t, T *, int64_t, int64_t, int, hipStream_t); \
    template chol_status wave_dot<T>(int, const T *, const T *, T *, const T *, T *, T *, int, hipStream_t);
CHOL_INST(float)
CHOL_INST(double)
#undef CHOL_INST

} // namespace chol
