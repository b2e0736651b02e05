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
#include "side.hpp"
#include "plan.hpp"

namespace chol {

template <typename T>
chol_status diag_potrf(int n, T *W, int64_t ld, int32_t *info, int info_mode, int64_t info_base, T *inv,
                       int64_t ldinv, hipStream_t st);

// edge of a diagonal-tile inverse slot in the library's side buffer
static constexpr int MAX_TILE = CHOL_MAX_NB;

// ------------------------------------------------------------ elementwise ----
enum { TRI_COPY_LOWER = 0, TRI_ZERO_UPPER = 1, TRI_ADD_LOWER = 2, TRI_ZERO_LOWER = 3 };

// 32 x 32 element tiles; a block covers one tile with 256 threads.
template <typename T, int MODE>
__global__ void __launch_bounds__(256)
k_tri(int64_t n, int64_t w, const T *src, int64_t lds, T *dst, int64_t ldd)
{
    const int64_t i0 = (int64_t)blockIdx.y * 32, j0 = (int64_t)blockIdx.x * 32;
    if (MODE == TRI_ZERO_UPPER ? (j0 + 31 <= i0) : (j0 > i0 + 31))
        return;
    const int tj = threadIdx.x % 32, ti = threadIdx.x / 32;
    for (int r = ti; r < 32; r += 8) {
        const int64_t i = i0 + r, j = j0 + tj;
        if (i >= n || j >= w)
            continue;
        if (MODE == TRI_COPY_LOWER) {
            if (j <= i)
                dst[i * ldd + j] = src[i * lds + j];
        } else if (MODE == TRI_ZERO_UPPER) {
            if (j > i)
                dst[i * ldd + j] = T(0);
        } else if (MODE == TRI_ZERO_LOWER) {
            if (j <= i)
                dst[i * ldd + j] = T(0);
        } else {
            if (j <= i)
                dst[i * ldd + j] += src[i * lds + j];
        }
    }
}

// the entries of the n x n operand in columns 0 .. w-1 (w <= n; the lower ones
// for COPY_LOWER and ADD_LOWER, the strict upper ones for ZERO_UPPER)
template <typename T, int MODE>
static chol_status tri_op(int64_t n, const T *src, int64_t lds, T *dst, int64_t ldd, hipStream_t st,
                          int64_t w = -1)
{
    if (w < 0 || w > n)
        w = n;
    // lower entries of the first w columns: w (n - w) + w (w + 1) / 2
    const double tri = (double)w * (n - w) + (double)w * (w + 1) / 2, es = (double)sizeof(T);
    const double bytes = MODE == TRI_COPY_LOWER ? 2 * tri * es
                       : MODE == TRI_ZERO_UPPER ? ((double)n * w - tri) * es
                       : MODE == TRI_ZERO_LOWER ? tri * es : 3 * tri * es;
    prof::Scope ps(CHOL_K_ELEMENTWISE, st, bytes);
    const unsigned tr = (unsigned)((n + 31) / 32), tc = (unsigned)((w + 31) / 32);
    if (tr == 0 || tc == 0)
        return CHOL_OK;
    hipLaunchKernelGGL((k_tri<T, MODE>), dim3(tc, tr), dim3(256), 0, st, n, w, src, lds, dst, ldd);
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
//   out_mode 1: X written to ws + t*ws_stride with leading dim ws_ld, the
//               zeros above its diagonal included (the kb x kb block), so
//               that products can read it as a plain operand.
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
    // all of the thread's loads are issued before the first LDS write
    constexpr int PER = NP * NP / 256;
    T stage[PER];
#pragma unroll
    for (int q = 0; q < PER; ++q) {
        const int idx = tid + 256 * q, i = idx / NP, k = idx % NP;
        stage[q] = (i == k) ? T(1) : T(0);
        if (i < kb && k <= i)
            stage[q] = Lkk[(int64_t)i * ld + k];
    }
#pragma unroll
    for (int q = 0; q < PER; ++q) {
        const int idx = tid + 256 * q, i = idx / NP, k = idx % NP;
        ls[i * LP + k] = stage[q];
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

    if (out_mode == 0) {
#pragma unroll
        for (int a = 0; a < E; ++a)
#pragma unroll
            for (int b = 0; b < a + 1; ++b) {
                const int i = lr + G * a, j = lc + G * b;
                if (i < kb && j < i)
                    W[(k0 + j) * ld + k0 + i] = x[a][b];
            }
        return;
    }
    T *X = ws + (int64_t)blockIdx.x * ws_stride;
#pragma unroll
    for (int a = 0; a < E; ++a)
#pragma unroll
        for (int b = 0; b < E; ++b) {
            const int i = lr + G * a, j = lc + G * b;
            if (i < kb && j < kb)
                X[(int64_t)i * ws_ld + j] = (b <= a && j <= i) ? x[a][b] : T(0);
        }
}

// C_lower(n x n) -= sum_s part[s] (lower entries only).  A block takes 64
// consecutive entries; its four waves each sum every fourth split (wave w:
// splits w, w+4, ...), and the four sums are added in wave order, so the
// result does not depend on scheduling.  With up to 128 partials of a
// 128 x 128 tile this spreads the reads over 256 blocks instead of leaving
// one thread per entry to walk all of them.
template <typename T>
__global__ void __launch_bounds__(256)
k_splitk_reduce_lower(int n, int splits, const T *part, T *c, int64_t ldc)
{
    __shared__ T sums[4][64];
    const int lane = threadIdx.x % 64, w = threadIdx.x / 64;
    const int64_t tot = (int64_t)n * n;
    const int64_t idx = (int64_t)blockIdx.x * 64 + lane;
    const int r = (int)(idx / n), col = (int)(idx % n);
    const bool live = idx < tot && col <= r;
    T s = T(0);
    if (live)
        for (int q = w; q < splits; q += 4)
            s += part[(int64_t)q * tot + idx];
    sums[w][lane] = s;
    __syncthreads();
    if (w == 0 && live)
        c[(int64_t)r * ldc + col] -= ((sums[0][lane] + sums[1][lane]) + sums[2][lane]) + sums[3][lane];
}

// The partial sums a split-contraction product left for its M x N output
// (C_PARTIAL, row-major M x N per slot): `splits` slots per entry, or with
// `piece` > 0 the slots of the pieces that touched the entry's 128 x 128 tile
// (tiles TJ per row of tiles, contraction nku units long, pieces numbered
// along the tiles' contractions laid end to end); none when part is null.
template <typename T> struct Partials {
    const T *part = nullptr;
    int M = 0, N = 0, splits = 0, TJ = 1;
    int64_t nku = 0, piece = 0;
    __host__ __device__ int count(int r, int c) const
    {
        if (!part)
            return 0;
        if (piece <= 0)
            return splits;
        const int64_t t = (int64_t)(r / 128) * TJ + c / 128;
        return (int)(((t + 1) * nku - 1) / piece - (t * nku) / piece + 1);
    }
};

// C(M x N) -= the sum of the partials (slots in contraction order), then
// C -= slot in the first kn rows (slot row-major kn x N; null: none): the sums
// of a split product and of a term computed elsewhere, one pass over C.
template <typename T>
__global__ void __launch_bounds__(256)
k_splitk_reduce(int M, int N, Partials<T> ps, const T *slot, int kn, T *c, int64_t ldc)
{
    const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
    const int64_t tot = (int64_t)M * N;
    if (idx >= tot)
        return;
    const int r = (int)(idx / N), col = (int)(idx % N);
    const int cnt = ps.count(r, col);
    T s = T(0);
    for (int q = 0; q < cnt; ++q)
        s += ps.part[(int64_t)q * tot + idx];
    T x = c[(int64_t)r * ldc + col] - s;
    if (slot && r < kn)
        x -= slot[idx];
    c[(int64_t)r * ldc + col] = x;
}

template <typename T>
static chol_status splitk_reduce(int M, int N, const Partials<T> &ps, const T *slot, int kn, T *c, int64_t ldc,
                                 hipStream_t st)
{
    const int64_t tot = (int64_t)M * N;
    if (tot <= 0)
        return CHOL_OK;
    double slots = ps.part ? ps.splits : 0;
    if (ps.part && ps.piece > 0) {
        const int64_t tiles = (int64_t)((M + 127) / 128) * ps.TJ;
        slots = (double)((tiles * ps.nku + ps.piece - 1) / ps.piece) / tiles + 1;
    }
    const double sbytes = slot ? (double)kn * N * sizeof(T) : 0.0;
    prof::Scope pscope(CHOL_K_REDUCE, st, (double)tot * (slots + 2) * sizeof(T) + sbytes);
    hipLaunchKernelGGL((k_splitk_reduce<T>), dim3((unsigned)((tot + 255) / 256)), dim3(256), 0, st, M, N, ps, slot,
                       kn, c, ldc);
    CHOL_LAUNCH_CHECK();
    return CHOL_OK;
}

// contraction length per split: a whole number of fp32 chunks (32), which is
// also a whole number of fp64 chunks (16)
static inline int split_chunk(int64_t K, int splits)
{
    int c = (int)((K + splits - 1) / splits);
    return (c + 31) / 32 * 32;
}

// ------------------------------------------------------------- forward ----
// Two library streams: `sx` runs every kernel that spans the matrix (panel
// solves and trailing updates) in order; `sc` runs only the one-block kernels
// of the next tile column (diagonal factor and its inverse), beside the wide
// update that follows it on sx (where no such update is left, the factor
// runs on sx itself).  The order of the launches, the deferred
// trailing update and the joins between the streams are the host-side plan of
// plan.cpp; this executor launches that plan as it stands.
template <typename T>
static chol_status blocked_potrf_on(int64_t n, const T *A, int64_t lda, T *L, int64_t ldl, int32_t *info,
                                    int nb, hipStream_t sc, hipStream_t sx, hipEvent_t e_diag, hipEvent_t e_next,
                                    int *sched_x, int cap_x, T *inv2)
{
    auto slot_ptr = [&](int slot) { return inv2 + (int64_t)slot * MAX_TILE * MAX_TILE; };
    // lower part of W[c:, c:c+w] -= Q[c:] Q[c:c+w]^T with Q = panels f .. f+np-1
    // (tile columns f .. f+np-1 of L); tri: the whole trailing triangle W[c:, c:]
    // instead, restricted to the 128 x 128 tiles t0 .. t0+tn-1 (row-major over
    // the lower tiles), taken by persistent blocks; from_a: W's current values
    // are those of A (the tiles' first update), the results go to L
    auto lower_update = [&](int64_t c, int64_t w, int64_t f, int np, bool tri, int t0, int tn,
                            bool from_a) -> chol_status {
        const int64_t M = n - c;
        const int Kd = np * nb;
        GemmArgs<T> p{};
        p.M = (int)M; p.N = (int)(tri ? M : w); p.K = Kd;
        p.a = L + c * ldl + f * nb; p.lda = ldl;
        p.b = L + c * ldl + f * nb; p.ldb = ldl;
        p.c = L + c * ldl + c; p.ldc = ldl;
        if (from_a) {
            p.cin = A + c * lda + c;
            p.ldcin = lda;
        }
        double flops;
        if (tri) {
            p.tri = 1;
            p.t0 = t0;
            p.tn = tn;
            p.sched = sched_x;
            p.cap = cap_x;
            // tiles of the window: full ones 2*128*128*Kd flops, diagonal ones
            // the lower half (rows of the last tile row may be short)
            flops = 0;
            int64_t r = 0, t = 0;
            while (t + r + 1 <= t0) { t += r + 1; ++r; }
            for (int64_t q = t0, cc = t0 - t; q < (int64_t)t0 + tn; ++q) {
                const double hr = (double)std::min<int64_t>(128, M - r * 128);
                flops += (cc == r) ? hr * (hr + 1) * Kd : 2.0 * hr * 128 * Kd;
                if (++cc > r) { cc = 0; ++r; }
            }
        } else {
            flops = (double)w * (w + 1) * Kd + 2.0 * (M - w) * w * Kd;
        }
        prof::Scope ps(CHOL_K_TRAILING_UPDATE, sx, flops);
        // the narrow updates of single panels (128 deep) and those with few
        // 128 x 128 tiles take 64 x 128 tiles: a 128-deep 128 x 128 tile is
        // ~20 us of one CU's matrix cores, and a short launch is as long as
        // its slowest tile (up to 3 x 256 of the smaller tiles are resident
        // at once, three per CU: nothing runs beside these launches)
        if (!tri) {
            const int64_t tiles128 = ((M + 127) / 128) * ((w + 127) / 128);
            if (Kd <= 128 || tiles128 <= 384) {
                // fewer 64 x 128 tiles than CUs: 64 x 64 tiles, twice as many
                if (2 * tiles128 < 256)
                    return gemm<T, OP_MK, OP_MK, C_SUB_LOWER, 64, 64>(p, 1, sx);
                return gemm<T, OP_MK, OP_MK, C_SUB_LOWER, 64>(p, 1, sx);
            }
            return gemm<T, OP_MK, OP_MK, C_SUB_LOWER>(p, 1, sx);
        }
        // a far-triangle part of at most half a round of the persistent grid
        // runs as the halves (64 x 128) of its tiles: one round of items half
        // as long, on the same slots (two per CU, so a CU with one of them
        // still has room for the diagonal factor beside it)
        if (2 * (int64_t)tn <= cap_x)
            return gemm<T, OP_MK, OP_MK, C_SUB_LOWER, 64>(p, 1, sx);
        return gemm<T, OP_MK, OP_MK, C_SUB_LOWER>(p, 1, sx);
    };
    const std::vector<FwdOp> plan = forward_plan(n, nb, A != L, cap_x);
    for (const FwdOp &o : plan) {
        chol_status s = CHOL_OK;
        switch (o.kind) {
        case FWD_COPY:
            s = tri_op<T, TRI_COPY_LOWER>(n, A, lda, L, ldl, sc, o.w);
            break;
        case FWD_DIAG: {
            const int64_t k0 = o.k * nb;
            const int kb = (int)std::min<int64_t>(nb, n - k0);
            const double kb3 = (double)kb * kb * kb;
            hipStream_t ds = o.stream == FWD_WIDE ? sx : sc;
            prof::Scope ps(CHOL_K_DIAG_FACTOR, ds, o.slot >= 0 ? 2 * kb3 / 3 : kb3 / 3);
            s = diag_potrf<T>(kb, L + k0 * ldl + k0, ldl, info, o.k == 0 ? 1 : 2, k0,
                              o.slot >= 0 ? slot_ptr(o.slot) : nullptr, MAX_TILE, ds);
            break;
        }
        case FWD_PANEL: {
            // L_ik = W_ik * Linv^T  (in place; one block spans the full panel
            // width; Linv is read whole from its slot, element (j, t) = Linv[j][t])
            const int64_t k0 = o.k * nb;
            const int kb = (int)std::min<int64_t>(nb, n - k0);
            const int64_t r0 = k0 + kb, m = n - r0;
            GemmArgs<T> p{};
            p.M = (int)m; p.N = kb; p.K = kb;
            p.a = L + r0 * ldl + k0; p.lda = ldl;
            p.b = slot_ptr(o.slot); p.ldb = MAX_TILE;
            p.c = L + r0 * ldl + k0; p.ldc = ldl;
            prof::Scope ps(CHOL_K_PANEL_SOLVE, sx, (double)m * kb * kb);
            // 32-row tiles, each a whole 128-wide row panel (in place): twice
            // the blocks of 64-row tiles, each half as long a product
            s = gemm<T, OP_MK, OP_MK, C_STORE, 32>(p, 1, sx);
            break;
        }
        case FWD_UPDATE:
            s = lower_update(o.c, o.w, o.f, o.np, false, 0, 0, false);
            break;
        case FWD_TRI:
            s = lower_update(o.c, 0, o.f, o.np, true, o.t0, o.tn, o.slot == 1);
            break;
        case FWD_JOIN: {
            hipEvent_t ev = o.slot == 0 ? e_diag : e_next;
            const bool wide = o.stream == FWD_WIDE;
            if (stream_join(wide ? sx : sc, wide ? sc : sx, ev) != hipSuccess)
                s = CHOL_ERR_HIP;
            break;
        }
        case FWD_ZERO_UPPER:
            s = tri_op<T, TRI_ZERO_UPPER>(n, nullptr, 0, L, ldl, sc);
            break;
        default:
            s = CHOL_ERR_INVALID_VALUE;
        }
        if (s != CHOL_OK)
            return s;
    }
    return CHOL_OK;
}

template <typename T>
chol_status blocked_potrf(int64_t n, const T *A, int64_t lda, T *L, int64_t ldl, int32_t *info, int nb,
                          hipStream_t st)
{
    Side *sd = side_resources();
    if (!sd)
        return CHOL_ERR_HIP;
    std::lock_guard<std::mutex> lk(sd->mu);
    // both library streams start after the caller's earlier work; the caller's
    // stream resumes after both are done.  The persistent grids' work counters
    // are zeroed first, in stream order (a call that did not complete cannot
    // leave a later one starting from a stale count).
    if (stream_join(sd->chain, st, sd->ev[2]) != hipSuccess || stream_join(sd->x, st, sd->ev[2]) != hipSuccess ||
        zero_ints(sd->sched, SCHED_INTS, sd->x) != hipSuccess)
        return CHOL_ERR_HIP;
    const chol_status s = blocked_potrf_on<T>(n, A, lda, L, ldl, info, nb, sd->chain, sd->x, sd->ev[0], sd->ev[1],
                                              sd->sched, 2 * sd->wide_cus, (T *)sd->fwd_inv);
    const bool joined = stream_join(sd->chain, sd->x, sd->ev[3]) == hipSuccess &&
                        stream_join(st, sd->chain, sd->ev[4]) == hipSuccess;
    if (s != CHOL_OK)
        return s;
    return joined ? CHOL_OK : CHOL_ERR_HIP;
}

// ------------------------------------------------------------- adjoint ----
// Workspace layout (each part 256-byte aligned):
//   [Wb    : n * n]                         running gradient (absent when formed in adj_A)
//   [inv   : K * nb * nb]                   inverses of the diagonal tiles of L
//   [part_x: max_splits * n * nb]           split partials of the large symmetric product
//   [part_b: (ceil(n / 128) + 1) * nb * nb] one partial of the tile column's diagonal
//                                           update per 128-row tile of its panel, plus the
//                                           slot the tile adjoint adds
//   [part_c: 2 * nb * nb]                   the tile adjoint's scratch tiles
//   [dense : K * nb * nb]                   Sym(G) of every diagonal tile, whole (nb = 128)
static inline size_t align256(size_t x) { return (x + 255) & ~size_t(255); }
// partials of the diagonal update: one per 128-row tile of the longest panel
static inline int64_t panel_tiles(int64_t n) { return (n + 127) / 128; }
static const int SIDE_SPLIT_MAX = 32;    // splits of the large symmetric product

size_t blocked_adjoint_workspace(int64_t n, int nb, size_t esize, bool need_wb, int max_splits)
{
    const int64_t K = (n + nb - 1) / nb;
    size_t s = 0;
    if (need_wb)
        s += align256((size_t)n * n * esize);
    s += align256((size_t)K * nb * nb * esize);
    s += align256((size_t)max_splits * n * nb * esize);
    s += align256((size_t)(panel_tiles(n) + 1) * nb * nb * esize);
    s += align256((size_t)2 * nb * nb * esize);
    s += align256((size_t)K * nb * nb * esize);
    return s;
}

// C (M x N) -= Sym(S)[0:M, 0:K] B with S symmetric stored as its lower triangle
// (diagonal doubled by the operand), its leading excl x excl block left out,
// and B k-major; the contraction is split so
// that the launch fills at most one wave of blocks, and the partials are summed
// in a fixed order, so the result does not depend on scheduling.
template <typename T>
static chol_status sym_product(int M, int N, int K, const T *S, int64_t lds, const T *B, int64_t ldb, T *C,
                               int64_t ldc, int excl, const T *dg, T *part, int max_splits, int min_chunk,
                               int *sched, int cap, double flops, hipStream_t st, Partials<T> *defer = nullptr)
{
    if (M <= 0 || N <= 0 || K <= 0)
        return CHOL_OK;
    GemmArgs<T> p{};
    p.M = M; p.N = N; p.K = K;
    p.a = S; p.lda = lds;
    p.b = B; p.ldb = ldb;
    p.c = C; p.ldc = ldc;
    // (split, tile) items are taken by `cap` persistent blocks; pick the split
    // count that minimises the estimated time: rounds of items x chunk length
    // (a last round that is only partly full costs a whole chunk time) plus
    // the partials each split writes and the reduction reads back, expressed
    // in contraction elements (a 128 x 128 block advances 16 of them in about
    // 5 us; the partial traffic moves at about 5 TB/s)
    const int64_t tiles = (int64_t)((M + 127) / 128) * ((N + 127) / 128);
    const double per_split = (double)M * N * 2.0 * sizeof(T) / 5e12 / (5e-6 / 16);
    double best_t = -1;
    int kchunk = K;
    for (int sp = 1; sp <= max_splits; ++sp) {
        const int c = split_chunk(K, sp);
        if (sp > 1 && c < min_chunk)
            break;
        const int used = (K + c - 1) / c;
        const int64_t items = tiles * used;
        const double t = (double)((items + cap - 1) / cap) * c + per_split * used;
        if (best_t < 0 || t < best_t) {
            best_t = t;
            kchunk = c;
        }
    }
    // Pieces instead: the tiles' contractions laid end to end and cut into
    // equal pieces, so that r rounds of the grid hold exactly the work (equal
    // splits leave part of the last round idle); a tile then sums a partial
    // per piece that touched it (at most ceil(units / piece) + 1)
    const int64_t nku = ((int64_t)K + SK_UNIT - 1) / SK_UNIT, W = tiles * nku;
    const int64_t min_units = std::max<int64_t>(1, min_chunk / SK_UNIT);
    int64_t piece = 0;
    for (int r = 1; r <= 64; ++r) {
        const int64_t P = (W + (int64_t)cap * r - 1) / ((int64_t)cap * r);
        if (P < min_units)
            break;
        if ((nku + P - 1) / P + 1 > max_splits)
            continue;
        const int64_t items = (W + P - 1) / P;
        const double t = (double)((items + cap - 1) / cap) * P * SK_UNIT + per_split * ((double)items / tiles + 1);
        if (t < best_t) {
            best_t = t;
            piece = P;
        }
    }
    p.kchunk = kchunk;
    p.piece = (int)piece;
    const int used = (K + p.kchunk - 1) / p.kchunk;
    p.part = part;
    p.sched = sched;
    p.cap = cap;
    p.excl = excl;
    p.dg = dg;
    {
        prof::LaunchEvents pe(CHOL_K_ADJ_TRAILING, flops);
        chol_status s = gemm<T, OP_SYM, OP_KM, C_PARTIAL>(p, used, st, pe.a, pe.b);
        if (s != CHOL_OK)
            return s;
    }
    Partials<T> ps;
    ps.part = part;
    ps.M = M;
    ps.N = N;
    ps.splits = used;
    ps.TJ = (N + 127) / 128;
    ps.nku = nku;
    ps.piece = piece;
    // C -= the sum of the partials, now or (defer) by the caller's next pass
    // over C
    if (defer) {
        *defer = ps;
        return CHOL_OK;
    }
    return splitk_reduce<T>(M, N, ps, (const T *)nullptr, 0, C, ldc, st);
}

template <typename T>
__device__ __forceinline__ int vec_ok(const T *p, int64_t ld)
{
    return ((uintptr_t)p % 16 == 0) && (ld % (16 / (int64_t)sizeof(T)) == 0);
}

// Adjoint of chol on one kb x kb diagonal tile (kb <= 128), in place on the
// lower triangle of Wb, from the tile's factor L and its inverse Linv (stored
// with its zeros, kb x kb, leading dimension ldi), as four stages, each one
// kb x kb x kb matrix-core product:
//   stage 0: M = L^T tril(Wb); Psi = Phi(M) + Phi(M)^T (the lower part of M
//            mirrored, diagonal M_ii) whole into the scratch s1
//   stage 1: V = Psi Linv into the scratch s2
//   stage 2: Z = Linv^T V (symmetric); G = Phi(Z) into Wb (lower), and
//            Sym(G) = G + G^T (the lower part of Z mirrored) whole into sg,
//            the tile's dense copy that the symmetric products of later tile
//            columns read as their diagonal block
//   stage 3: when `slot` is given, the one term of the previous tile column's
//            trailing-update adjoint that needs G: slot = Sym(G) Lnext (kb x
//            nj, row major), Lnext = L[this tile's rows, previous tile column]
// Each stage is a launch of one block per ADJ_TILE x ADJ_TILE block of its
// product (stages 0 and 2 skip the blocks above the diagonal), so that the
// chain of tile adjoints, which sets the pace of the sweep while the trailing
// blocks are small, is spread over ten to sixteen CUs (a one-block kernel
// doing all four stages took 90 us per tile; with 64 x 64 blocks a stage took
// about 10 us, most of it one block's 64-deep share of the matrix cores).
// The stream orders the stages, so each reads what the one before wrote.  In
// stages 0 and 2 a block writes the entries (r, c), c <= r, of its block and
// their mirrors (c, r): the mirrors of a block below the diagonal land in a
// skipped one, those of a diagonal block in its own upper part, so no two
// blocks write the same entry.  Only stage 0 reads masked triangles (of the
// caller's L and Wb); the others read plain whole operands.
constexpr int ADJ_TILE = 32;
template <typename T, int STAGE>
__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2)))
k_tile_adjoint_stage(int kb, const T *L, int64_t ldl, T *Wb, int64_t ldw, const T *inv, int64_t ldi, T *s1,
                     T *s2, int64_t lds_scr, const T *Lnext, int nj, T *slot, T *sg, int64_t ldsg)
{
    using namespace gemm_detail;
    typedef typename Acc<T>::type acc_t;
    constexpr int TM = ADJ_TILE, TN = ADJ_TILE;
    __builtin_amdgcn_s_setprio(3);
    __shared__ T lds[LDS_ELEMS<T, TM>];
    const int r0 = (int)blockIdx.x * TM, c0 = (int)blockIdx.y * TN;
    // stages 0 and 2 keep only the lower part of their (symmetric) result
    const bool lower_only = STAGE == 0 || STAGE == 2;
    if (r0 >= kb || c0 >= (STAGE == 3 ? nj : kb) || (lower_only && r0 + TM <= c0))
        return;
    AccTile<T, TM, TN> acc;
#pragma unroll
    for (int i = 0; i < WaveTile<TM, TN>::FRM; ++i)
#pragma unroll
        for (int j = 0; j < WaveTile<TM, TN>::FRN; ++j)
            acc[i][j] = acc_t{0, 0, 0, 0};
    const int vs = vec_ok(s1, lds_scr) && vec_ok(s2, lds_scr);
    const int vi = vec_ok(inv, ldi);
    if (STAGE == 0) {
        Operand<T, OP_KM_LOWER, TM> A{L, ldl, r0, kb, vec_ok(L, ldl)};
        Operand<T, OP_KM_LOWER, TN> B{Wb, ldw, c0, kb, vec_ok(Wb, ldw)};
        tile_mma<T, OP_KM_LOWER, OP_KM_LOWER, false, false, false, TM, TN>(acc, A, B, 0, kb, lds);
    } else if (STAGE == 1) {
        Operand<T, OP_MK, TM> A{s1, lds_scr, r0, kb, vs};
        Operand<T, OP_KM, TN> B{inv, ldi, c0, kb, vs && vi};
        tile_mma<T, OP_MK, OP_KM, false, false, false, TM, TN>(acc, A, B, 0, kb, lds);
    } else if (STAGE == 2) {
        Operand<T, OP_KM, TM> A{inv, ldi, r0, kb, vs && vi};
        Operand<T, OP_KM, TN> B{s2, lds_scr, c0, kb, vs && vi};
        tile_mma<T, OP_KM, OP_KM, false, false, false, TM, TN>(acc, A, B, 0, kb, lds);
    } else {
        Operand<T, OP_MK, TM> A{sg, ldsg, r0, kb, vec_ok(sg, ldsg)};
        Operand<T, OP_KM, TN> B{Lnext, ldl, c0, nj, vs && vec_ok(Lnext, ldl)};
        tile_mma<T, OP_MK, OP_KM, false, false, false, TM, TN>(acc, A, B, 0, kb, lds);
    }
#pragma unroll
    for (int i = 0; i < WaveTile<TM, TN>::FRM; ++i)
#pragma unroll
        for (int j = 0; j < WaveTile<TM, TN>::FRN; ++j)
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                int r, c;
                acc_pos<T, TM, TN>(i, j, v, r, c);
                r += r0;
                c += c0;
                const T x = acc[i][j][v];
                if (STAGE == 0) {
                    if (r < kb && c <= r) {
                        s1[(int64_t)r * lds_scr + c] = x;
                        s1[(int64_t)c * lds_scr + r] = x;
                    }
                } else if (STAGE == 1) {
                    if (r < kb && c < kb)
                        s2[(int64_t)r * lds_scr + c] = x;
                } else if (STAGE == 2) {
                    if (r < kb && c <= r) {
                        Wb[(int64_t)r * ldw + c] = (r == c) ? T(0.5) * x : x;
                        if (sg) {
                            sg[(int64_t)r * ldsg + c] = x;
                            sg[(int64_t)c * ldsg + r] = x;
                        }
                    }
                } else {
                    if (r < kb && c < nj)
                        slot[(int64_t)r * nj + c] = x;
                }
            }
}

template <typename T>
static chol_status tile_adjoint_stages(hipStream_t st, int kb, const T *L, int64_t ldl, T *Wb, int64_t ldw,
                                       const T *inv, int64_t ldi, T *s1, T *s2, int64_t lds_scr, const T *Lnext,
                                       int nj, T *slot, T *sg, int64_t ldsg)
{
    const unsigned q = (unsigned)((kb + ADJ_TILE - 1) / ADJ_TILE);
    const dim3 grid(q, q), grid3(q, (unsigned)((nj + ADJ_TILE - 1) / ADJ_TILE));
    hipLaunchKernelGGL((k_tile_adjoint_stage<T, 0>), grid, dim3(256), 0, st, kb, L, ldl, Wb, ldw, inv, ldi, s1, s2,
                       lds_scr, Lnext, nj, slot, sg, ldsg);
    CHOL_LAUNCH_CHECK();
    hipLaunchKernelGGL((k_tile_adjoint_stage<T, 1>), grid, dim3(256), 0, st, kb, L, ldl, Wb, ldw, inv, ldi, s1, s2,
                       lds_scr, Lnext, nj, slot, sg, ldsg);
    CHOL_LAUNCH_CHECK();
    hipLaunchKernelGGL((k_tile_adjoint_stage<T, 2>), grid, dim3(256), 0, st, kb, L, ldl, Wb, ldw, inv, ldi, s1, s2,
                       lds_scr, Lnext, nj, slot, slot ? sg : (T *)nullptr, ldsg);
    CHOL_LAUNCH_CHECK();
    if (slot) {
        hipLaunchKernelGGL((k_tile_adjoint_stage<T, 3>), grid3, dim3(256), 0, st, kb, L, ldl, Wb, ldw, inv, ldi, s1,
                           s2, lds_scr, Lnext, nj, slot, sg, ldsg);
        CHOL_LAUNCH_CHECK();
    }
    return CHOL_OK;
}

// Below this many trailing rows the sum of a tile column's second term and
// its panel adjoint run on the chain stream (the symmetric product beside a
// tile adjoint is then shorter than the chain, about 90 us at 3840 rows).
constexpr int64_t ADJ_CHAIN_PANEL_ROWS = 3840;
// adj_L is copied into the running gradient as the last ADJ_COPY_FIRST tile
// columns up front and the rest in bands of ADJ_COPY_BAND tile columns
constexpr int64_t ADJ_COPY_FIRST = 8, ADJ_COPY_BAND = 4;
// tile columns of the gradient added into adj_A per iteration, beyond its own,
// once the chain no longer sets the pace
constexpr int64_t ADJ_ADD_CATCHUP = 2;

// Reverse sweep over the tile columns with depth-1 look-ahead.  Tile column
// j's adjoint of the trailing update, Wb_panel(j) -= Sym(Wb22(j)) L_panel(j),
// with Wb22(j) starting at tile column k = j+1, is split as
//   Sym(Wb22(j)) without its leading block Wb_kk:  available once the
//                 panel-solve adjoint of tile column k has produced
//                 X(k) = Wb_panel(k) (the rest of Wb22(k) is final by then);
//   Sym(G(k)) L[tile k, tile j]:  needs the tile adjoint G(k) = the final Wb_kk.
// The wide stream sx runs, per tile column k: the reduction that adds the
// second term of tile column k (from tile column k+1's tile adjoint), the
// panel-solve adjoint X(k) = Wb_panel(k) Linv_k, and then the first term of
// tile column k-1 as one symmetric product, while the chain stream sc runs
// the tile-sized product Wb_kk -= tril(X^T L_panel) and the tile adjoint G(k),
// ending with the second term of tile column k-1.
template <typename T>
static chol_status blocked_adjoint_on(int64_t n, const T *L, int64_t ldl, const T *adjL, int64_t ldal, T *adjA,
                                      int64_t ldaa, int accumulate, int nb, void *ws, int max_splits,
                                      hipStream_t sc, hipStream_t sx, hipEvent_t e_tile, hipEvent_t e_wide,
                                      int *sched_x, int cap_x)
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
    T *part_x = (T *)w;
    w += align256((size_t)max_splits * n * nb * sizeof(T));
    T *part_b = (T *)w;
    w += align256((size_t)(panel_tiles(n) + 1) * nb * nb * sizeof(T));
    T *part_c = (T *)w;
    w += align256((size_t)2 * nb * nb * sizeof(T));
    // dense Sym(G) per diagonal tile: the symmetric products read their
    // diagonal blocks from it when the tile is the product's 128-wide tile
    T *dense = nb == 128 ? (T *)w : nullptr;
    T *slot = part_b + panel_tiles(n) * nb * nb;   // Sym(G(k)) L[tile k, tile k-1]

    // adj_L into the running gradient: the last ADJ_COPY_FIRST tile columns
    // (all that the first iterations touch) now, the others in bands of
    // ADJ_COPY_BAND tile columns on sx during the first iterations, where sx
    // waits for the chain; each band ahead of the iteration that first uses it
    const bool copy = (const T *)Wb != adjL;
    const int64_t kc = copy ? std::max<int64_t>(0, K - ADJ_COPY_FIRST) : 0;
    if (copy) {
        const int64_t c0 = kc * nb;
        if ((s = tri_op<T, TRI_COPY_LOWER>(n - c0, adjL + c0 * ldal + c0, ldal, Wb + c0 * ldw + c0, ldw, sx)) !=
            CHOL_OK)
            return s;
    }
    {
        prof::Scope ps(CHOL_K_DIAG_INVERSE, sx, (double)K * nb * nb * nb / 3);
        hipLaunchKernelGGL((k_trinv<T>), dim3((unsigned)K), dim3(256), 0, sx, n, nb, (int64_t)0, (int64_t)nb,
                           const_cast<T *>(L), ldl, 1, inv, (int64_t)nb * nb, (int64_t)nb);
        CHOL_LAUNCH_CHECK();
    }

    // tile columns [add_lo, add_hi) are final and not yet added into adj_A
    int64_t add_lo = K, add_hi = K;
    // partials of the last symmetric product not yet summed into the next
    // tile column's panel
    Partials<T> pend{};
    auto add_columns = [&](int64_t lo, int64_t hi) {
        const int64_t c0 = lo * nb;
        return tri_op<T, TRI_ADD_LOWER>(n - c0, Wb + c0 * ldw + c0, ldw, adjA + c0 * ldaa + c0, ldaa, sc,
                                        (hi - lo) * nb);
    };

    for (int64_t k = K - 1; k >= 0; --k) {
        const int64_t k0 = k * nb;
        const int kb = (int)std::min<int64_t>(nb, n - k0);
        const int64_t r0 = k0 + kb, m = n - r0;
        const int kn = (int)std::min<int64_t>(nb, m);
        const T *Lkk = L + k0 * ldl + k0;
        T *Wkk = Wb + k0 * ldw + k0;
        const T *invk = inv + k * nb * nb;
        const T *Lp = L + r0 * ldl + k0;       // L_panel, m x kb
        T *Wp = Wb + r0 * ldw + k0;            // Wb_panel, m x kb
        // Where the trailing block is short, the chain of tile adjoints paces
        // the sweep: the two launches that start tile column k (the sum of its
        // second term and the panel adjoint) then run on sc as well, so the
        // chain goes from one tile adjoint to the next with no wait on sx in
        // between (what they need from sx, the symmetric product of tile
        // column k, ran beside the previous tile adjoint and is long done).
        // Further on, sx's symmetric products are the longer path and the two
        // launches stay on sx, where they follow the product directly.
        const bool on_chain = m <= ADJ_CHAIN_PANEL_ROWS;
        hipStream_t sp = on_chain ? sc : sx;
        // on sc, these launches need everything sx has done so far (the copy of
        // adj_L, the tile inverses, the symmetric product of this tile column);
        // on sx, the second term from tile column k+1's tile adjoint on sc
        if (on_chain || m > 0) {
            if (stream_join(on_chain ? sc : sx, on_chain ? sx : sc, e_tile) != hipSuccess)
                return CHOL_ERR_HIP;
        }
        // the next band of adj_L (tile columns [lo, hi)), first used at
        // iteration hi - 1 < k
        if (const int64_t q = K - 1 - k; copy && q * ADJ_COPY_BAND < kc) {
            const int64_t hi = kc - q * ADJ_COPY_BAND, lo = std::max<int64_t>(0, hi - ADJ_COPY_BAND);
            const int64_t c0 = lo * nb;
            if ((s = tri_op<T, TRI_COPY_LOWER>(n - c0, adjL + c0 * ldal + c0, ldal, Wb + c0 * ldw + c0, ldw, sx,
                                               (hi - lo) * nb)) != CHOL_OK)
                return s;
        }
        if (m > 0) {
            // the second term of this tile column lands in the first kn rows
            // of Wb_panel, in the same pass as the sum of the first term's
            // partials when the symmetric product left it (where this tile
            // column's panel adjoint runs on sx, right after that product)
            if (pend.part) {
                if ((s = splitk_reduce<T>((int)m, kb, pend, (const T *)slot, kn, Wp, ldw, sp)) != CHOL_OK)
                    return s;
            } else if ((s = splitk_reduce<T>(kn, kb, Partials<T>{}, (const T *)slot, kn, Wp, ldw, sp)) != CHOL_OK) {
                return s;
            }
            pend = Partials<T>{};
            // R2a: X = Wb_panel L_kk^{-1} (in place, full panel width per block,
            // 32-row tiles; the stored inverse carries its zeros, so it is a
            // plain operand)
            {
                GemmArgs<T> p{};
                p.M = (int)m; p.N = kb; p.K = kb;
                p.a = Wp; p.lda = ldw;
                p.b = invk; p.ldb = nb;
                p.c = Wp; p.ldc = ldw;
                prof::Scope ps(CHOL_K_ADJ_PANEL, sp, (double)m * kb * kb);
                if ((s = gemm<T, OP_MK, OP_KM, C_STORE, 32>(p, 1, sp)) != CHOL_OK)
                    return s;
            }
        }
        // from here on sc: R2b (it only feeds the tile adjoint), then the tile
        // adjoint of tile column k, whose last stage is the second term of
        // tile column k-1; meanwhile sx goes on with the symmetric product,
        // which needs the panel adjoint
        const int64_t j0 = k0 - nb;                 // previous tile column (if k >= 1)
        if (stream_join(on_chain ? sx : sc, on_chain ? sc : sx, e_wide) != hipSuccess)
            return CHOL_ERR_HIP;
        if (m > 0) {
            // R2b: Wb_kk -= tril(X^T L_panel), split over the m rows into
            // 128-row chunks, the partials summed in chunk order
            GemmArgs<T> p{};
            p.M = kb; p.N = kb; p.K = (int)m;
            p.a = Wp; p.lda = ldw;
            p.b = Lp; p.ldb = ldl;
            p.kchunk = 128;
            p.part = part_b;
            const int splits = (int)((m + 127) / 128);
            {
                prof::Scope ps(CHOL_K_ADJ_DIAG_UPDATE, sc, 2.0 * m * kb * kb);
                // on the critical chain (short trailing block) as 64 x 64
                // tiles, four times the blocks; beside the large symmetric
                // products the 128 x 128 tiles, which leave them the CUs
                s = on_chain ? gemm<T, OP_KM, OP_KM, C_PARTIAL, 64, 64>(p, splits, sc)
                             : gemm<T, OP_KM, OP_KM, C_PARTIAL>(p, splits, sc);
                if (s != CHOL_OK)
                    return s;
            }
            const int64_t tot = (int64_t)kb * kb;
            prof::Scope ps(CHOL_K_REDUCE, sc, (double)tot * (splits + 2) * sizeof(T));
            hipLaunchKernelGGL((k_splitk_reduce_lower<T>), dim3((unsigned)((tot + 63) / 64)), dim3(256),
                               0, sc, kb, splits, (const T *)part_b, Wkk, ldw);
            CHOL_LAUNCH_CHECK();
        }
        {
            prof::Scope ps(CHOL_K_ADJ_DIAG, sc, 2.0 * kb * kb * kb / 3 + (k >= 1 ? 2.0 * kb * kb * nb : 0.0));
            const T *Lnext = (k >= 1) ? L + k0 * ldl + j0 : nullptr;
            T *sg = dense ? dense + k * nb * nb : part_c;
            if ((s = tile_adjoint_stages<T>(sc, kb, Lkk, ldl, Wkk, ldw, invk, (int64_t)nb, part_c,
                                            part_c + (int64_t)nb * nb, (int64_t)nb, Lnext, nb,
                                            k >= 1 ? slot : (T *)nullptr, sg, (int64_t)nb)) != CHOL_OK)
                return s;
        }
        // tile column k of the gradient is final (its panel since the panel
        // adjoint, its diagonal tile since the tile adjoint): lower(adj_A) +=
        // it, on sc.  Where sc carries the chain the columns wait; once the
        // products are large, sc waits for sx and has the time: there it adds
        // its own tile column and up to ADJ_ADD_CATCHUP waiting ones.
        if (need_wb) {
            if (on_chain) {
                add_lo = k;
            } else {
                if ((s = add_columns(k, k + 1)) != CHOL_OK)
                    return s;
                const int64_t lo = std::max(add_lo, add_hi - ADJ_ADD_CATCHUP);
                if (lo < add_hi && (s = add_columns(lo, add_hi)) != CHOL_OK)
                    return s;
                add_hi = lo;
            }
        }
        // first term of tile column k-1: rows and columns from tile column k on,
        // the block Wb_kk left out
        if (k >= 1 && m > 0) {
            const double flops = 2.0 * nb * ((double)(m + kb) * (m + kb) - (double)kb * kb);
            const T *dg = dense ? dense + k * nb * nb : nullptr;   // diagonal tiles from tile k on
            // the sum of its partials waits for tile column k-1's second term
            // where that column's panel adjoint runs on sx
            const bool next_on_chain = m + nb <= ADJ_CHAIN_PANEL_ROWS;
            if ((s = sym_product<T>((int)(m + kb), nb, (int)(m + kb), Wkk, ldw, L + k0 * ldl + j0, ldl,
                                    Wb + k0 * ldw + j0, ldw, kb, dg, part_x, max_splits, 128, sched_x,
                                    cap_x, flops, sx, next_on_chain ? nullptr : &pend)) != CHOL_OK)
                return s;
        }
    }
    if (need_wb && add_lo < add_hi && (s = add_columns(add_lo, add_hi)) != CHOL_OK)
        return s;
    if (stream_join(sx, sc, e_tile) != hipSuccess)
        return CHOL_ERR_HIP;
    return CHOL_OK;
}

template <typename T>
chol_status blocked_adjoint(int64_t n, const T *L, int64_t ldl, const T *adjL, int64_t ldal, T *adjA,
                            int64_t ldaa, int accumulate, int nb, void *ws, hipStream_t st)
{
    Side *sd = side_resources();
    if (!sd)
        return CHOL_ERR_HIP;
    std::lock_guard<std::mutex> lk(sd->mu);
    if (stream_join(sd->chain, st, sd->ev[2]) != hipSuccess || stream_join(sd->x, st, sd->ev[2]) != hipSuccess ||
        zero_ints(sd->sched, SCHED_INTS, sd->x) != hipSuccess)
        return CHOL_ERR_HIP;
    const chol_status s = blocked_adjoint_on<T>(n, L, ldl, adjL, ldal, adjA, ldaa, accumulate, nb, ws,
                                                SIDE_SPLIT_MAX, sd->chain, sd->x, sd->ev[0], sd->ev[1], sd->sched,
                                                2 * sd->wide_cus);
    const bool joined = stream_join(sd->chain, sd->x, sd->ev[3]) == hipSuccess &&
                        stream_join(st, sd->chain, sd->ev[4]) == hipSuccess;
    if (s != CHOL_OK)
        return s;
    return joined ? CHOL_OK : CHOL_ERR_HIP;
}

size_t blocked_adjoint_workspace(int64_t n, int nb, size_t esize, bool need_wb)
{
    return blocked_adjoint_workspace(n, nb, esize, need_wb, SIDE_SPLIT_MAX);
}

// The adjoint on the caller's stream alone, with a caller-given workspace of
// blocked_adjoint_workspace(n, nb, es, accumulate, NOALLOC_SPLIT_MAX) bytes
// and its own work-counter slot: no library stream, event or allocation is
// involved (the entry point for callers that cannot allocate).
template <typename T>
chol_status blocked_adjoint_single_stream(int64_t n, const T *L, int64_t ldl, const T *adjL, int64_t ldal, T *adjA,
                                          int64_t ldaa, int accumulate, int nb, void *ws, int *sched, int cus,
                                          hipStream_t st)
{
    if (zero_ints(sched, 2, st) != hipSuccess)
        return CHOL_ERR_HIP;
    return blocked_adjoint_on<T>(n, L, ldl, adjL, ldal, adjA, ldaa, accumulate, nb, ws, NOALLOC_SPLIT_MAX, st, st,
                                 nullptr, nullptr, sched, 2 * cus);
}

// Loads this file's kernels on the current device (their code object is
// otherwise loaded on first launch).

// --------------------------------------------------------------- solve ----
// X = (L L^T)^{-1} B for n > CHOL_SMALL_MAX_N: the two triangular solves
// against L, tile by tile, each diagonal block applied as a product with its
// stored inverse (all K inverses are formed first, one block per tile, into
// the caller's workspace) and each off-diagonal block as an update:
//   forward  (k = 0 .. K-1):   X_k = Linv_kk X_k ;   X[r0:] -= L[r0:, k] X_k
//   backward (k = K-1 .. 0):   X_k = Linv_kk^T X_k ; X[:k0] -= L[k, :k0]^T X_k
// X_k = Linv X_k runs in place: its product has one 128-row tile row, and a
// block reads its 128-column span of X_k whole before it writes that span.

// rows x cols copy of a row-major block (leading dimensions lds, ldd)
template <typename T>
__global__ void __launch_bounds__(256)
k_copy2d(int64_t rows, int64_t cols, const T *src, int64_t lds, T *dst, int64_t ldd)
{
    const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (idx >= rows * cols)
        return;
    const int64_t r = idx / cols, c = idx % cols;
    dst[r * ldd + c] = src[r * lds + c];
}

template <typename T>
static chol_status copy2d(int64_t rows, int64_t cols, const T *src, int64_t lds, T *dst, int64_t ldd, hipStream_t st)
{
    const int64_t tot = rows * cols;
    if (tot <= 0)
        return CHOL_OK;
    hipLaunchKernelGGL((k_copy2d<T>), dim3((unsigned)((tot + 255) / 256)), dim3(256), 0, st, rows, cols, src, lds,
                       dst, ldd);
    CHOL_LAUNCH_CHECK();
    return CHOL_OK;
}

// C (M x N, leading dimension ldc) = sum of the split partials, in split order
template <typename T>
__global__ void __launch_bounds__(256)
k_splitk_sum(int M, int N, int splits, const T *part, T *c, int64_t ldc)
{
    const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
    const int64_t tot = (int64_t)M * N;
    if (idx >= tot)
        return;
    const int r = (int)(idx / N), col = (int)(idx % N);
    T s = T(0);
    for (int q = 0; q < splits; ++q)
        s += part[(int64_t)q * tot + idx];
    c[(int64_t)r * ldc + col] = s;
}

static int64_t solve_tiles(int64_t n, int nb) { return (n + nb - 1) / nb; }

// The solve's per-tile products for few right-hand sides (nrhs <= SK_N):
// C (M x N) = or -= A (M x K) B (K x N) with K <= 128 (one tile).  With N
// small each product is short, and the matrix-core loop, which has one
// 16-deep chunk in flight at a time, would wait for memory once per chunk;
// here a block loads its whole 32-row slab of A and all of B into LDS with
// one wait, then forms its outputs on the vector ALUs.  A is row-major
// (A_KM = 0: A(m, t) = a[m * lda + t]) or k-major (A_KM = 1: a[t * lda + m]).
constexpr int SK_ROWS = 32, SK_K = 128, SK_N = 64;
template <typename T, int A_KM, bool SUB>
__global__ void __launch_bounds__(256)
k_solve_skinny(int M, int N, int K, const T *a, int64_t lda, const T *b, int64_t ldb, T *c, int64_t ldc)
{
    __shared__ T sa[SK_ROWS * (SK_K + 1)];
    __shared__ T sb[SK_K * SK_N];
    const int r0 = blockIdx.x * SK_ROWS, c0 = blockIdx.y * SK_N;
    const int rows = min(SK_ROWS, M - r0), cols = min(SK_N, N - c0);
    const int tid = threadIdx.x;
    // every load of the thread is issued before the first LDS write, so the
    // block waits for memory once
    constexpr int PA = SK_ROWS * SK_K / 256, PB = SK_K * SK_N / 256;
    T va[PA], vb[PB];
#pragma unroll
    for (int q = 0; q < PA; ++q) {
        const int e = tid + 256 * q;
        const int i = A_KM ? e % SK_ROWS : e / SK_K, t = A_KM ? e / SK_ROWS : e % SK_K;
        va[q] = T(0);
        if (i < rows && t < K)
            va[q] = A_KM ? a[(int64_t)t * lda + r0 + i] : a[(int64_t)(r0 + i) * lda + t];
    }
#pragma unroll
    for (int q = 0; q < PB; ++q) {
        const int e = tid + 256 * q, t = e / SK_N, j = e % SK_N;
        vb[q] = (j < cols && t < K) ? b[(int64_t)t * ldb + c0 + j] : T(0);
    }
#pragma unroll
    for (int q = 0; q < PA; ++q) {
        const int e = tid + 256 * q;
        const int i = A_KM ? e % SK_ROWS : e / SK_K, t = A_KM ? e / SK_ROWS : e % SK_K;
        sa[i * (SK_K + 1) + t] = va[q];
    }
#pragma unroll
    for (int q = 0; q < PB; ++q)
        sb[tid + 256 * q] = vb[q];
    __syncthreads();
    for (int o = tid; o < rows * cols; o += 256) {
        const int i = o / cols, j = o % cols;
        const T *ai = sa + i * (SK_K + 1);
        T acc0 = T(0), acc1 = T(0), acc2 = T(0), acc3 = T(0);
        int t = 0;
        for (; t + 4 <= K; t += 4) {
            acc0 += ai[t] * sb[t * SK_N + j];
            acc1 += ai[t + 1] * sb[(t + 1) * SK_N + j];
            acc2 += ai[t + 2] * sb[(t + 2) * SK_N + j];
            acc3 += ai[t + 3] * sb[(t + 3) * SK_N + j];
        }
        for (; t < K; ++t)
            acc0 += ai[t] * sb[t * SK_N + j];
        const T acc = (acc0 + acc1) + (acc2 + acc3);
        T *dst = c + (int64_t)(r0 + i) * ldc + c0 + j;
        if (SUB)
            *dst -= acc;
        else
            *dst = acc;
    }
}

template <typename T, int A_KM, bool SUB>
static chol_status solve_skinny(int M, int N, int K, const T *a, int64_t lda, const T *b, int64_t ldb, T *c,
                                int64_t ldc, hipStream_t st)
{
    if (M <= 0 || N <= 0)
        return CHOL_OK;
    if (K > SK_K)
        return CHOL_ERR_INVALID_VALUE;
    const dim3 grid((unsigned)((M + SK_ROWS - 1) / SK_ROWS), (unsigned)((N + SK_N - 1) / SK_N));
    hipLaunchKernelGGL((k_solve_skinny<T, A_KM, SUB>), grid, dim3(256), 0, st, M, N, K, a, lda, b, ldb, c, ldc);
    CHOL_LAUNCH_CHECK();
    return CHOL_OK;
}

// Few right-hand sides: both sweeps with the short products above, out of
// place so that no product reads what another block of it writes.  The
// forward sweep leaves Y = L^{-1} X (tile k: Y_k = Linv_kk X_k, then
// X[r0:] -= L[r0:, k] Y_k); the backward sweep writes the solution into X
// (X_k = Linv_kk^T Y_k, then Y[:k0] -= L[k, :k0]^T X_k).
template <typename T>
static chol_status blocked_solve_skinny(int64_t n, int64_t nrhs, const T *L, int64_t ldl, T *X, int64_t ldx, int nb,
                                        const T *inv, T *Y, hipStream_t st)
{
    const int64_t K = solve_tiles(n, nb);
    const int N = (int)nrhs;
    chol_status s;
    for (int64_t k = 0; k < K; ++k) {
        const int64_t k0 = k * nb;
        const int kb = (int)std::min<int64_t>(nb, n - k0);
        const int64_t r0 = k0 + kb;
        const T *invk = inv + k * (int64_t)nb * nb;
        if ((s = solve_skinny<T, 0, false>(kb, N, kb, invk, nb, X + k0 * ldx, ldx, Y + k0 * nrhs, nrhs, st)) != CHOL_OK)
            return s;
        if ((s = solve_skinny<T, 0, true>((int)(n - r0), N, kb, L + r0 * ldl + k0, ldl, Y + k0 * nrhs, nrhs,
                                          X + r0 * ldx, ldx, st)) != CHOL_OK)
            return s;
    }
    for (int64_t k = K - 1; k >= 0; --k) {
        const int64_t k0 = k * nb;
        const int kb = (int)std::min<int64_t>(nb, n - k0);
        const T *invk = inv + k * (int64_t)nb * nb;
        if ((s = solve_skinny<T, 1, false>(kb, N, kb, invk, nb, Y + k0 * nrhs, nrhs, X + k0 * ldx, ldx, st)) != CHOL_OK)
            return s;
        if ((s = solve_skinny<T, 1, true>((int)k0, N, kb, L + k0 * ldl, ldl, X + k0 * ldx, ldx, Y, nrhs, st)) !=
            CHOL_OK)
            return s;
    }
    return CHOL_OK;
}

template <typename T>
static chol_status blocked_solve_on(int64_t n, int64_t nrhs, const T *L, int64_t ldl, T *X, int64_t ldx, int nb,
                                    const T *inv, hipStream_t st)
{
    const int64_t K = solve_tiles(n, nb);
    chol_status s;
    for (int pass = 0; pass < 2; ++pass) {
        const bool back = pass == 1;
        for (int64_t q = 0; q < K; ++q) {
            const int64_t k = back ? K - 1 - q : q;
            const int64_t k0 = k * nb;
            const int kb = (int)std::min<int64_t>(nb, n - k0);
            const int64_t r0 = k0 + kb;
            {
                // X_k = Linv_kk X_k (forward) or Linv_kk^T X_k (backward), in place
                GemmArgs<T> p{};
                p.M = kb; p.N = (int)nrhs; p.K = kb;
                p.a = inv + k * (int64_t)nb * nb; p.lda = nb;
                p.b = X + k0 * ldx; p.ldb = ldx;
                p.c = X + k0 * ldx; p.ldc = ldx;
                s = back ? gemm<T, OP_KM, OP_KM, C_STORE>(p, 1, st) : gemm<T, OP_MK, OP_KM, C_STORE>(p, 1, st);
                if (s != CHOL_OK)
                    return s;
            }
            const int64_t m = back ? k0 : n - r0;
            if (m == 0)
                continue;
            GemmArgs<T> p{};
            p.M = (int)m; p.N = (int)nrhs; p.K = kb;
            p.b = X + k0 * ldx; p.ldb = ldx;
            p.lda = ldl;
            if (back) {
                // X[:k0] -= L[k, :k0]^T X_k : A(m, t) = L[k0 + t][m]
                p.a = L + k0 * ldl;
                p.c = X; p.ldc = ldx;
                s = gemm<T, OP_KM, OP_KM, C_SUB, 64>(p, 1, st);
            } else {
                // X[r0:] -= L[r0:, k] X_k : A(m, t) = L[r0 + m][k0 + t]
                p.a = L + r0 * ldl + k0;
                p.c = X + r0 * ldx; p.ldc = ldx;
                s = gemm<T, OP_MK, OP_KM, C_SUB, 64>(p, 1, st);
            }
            if (s != CHOL_OK)
                return s;
        }
    }
    return CHOL_OK;
}

template <typename T>
static chol_status solve_inverses(int64_t n, const T *L, int64_t ldl, int nb, T *inv, hipStream_t st)
{
    const int64_t K = solve_tiles(n, nb);
    hipLaunchKernelGGL((k_trinv<T>), dim3((unsigned)K), dim3(256), 0, st, n, nb, (int64_t)0, (int64_t)nb,
                       const_cast<T *>(L), ldl, 1, inv, (int64_t)nb * nb, (int64_t)nb);
    CHOL_LAUNCH_CHECK();
    return CHOL_OK;
}

// split count of the adjoint's products P = [S|X]^T L (2 nrhs x n, n deep):
// enough (row tile, column tile, split) items for the device's block slots
static int solve_adj_splits(int64_t n, int64_t nrhs)
{
    const int64_t tiles = ((2 * nrhs + 127) / 128) * ((n + 127) / 128);
    const int64_t want = (480 + tiles - 1) / tiles;
    return (int)std::max<int64_t>(1, std::min<int64_t>(32, std::min<int64_t>(want, n / 256 + 1)));
}

// tile inverses, then (few right-hand sides) the forward sweep's n x nrhs result
size_t blocked_solve_workspace(int64_t n, int64_t nrhs, int nb, size_t es)
{
    size_t bytes = align256((size_t)solve_tiles(n, nb) * nb * nb * es);
    if (nrhs <= SK_N)
        bytes += align256((size_t)n * nrhs * es);
    return bytes;
}

template <typename T>
static chol_status solve_sweeps(int64_t n, int64_t nrhs, const T *L, int64_t ldl, T *X, int64_t ldx, int nb,
                                void *ws, hipStream_t st)
{
    const T *inv = (const T *)ws;
    if (nrhs <= SK_N) {
        T *Y = (T *)((char *)ws + align256((size_t)solve_tiles(n, nb) * nb * nb * sizeof(T)));
        return blocked_solve_skinny<T>(n, nrhs, L, ldl, X, ldx, nb, inv, Y, st);
    }
    return blocked_solve_on<T>(n, nrhs, L, ldl, X, ldx, nb, inv, st);
}

size_t blocked_solve_adjoint_workspace(int64_t n, int64_t nrhs, int nb, size_t es)
{
    const int sp = solve_adj_splits(n, nrhs);
    return blocked_solve_workspace(n, nrhs, nb, es) + 2 * align256((size_t)n * 2 * nrhs * es) +
           align256((size_t)2 * nrhs * n * es) + (sp > 1 ? align256((size_t)sp * 2 * nrhs * n * es) : 0);
}

template <typename T>
chol_status blocked_potrs(int64_t n, int64_t nrhs, const T *L, int64_t ldl, const T *B, int64_t ldb, T *X,
                          int64_t ldx, int nb, void *ws, hipStream_t st)
{
    T *inv = (T *)ws;
    prof::Scope ps(CHOL_K_SOLVE, st, 2.0 * n * n * nrhs);
    chol_status s = solve_inverses<T>(n, L, ldl, nb, inv, st);
    if (s == CHOL_OK && X != B)
        s = copy2d<T>(n, nrhs, B, ldb, X, ldx, st);
    if (s != CHOL_OK)
        return s;
    return solve_sweeps<T>(n, nrhs, L, ldl, X, ldx, nb, ws, st);
}

// adj_B = (L L^T)^{-1} adj_X; lower(adj_L) (+)= -tril((adj_B X^T + X adj_B^T) L).
// With S = adj_B, [S|X]^T L = [Q; P] (Q = S^T L, P = X^T L, L read as its
// lower triangle), and S P + X Q = [X|S] [Q; P], so the gradient is one
// lower-only product of depth 2 nrhs.
template <typename T>
chol_status blocked_potrs_adjoint(int64_t n, int64_t nrhs, const T *L, int64_t ldl, const T *X, int64_t ldx,
                                  const T *adjX, int64_t ldax, T *adjB, int64_t ldab, T *adjL, int64_t ldal,
                                  int accumulate, int nb, void *ws, hipStream_t st)
{
    char *w = (char *)ws;
    T *inv = (T *)w;
    void *solve_ws = w;
    w += blocked_solve_workspace(n, nrhs, nb, sizeof(T));
    T *sx = (T *)w;                       // [S | X], n x 2 nrhs
    w += align256((size_t)n * 2 * nrhs * sizeof(T));
    T *xs = (T *)w;                       // [X | S]
    w += align256((size_t)n * 2 * nrhs * sizeof(T));
    T *qp = (T *)w;                       // [Q; P], 2 nrhs x n
    w += align256((size_t)2 * nrhs * n * sizeof(T));
    T *part = (T *)w;
    const int sp = solve_adj_splits(n, nrhs);

    chol_status s;
    {
        prof::Scope ps(CHOL_K_SOLVE, st, 2.0 * n * n * nrhs);
        s = solve_inverses<T>(n, L, ldl, nb, inv, st);
        if (s == CHOL_OK && adjB != adjX)
            s = copy2d<T>(n, nrhs, adjX, ldax, adjB, ldab, st);
        if (s == CHOL_OK)
            s = solve_sweeps<T>(n, nrhs, L, ldl, adjB, ldab, nb, solve_ws, st);
    }
    prof::Scope ps(CHOL_K_SOLVE_ADJOINT, st, 4.0 * n * n * nrhs);
    if (s == CHOL_OK)
        s = copy2d<T>(n, nrhs, adjB, ldab, sx, 2 * nrhs, st);
    if (s == CHOL_OK)
        s = copy2d<T>(n, nrhs, X, ldx, sx + nrhs, 2 * nrhs, st);
    if (s == CHOL_OK)
        s = copy2d<T>(n, nrhs, X, ldx, xs, 2 * nrhs, st);
    if (s == CHOL_OK)
        s = copy2d<T>(n, nrhs, adjB, ldab, xs + nrhs, 2 * nrhs, st);
    if (s != CHOL_OK)
        return s;
    {
        // [Q; P] = [S|X]^T L: A(m, t) = sx[t][m], B(m = j, t) = L[t][j] for t >= j
        GemmArgs<T> p{};
        p.M = (int)(2 * nrhs); p.N = (int)n; p.K = (int)n;
        p.a = sx; p.lda = 2 * nrhs;
        p.b = L; p.ldb = ldl;
        if (sp > 1) {
            p.part = part;
            p.kchunk = split_chunk(n, sp);
            const int used = (int)((n + p.kchunk - 1) / p.kchunk);
            s = gemm<T, OP_KM, OP_KM_LOWER, C_PARTIAL>(p, used, st);
            if (s != CHOL_OK)
                return s;
            const int64_t tot = 2 * nrhs * n;
            hipLaunchKernelGGL((k_splitk_sum<T>), dim3((unsigned)((tot + 255) / 256)), dim3(256), 0, st,
                               (int)(2 * nrhs), (int)n, used, (const T *)part, qp, n);
            CHOL_LAUNCH_CHECK();
        } else {
            p.c = qp; p.ldc = n;
            s = gemm<T, OP_KM, OP_KM_LOWER, C_STORE>(p, 1, st);
            if (s != CHOL_OK)
                return s;
        }
    }
    if (!accumulate && (s = tri_op<T, TRI_ZERO_LOWER>(n, nullptr, 0, adjL, ldal, st)) != CHOL_OK)
        return s;
    // lower(adj_L) -= [X|S] [Q; P]: A(i, t) = xs[i][t], B(m = j, t) = qp[t][j]
    GemmArgs<T> p{};
    p.M = (int)n; p.N = (int)n; p.K = (int)(2 * nrhs);
    p.a = xs; p.lda = 2 * nrhs;
    p.b = qp; p.ldb = n;
    p.c = adjL; p.ldc = ldal;
    return gemm<T, OP_MK, OP_KM, C_SUB_LOWER>(p, 1, st);
}

chol_status blocked_load()
{
    hipFuncAttributes a;
    if (hip_failed(hipFuncGetAttributes(&a, reinterpret_cast<const void *>(&k_tri<double, TRI_COPY_LOWER>))))
        return CHOL_ERR_HIP;
    return CHOL_OK;
}

#define CHOL_INST(T)                                                                                     \
    template chol_status blocked_potrf<T>(int64_t, const T *, int64_t, T *, int64_t, int32_t *, int,     \
                                          hipStream_t);                                                  \
    template chol_status blocked_adjoint<T>(int64_t, const T *, int64_t, const T *, int64_t, T *, int64_t, \
                                            int, int, void *, hipStream_t);                              \
    template chol_status blocked_adjoint_single_stream<T>(int64_t, const T *, int64_t, const T *, int64_t, T *, \
                                                          int64_t, int, int, void *, int *, int, hipStream_t); \
    template chol_status blocked_potrs<T>(int64_t, int64_t, const T *, int64_t, const T *, int64_t, T *, int64_t, \
                                          int, void *, hipStream_t);                                     \
    template chol_status blocked_potrs_adjoint<T>(int64_t, int64_t, const T *, int64_t, const T *, int64_t,     \
                                                  const T *, int64_t, T *, int64_t, T *, int64_t, int, int,     \
                                                  void *, hipStream_t);
CHOL_INST(float)
CHOL_INST(double)
#undef CHOL_INST

} // namespace chol
