// Matrix-core product used by the blocked factor and adjoint:
//     C (M x N) op= A (M x K) * B (K x N)
// with each operand described by how its tile sits in memory.  Both operands
// are indexed (m, k): m runs along the output (rows of C for A, columns of C
// for B), k along the contraction.
//
//   OP_MK    element (m, k) at p[m * ld + k]   (rows of a row-major panel)
//   OP_KM    element (m, k) at p[k * ld + m]
//   OP_SYM   symmetric matrix stored as its lower triangle: (m, k) is
//            p[m][k] below the diagonal, p[k][m] above, 2 p[m][m] on it
//            (the adjoint of a lower-triangle-only trailing update reads the
//            gradient this way)
//   OP_KM_LOWER  OP_KM with entries k < m replaced by 0
//
// Design for gfx950: a 256-thread block computes a 128 x 128 tile as 2 x 2
// wavefronts of 64 x 64, each a 4 x 4 grid of 16x16x4 MFMA steps.  K advances
// in chunks of 16 staged in LDS k-major (S[k][m]) and double-buffered; the next
// chunk is fetched into registers with 16-byte global loads while the current
// one feeds the matrix cores (the thread-to-element maps are given at Map
// below).  Blocks are mapped to tiles so that each of the 8 XCDs receives a
// contiguous row-major range of tiles (rows of A and columns of B stay in one
// XCD's L2).
#pragma once

#include <algorithm>
#include <type_traits>

#include "common.hpp"

namespace chol {

enum { OP_MK = 0, OP_KM = 1, OP_SYM = 2, OP_KM_LOWER = 3 };
enum { C_SUB = 0,        // C -= AB
       C_SUB_LOWER = 1,  // C -= AB where row >= col
       C_STORE = 2,      // C  = AB
       C_PARTIAL = 3 };  // part[split] = AB (row-major M x N)

template <typename T> struct GemmArgs {
    int M, N, K;
    const T *a; int64_t lda;
    const T *b; int64_t ldb;
    T *c; int64_t ldc;
    int kchunk;          // split-K: contraction length per split (multiple of 16)
    T *part;             // C_PARTIAL destination, splits * M * N
    int tri;             // 1: lower-triangular tile grid (M == N)
    int vec;             // 1: 16-byte global loads are legal for both operands
    int splits;          // split count (C_PARTIAL)
    int excl;            // OP_SYM A operand: entries (m, k) with m < excl and
                         // k < excl read as zero (a block left out of the product)
    int t0, tn;          // tile window: tiles t0 .. t0 + tn - 1 of the (row-major
                         // or lower-triangular) tile grid; tn == 0: every tile
    int cap;             // persistent grid size with `sched` (0: two blocks per CU of 240)
    int *sched;          // non-null: blocks take (split, tile) items from this
                         // device counter pair (item, finished blocks), which
                         // must be zero at launch and is zero again afterwards
    const T *dg;         // OP_SYM A operand, optional: the symmetric 128 x 128
                         // diagonal blocks written whole (block I at dg + I*128*128,
                         // row-major), read on the 16-byte path instead of
                         // assembling them from the lower triangle element by element
};

namespace gemm_detail {

constexpr int BM = 128, BN = 128, BK = 16;
constexpr int NT = 256;
// LDS pitch of a k row (elements): even, so 16-byte writes stay aligned, and
// chosen so the row-panel scatter is at most 2-way bank conflicted.
template <typename T> struct Pitch;
template <> struct Pitch<double> { static constexpr int v = 130; };
template <> struct Pitch<float> { static constexpr int v = 132; };

// element (m, k) of an operand, with bounds (m < mlim, k < klim) -> 0 outside
template <typename T, int OP>
__device__ __forceinline__ T elem(const T *p, int64_t ld, int m, int k, int mlim, int klim, int excl)
{
    if (m >= mlim || k >= klim)
        return T(0);
    if (OP == OP_SYM && m < excl && k < excl)
        return T(0);
    if (OP == OP_MK)
        return p[(int64_t)m * ld + k];
    if (OP == OP_KM)
        return p[(int64_t)k * ld + m];
    if (OP == OP_KM_LOWER)
        return k >= m ? p[(int64_t)k * ld + m] : T(0);
    // OP_SYM
    if (m > k)
        return p[(int64_t)m * ld + k];
    if (m < k)
        return p[(int64_t)k * ld + m];
    return T(2) * p[(int64_t)m * ld + m];
}

// Eight elements per thread per chunk, fetched as 16-byte loads of PER
// consecutive elements.  Element j of thread t (wave w = t / 64, lane l):
//   q = j / PER (load number), e = j % PER
//   row-panel layout (LAY_MK): LPR = 16 / PER lanes cover the 16 k of one row
//       m = w * 32 + q * (64 / LPR) + l / LPR,   k = (l % LPR) * PER + e
//   k-major layout (LAY_KM): LPK = 128 / PER lanes cover the 128 m of one k row
//       k = w * 4 + q * (64 / LPK) + l / LPK,    m = (l % LPK) * PER + e
// so every load instruction reads whole 64- or 128-byte segments.
template <typename T> struct Vec8 { T v[8]; };
enum { LAY_MK = 0, LAY_KM = 1 };

// LDS pitch of a chunk staged on the 16-byte path with layout LAY.  fp64
// row-panel chunks (LAY_MK) take an odd pitch: a wave's 8-byte writes then
// fall on distinct banks in every group of 16 lanes (with the even pitch,
// lanes whose k differs by 8 collided); k-major chunks keep the even pitch
// their 16-byte writes need.
template <typename T, int LAY> struct LayPitch { static constexpr int v = Pitch<T>::v; };
template <> struct LayPitch<double, LAY_MK> { static constexpr int v = 129; };

// staging layouts an operand kind can use on the 16-byte path
constexpr bool can_lay(int op, int lay)
{
    return op == OP_SYM || (op == OP_MK ? lay == LAY_MK : lay == LAY_KM);
}

template <typename T> struct Map {
    static constexpr int PER = 16 / sizeof(T);
    static constexpr int LPR = BK / PER;        // lanes per row (row-panel)
    static constexpr int LPK = BM / PER;        // lanes per k row (k-major)
    static __device__ __forceinline__ void mk(int t, int j, int &m, int &k)
    {
        const int w = t / 64, l = t % 64, q = j / PER, e = j % PER;
        m = w * 32 + q * (64 / LPR) + l / LPR;
        k = (l % LPR) * PER + e;
    }
    static __device__ __forceinline__ void km(int t, int j, int &m, int &k)
    {
        const int w = t / 64, l = t % 64, q = j / PER, e = j % PER;
        k = w * 4 + q * (64 / LPK) + l / LPK;
        m = (l % LPK) * PER + e;
    }
};

template <typename T, int OP>
struct Operand {
    const T *p;
    int64_t ld;
    int m0;      // tile origin along m
    int mlim;    // M (or N) bound
    int vec;
    int excl;    // OP_SYM: leading excl x excl block left out

    // layout used for a chunk starting at k0 (uniform over the block)
    __device__ __forceinline__ int layout(int k0) const
    {
        if (OP == OP_MK)
            return LAY_MK;
        if (OP == OP_SYM)
            return (m0 >= k0 + BK) ? LAY_MK : LAY_KM;
        return LAY_KM;
    }
    // does the chunk need the per-element path (edges, diagonal crossing, masks)?
    __device__ __forceinline__ bool generic(int k0, int klim) const
    {
        if (!vec || m0 + BM > mlim || k0 + BK > klim)
            return true;
        if (OP == OP_SYM)
            return !(m0 >= k0 + BK || m0 + BM <= k0) || (m0 < excl && k0 < excl);
        if (OP == OP_KM_LOWER)
            return !(k0 >= m0 + BM - 1);         // plain only if every k >= every m
        return false;
    }

    // layout of the chunk at k0 if it can take the 16-byte path, else -1
    __device__ __forceinline__ int fast_lay(int k0, int klim) const
    {
        return generic(k0, klim) ? -1 : layout(k0);
    }

    // 16-byte loads of a chunk known to be on the fast path with layout LAY
    template <int LAY>
    __device__ __forceinline__ void fetch_fast(Vec8<T> &r, int tid, int k0) const
    {
        typedef Map<T> MP;
        typedef T vt __attribute__((ext_vector_type(MP::PER)));
#pragma unroll
        for (int q = 0; q < 8 / MP::PER; ++q) {
            int m, k;
            if (LAY == LAY_MK)
                MP::mk(tid, q * MP::PER, m, k);
            else
                MP::km(tid, q * MP::PER, m, k);
            const T *src = (LAY == LAY_MK) ? p + (int64_t)(m0 + m) * ld + k0 + k
                                           : p + (int64_t)(k0 + k) * ld + m0 + m;
            const vt x = *reinterpret_cast<const vt *>(src);
#pragma unroll
            for (int e = 0; e < MP::PER; ++e)
                r.v[q * MP::PER + e] = x[e];
        }
    }

    template <int LAY>
    static __device__ __forceinline__ void stash_lay(const Vec8<T> &r, T *S, int tid)
    {
        typedef Map<T> MP;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            int m, k;
            if (LAY == LAY_MK)
                MP::mk(tid, j, m, k);
            else
                MP::km(tid, j, m, k);
            S[k * LayPitch<T, LAY>::v + m] = r.v[j];
        }
    }

    __device__ __forceinline__ void fetch(Vec8<T> &r, int tid, int k0, int klim) const
    {
        typedef Map<T> MP;
        const int lay = layout(k0);
        if (!generic(k0, klim)) {
            typedef T vt __attribute__((ext_vector_type(MP::PER)));
#pragma unroll
            for (int q = 0; q < 8 / MP::PER; ++q) {
                int m, k;
                if (lay == LAY_MK)
                    MP::mk(tid, q * MP::PER, m, k);
                else
                    MP::km(tid, q * MP::PER, m, k);
                const T *src = (lay == LAY_MK) ? p + (int64_t)(m0 + m) * ld + k0 + k
                                               : p + (int64_t)(k0 + k) * ld + m0 + m;
                const vt x = *reinterpret_cast<const vt *>(src);
#pragma unroll
                for (int e = 0; e < MP::PER; ++e)
                    r.v[q * MP::PER + e] = x[e];
            }
            return;
        }
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            int m, k;
            if (lay == LAY_MK)
                MP::mk(tid, j, m, k);
            else
                MP::km(tid, j, m, k);
            r.v[j] = elem<T, OP>(p, ld, m0 + m, k0 + k, mlim, klim, excl);
        }
    }

    // per-element path straight into the LDS chunk
    __device__ __forceinline__ void put(T *S, int tid, int k0, int klim) const
    {
        typedef Map<T> MP;
        const int lay = layout(k0);
#pragma unroll 1
        for (int j = 0; j < 8; ++j) {
            int m, k;
            if (lay == LAY_MK)
                MP::mk(tid, j, m, k);
            else
                MP::km(tid, j, m, k);
            S[k * Pitch<T>::v + m] = elem<T, OP>(p, ld, m0 + m, k0 + k, mlim, klim, excl);
        }
    }

    __device__ __forceinline__ void stash(const Vec8<T> &r, T *S, int tid, int k0) const
    {
        typedef Map<T> MP;
        const int lay = layout(k0);
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            int m, k;
            if (lay == LAY_MK)
                MP::mk(tid, j, m, k);
            else
                MP::km(tid, j, m, k);
            S[k * Pitch<T>::v + m] = r.v[j];
        }
    }
};

// blockIdx.x -> tile index so that each XCD (blocks b with equal b % 8) takes a
// contiguous range of the row-major tile order.
__device__ __forceinline__ int xcd_tile(int b, int nt)
{
    const int per = nt / 8, rem = nt % 8;
    const int x = b % 8, i = b / 8;
    return x * per + (x < rem ? x : rem) + i;
}

} // namespace gemm_detail

namespace gemm_detail {

// acc += (NEG ? -A : B) over one chunk staged at SA (A, pitch PA) and SB (B,
// pitch PB) in LDS
template <typename T, bool NEG, int PA = Pitch<T>::v, int PB = Pitch<T>::v>
__device__ __forceinline__ void chunk_mma(typename Acc<T>::type (&acc)[4][4], const T *SA, const T *SB, int lane,
                                          int wm, int wn)
{
#pragma unroll
    for (int kk = 0; kk < BK; kk += 4) {
        const int kr = kk + lane / 16;
        T af[4], bf[4];
#pragma unroll
        for (int i = 0; i < 4; ++i)
            af[i] = SA[kr * PA + wm * 64 + i * 16 + lane % 16];
#pragma unroll
        for (int j = 0; j < 4; ++j)
            bf[j] = SB[kr * PB + wn * 64 + j * 16 + lane % 16];
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j)
                acc[i][j] = mfma16x16x4_s<NEG>(af[i], bf[j], acc[i][j]);
    }
}

// A run of nc >= 1 chunks starting at k0, all on the 16-byte path with fixed
// layouts.  Software pipeline: while the matrix cores work on one LDS buffer,
// the other is filled from registers loaded one chunk earlier, and the next
// chunk's loads are issued.  Every load is unconditional (indices past the run
// repeat its last chunk), so no loaded register ever merges with an older
// value and the loads stay in flight across the matrix-core work.
template <typename T, int AOP, int BOP, int LA, int LB, bool NEG>
__device__ __forceinline__ void mma_run(typename Acc<T>::type (&acc)[4][4], const Operand<T, AOP> &A,
                                        const Operand<T, BOP> &B, int k0, int nc, T *lds)
{
    constexpr int SZ = BK * Pitch<T>::v;
    const int tid = threadIdx.x, lane = tid % 64, wave = tid / 64;
    const int wm = wave / 2, wn = wave % 2;
    auto kc = [&](int c) { return k0 + (c < nc ? c : nc - 1) * BK; };
    Vec8<T> a, b;
    A.template fetch_fast<LA>(a, tid, k0);
    B.template fetch_fast<LB>(b, tid, k0);
    __syncthreads();                      // earlier users of the LDS buffers are done
    Operand<T, AOP>::template stash_lay<LA>(a, lds, tid);
    Operand<T, BOP>::template stash_lay<LB>(b, lds + SZ, tid);
    A.template fetch_fast<LA>(a, tid, kc(1));
    B.template fetch_fast<LB>(b, tid, kc(1));
    __syncthreads();
    for (int c = 0; c < nc; ++c) {
        const T *S = lds + (c & 1) * 2 * SZ;
        T *D = lds + ((c + 1) & 1) * 2 * SZ;
        chunk_mma<T, NEG, LayPitch<T, LA>::v, LayPitch<T, LB>::v>(acc, S, S + SZ, lane, wm, wn);                   // chunk c
        Operand<T, AOP>::template stash_lay<LA>(a, D, tid);                // chunk c+1
        Operand<T, BOP>::template stash_lay<LB>(b, D + SZ, tid);
        A.template fetch_fast<LA>(a, tid, kc(c + 2));
        B.template fetch_fast<LB>(b, tid, kc(c + 2));
        __syncthreads();
    }
}

// mma_run with A's loads two chunks ahead (A is the operand streamed from
// HBM; B stays one chunk ahead).  The loop takes chunks in pairs so the two A
// register sets alternate without copies; with an odd count the last pair
// skips only its second chunk's matrix-core work, and every load stays
// unconditional (indices past the run repeat its last chunk).
template <typename T, int AOP, int BOP, int LA, int LB, bool NEG>
__device__ __forceinline__ void mma_run2(typename Acc<T>::type (&acc)[4][4], const Operand<T, AOP> &A,
                                         const Operand<T, BOP> &B, int k0, int nc, T *lds)
{
    constexpr int SZ = BK * Pitch<T>::v;
    const int tid = threadIdx.x, lane = tid % 64, wave = tid / 64;
    const int wm = wave / 2, wn = wave % 2;
    auto kc = [&](int c) { return k0 + (c < nc ? c : nc - 1) * BK; };
    Vec8<T> a0, a1, b;
    A.template fetch_fast<LA>(a0, tid, k0);
    B.template fetch_fast<LB>(b, tid, k0);
    __syncthreads();                      // earlier users of the LDS buffers are done
    Operand<T, AOP>::template stash_lay<LA>(a0, lds, tid);
    Operand<T, BOP>::template stash_lay<LB>(b, lds + SZ, tid);
    A.template fetch_fast<LA>(a1, tid, kc(1));
    B.template fetch_fast<LB>(b, tid, kc(1));
    A.template fetch_fast<LA>(a0, tid, kc(2));
    __syncthreads();
    T *const L0 = lds, *const L1 = lds + 2 * SZ;
    for (int c = 0; c < nc; c += 2) {
        // chunk c from L0; chunk c+1 (a1, b) into L1; a1 <- chunk c+3
        chunk_mma<T, NEG, LayPitch<T, LA>::v, LayPitch<T, LB>::v>(acc, L0, L0 + SZ, lane, wm, wn);
        Operand<T, AOP>::template stash_lay<LA>(a1, L1, tid);
        Operand<T, BOP>::template stash_lay<LB>(b, L1 + SZ, tid);
        A.template fetch_fast<LA>(a1, tid, kc(c + 3));
        B.template fetch_fast<LB>(b, tid, kc(c + 2));
        __syncthreads();
        // chunk c+1 from L1; chunk c+2 (a0, b) into L0; a0 <- chunk c+4
        if (c + 1 < nc)
            chunk_mma<T, NEG, LayPitch<T, LA>::v, LayPitch<T, LB>::v>(acc, L1, L1 + SZ, lane, wm, wn);
        Operand<T, AOP>::template stash_lay<LA>(a0, L0, tid);
        Operand<T, BOP>::template stash_lay<LB>(b, L0 + SZ, tid);
        A.template fetch_fast<LA>(a0, tid, kc(c + 4));
        B.template fetch_fast<LB>(b, tid, kc(c + 3));
        __syncthreads();
    }
}

#ifndef CHOL_RUN_DEPTH
#define CHOL_RUN_DEPTH 2
#endif
template <typename T, int AOP, int BOP, int LA, int LB, bool NEG>
__device__ __forceinline__ void run_chunks(typename Acc<T>::type (&acc)[4][4], const Operand<T, AOP> &A,
                                           const Operand<T, BOP> &B, int k0, int nc, T *lds)
{
    if constexpr (CHOL_RUN_DEPTH == 2)
        mma_run2<T, AOP, BOP, LA, LB, NEG>(acc, A, B, k0, nc, lds);
    else
        mma_run<T, AOP, BOP, LA, LB, NEG>(acc, A, B, k0, nc, lds);
}

// The K loop through the general path, chunk by chunk, for tiles with edges,
// diagonal crossings or masks: every chunk is fetched by the path it needs
// (16-byte or per element).  A's loads run two chunks ahead, B's one.
template <typename T, int AOP, int BOP, bool NEG>
__device__ __forceinline__ void mma_general(typename Acc<T>::type (&acc)[4][4], const Operand<T, AOP> &A,
                                            const Operand<T, BOP> &B, int kbeg, int kend, T *lds)
{
    constexpr int SZ = BK * Pitch<T>::v;
    const int tid = threadIdx.x, lane = tid % 64, wave = tid / 64;
    const int wm = wave / 2, wn = wave % 2;
    Vec8<T> ra0, ra1, rb;
    __syncthreads();
    A.fetch(ra0, tid, kbeg, kend);
    B.fetch(rb, tid, kbeg, kend);
    A.stash(ra0, lds, tid, kbeg);
    B.stash(rb, lds + SZ, tid, kbeg);
    if (kbeg + BK < kend) {
        A.fetch(ra1, tid, kbeg + BK, kend);
        B.fetch(rb, tid, kbeg + BK, kend);
    }
    if (kbeg + 2 * BK < kend)
        A.fetch(ra0, tid, kbeg + 2 * BK, kend);
    __syncthreads();
    int c = 0;
    for (int k0 = kbeg; k0 < kend; k0 += BK, ++c) {
        const int buf = c & 1;
        const T *SA = lds + buf * 2 * SZ;
        chunk_mma<T, NEG>(acc, SA, SA + SZ, lane, wm, wn);
        if (k0 + BK < kend) {
            T *D = lds + (buf ^ 1) * 2 * SZ;
            B.stash(rb, D + SZ, tid, k0 + BK);
            if (k0 + 2 * BK < kend)
                B.fetch(rb, tid, k0 + 2 * BK, kend);
            // chunk c+1 of A sits in set (c+1)&1; refill that set with chunk c+3
            if ((c & 1) == 0) {
                A.stash(ra1, D, tid, k0 + BK);
                if (k0 + 3 * BK < kend)
                    A.fetch(ra1, tid, k0 + 3 * BK, kend);
            } else {
                A.stash(ra0, D, tid, k0 + BK);
                if (k0 + 3 * BK < kend)
                    A.fetch(ra0, tid, k0 + 3 * BK, kend);
            }
        }
        __syncthreads();
    }
}

} // namespace gemm_detail

// Pipelined runs over [kbeg, kend) where every chunk is on the 16-byte path
// (klim is the contraction bound the chunks are classified against): the range
// is cut where an operand's staging layout changes.
template <typename T, int AOP, int BOP, bool NEG>
__device__ __forceinline__ void tile_runs(typename Acc<T>::type (&acc)[4][4], const gemm_detail::Operand<T, AOP> &A,
                                          const gemm_detail::Operand<T, BOP> &B, int kbeg, int kend, int klim, T *lds)
{
    using namespace gemm_detail;
    int k = kbeg;
    while (k < kend) {
        const int la = A.fast_lay(k, klim), lb = B.fast_lay(k, klim);
        int nc = 1;
        while (k + nc * BK < kend && A.fast_lay(k + nc * BK, klim) == la && B.fast_lay(k + nc * BK, klim) == lb)
            ++nc;
        // only the layout pairs the operand kinds can produce are instantiated
        if constexpr (can_lay(AOP, LAY_MK) && can_lay(BOP, LAY_MK)) {
            if (la == LAY_MK && lb == LAY_MK)
                run_chunks<T, AOP, BOP, LAY_MK, LAY_MK, NEG>(acc, A, B, k, nc, lds);
        }
        if constexpr (can_lay(AOP, LAY_MK) && can_lay(BOP, LAY_KM)) {
            if (la == LAY_MK && lb == LAY_KM)
                run_chunks<T, AOP, BOP, LAY_MK, LAY_KM, NEG>(acc, A, B, k, nc, lds);
        }
        if constexpr (can_lay(AOP, LAY_KM) && can_lay(BOP, LAY_MK)) {
            if (la == LAY_KM && lb == LAY_MK)
                run_chunks<T, AOP, BOP, LAY_KM, LAY_MK, NEG>(acc, A, B, k, nc, lds);
        }
        if constexpr (can_lay(AOP, LAY_KM) && can_lay(BOP, LAY_KM)) {
            if (la == LAY_KM && lb == LAY_KM)
                run_chunks<T, AOP, BOP, LAY_KM, LAY_KM, NEG>(acc, A, B, k, nc, lds);
        }
        k += nc * BK;
    }
}

// The K loop of one 128 x 128 tile: acc += (NEG ? -A : A) B over k in
// [kbeg, kend), operands staged through `lds` (2 buffers x 2 operands x
// BK * Pitch<T>::v elements).  Called by all 256 threads of the block.  When
// every chunk can take the 16-byte path, the range is cut into runs of chunks
// on which both operands keep one layout each (pipelined); otherwise the tile
// takes the general loop.  PATH fixes at compile time which of the two the
// kernel carries (the host knows for plain operands and aligned sizes).
enum { PATH_GENERAL = 0,   // every tile through the general loop
       PATH_RUNS = 1,      // every chunk of every tile is on the 16-byte path
       PATH_MIXED = 2 };   // decided per tile

template <typename T, int AOP, int BOP, bool NEG, int PATH>
__device__ __forceinline__ void tile_mma(typename Acc<T>::type (&acc)[4][4], const gemm_detail::Operand<T, AOP> &A,
                                         const gemm_detail::Operand<T, BOP> &B, int kbeg, int kend, T *lds)
{
    using namespace gemm_detail;
    if constexpr (PATH == PATH_GENERAL) {
        mma_general<T, AOP, BOP, NEG>(acc, A, B, kbeg, kend, lds);
        return;
    }
    if constexpr (PATH == PATH_MIXED) {
        // the chunks that need the per-element path (a diagonal crossing, an
        // edge, a mask) span [g0, g1); they go through the general loop and
        // the runs of 16-byte chunks before and after stay pipelined.  The
        // three loops follow each other in straight-line code, which keeps
        // the pipelined runs as lean in registers as in a kernel without the
        // general loop.
        int g0 = kend, g1 = kend;
        for (int k = kbeg; k < kend; k += BK) {
            if (A.fast_lay(k, kend) < 0 || B.fast_lay(k, kend) < 0) {
                if (g0 == kend)
                    g0 = k;
                g1 = min(k + BK, kend);
            }
        }
        if (g0 > kbeg)
            tile_runs<T, AOP, BOP, NEG>(acc, A, B, kbeg, g0, kend, lds);
        if (g1 > g0)
            mma_general<T, AOP, BOP, NEG>(acc, A, B, g0, g1, lds);
        if (kend > g1)
            tile_runs<T, AOP, BOP, NEG>(acc, A, B, g1, kend, kend, lds);
        return;
    }
    tile_runs<T, AOP, BOP, NEG>(acc, A, B, kbeg, kend, kend, lds);
}

// Position of accumulator element (i, j, v) of this thread inside the 128 x 128 tile.
template <typename T>
__device__ __forceinline__ void acc_pos(int i, int j, int v, int &row, int &col)
{
    const int lane = threadIdx.x % 64, wave = threadIdx.x / 64;
    row = (wave / 2) * 64 + i * 16 + Acc<T>::row(lane, v);
    col = (wave % 2) * 64 + j * 16 + lane % 16;
}

// One 128 x 128 output tile (I, J) over the contraction range [kbeg, kend).
template <typename T, int AOP, int BOP, int CM, int PATH>
__device__ __forceinline__ void gemm_tile(const GemmArgs<T> &p, int I, int J, int split, int kbeg, int kend, T *lds)
{
    using namespace gemm_detail;
    typedef typename Acc<T>::type acc_t;
    const int r0 = I * BM, c0 = J * BN;

    // C -= AB runs as acc = C, acc += (-A) B: the accumulators start from C,
    // so the epilogue is a plain store and no accumulator has to leave the
    // matrix-core registers for a read-modify-write.
    constexpr bool FROM_C = (CM == C_SUB || CM == C_SUB_LOWER);
    // a tile inside M x N needs no per-entry bounds test: its loads of C and
    // its stores are issued back to back, without a branch around each one
    const bool interior = r0 + BM <= p.M && c0 + BN <= p.N;
    acc_t acc[4][4];
    if (FROM_C && interior) {
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j)
#pragma unroll
                for (int v = 0; v < 4; ++v) {
                    int row, col;
                    acc_pos<T>(i, j, v, row, col);
                    acc[i][j][v] = p.c[(int64_t)(row + r0) * p.ldc + col + c0];
                }
    } else {
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j)
#pragma unroll
                for (int v = 0; v < 4; ++v) {
                    T x = T(0);
                    if (FROM_C) {
                        int row, col;
                        acc_pos<T>(i, j, v, row, col);
                        row += r0;
                        col += c0;
                        if (row < p.M && col < p.N)
                            x = p.c[(int64_t)row * p.ldc + col];
                    }
                    acc[i][j][v] = x;
                }
    }

    Operand<T, AOP> A{p.a, p.lda, r0, p.M, p.vec, p.excl};
    Operand<T, BOP> B{p.b, p.ldb, c0, p.N, p.vec, 0};
    bool done = false;
    if constexpr (AOP == OP_SYM && BOP == OP_KM && PATH == PATH_MIXED) {
        // the tile's diagonal block [r0, r0 + 128) of the contraction, when it
        // is whole, not left out and within [kbeg, kend): a plain row panel of
        // its dense copy against B's rows shifted by r0; the parts left and
        // right of it hold no diagonal crossing
        const int d0 = max(kbeg, r0), d1 = min(kend, r0 + BM);
        if (p.dg && p.vec && r0 + BM <= p.M && r0 >= p.excl && d0 < d1) {
            if (d0 > kbeg)
                tile_mma<T, AOP, BOP, FROM_C, PATH>(acc, A, B, kbeg, d0, lds);
            Operand<T, OP_MK> D{p.dg + (int64_t)I * BM * BM, BM, 0, BM, 1, 0};
            Operand<T, OP_KM> B2{p.b + (int64_t)r0 * p.ldb, p.ldb, c0, p.N, p.vec, 0};
            tile_runs<T, OP_MK, OP_KM, FROM_C>(acc, D, B2, d0 - r0, d1 - r0, d1 - r0, lds);
            if (kend > d1)
                tile_mma<T, AOP, BOP, FROM_C, PATH>(acc, A, B, d1, kend, lds);
            done = true;
        }
    }
    if (!done)
        tile_mma<T, AOP, BOP, FROM_C, PATH>(acc, A, B, kbeg, kend, lds);

    if (interior && (CM != C_SUB_LOWER || I > J)) {
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j)
#pragma unroll
                for (int v = 0; v < 4; ++v) {
                    int row, col;
                    acc_pos<T>(i, j, v, row, col);
                    row += r0;
                    col += c0;
                    if (CM == C_PARTIAL)
                        p.part[(int64_t)split * p.M * p.N + (int64_t)row * p.N + col] = acc[i][j][v];
                    else
                        p.c[(int64_t)row * p.ldc + col] = acc[i][j][v];
                }
        return;
    }
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                int row, col;
                acc_pos<T>(i, j, v, row, col);
                row += r0;
                col += c0;
                if (row >= p.M || col >= p.N)
                    continue;
                const T val = acc[i][j][v];
                if (CM == C_SUB || CM == C_STORE) {
                    p.c[(int64_t)row * p.ldc + col] = val;
                } else if (CM == C_SUB_LOWER) {
                    if (row >= col)
                        p.c[(int64_t)row * p.ldc + col] = val;
                } else {
                    p.part[(int64_t)split * p.M * p.N + (int64_t)row * p.N + col] = val;
                }
            }
}

__device__ __forceinline__ void tile_of(int t, int tri, int TJ, int &I, int &J)
{
    if (tri) {
        int r = (int)((sqrtf(8.0f * t + 1.0f) - 1.0f) * 0.5f);
        while (r * (r + 1) / 2 > t) --r;
        while ((r + 1) * (r + 2) / 2 <= t) ++r;
        I = r;
        J = t - r * (r + 1) / 2;
    } else {
        I = t / TJ;
        J = t % TJ;
    }
}

// SCHED: which tile schedules the kernel carries.  The lower trailing update
// gets a dynamic-only kernel (dropping the static path avoids register
// spills there); the other products measured as fast or faster with both
// compiled in (the choice is then made at run time from p.sched).
enum { SCHED_BOTH = 0, SCHED_DYN = 1, SCHED_STATIC = 2 };

template <typename T, int AOP, int BOP, int CM, int PATH, int SCHED>
__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2)))
k_gemm(GemmArgs<T> p)
{
    using namespace gemm_detail;
    __shared__ T lds[2 * 2 * BK * Pitch<T>::v];
    const int TI = (p.M + BM - 1) / BM, TJ = (p.N + BN - 1) / BN;
    const int nt = p.tn ? p.tn : (p.tri ? TI * (TI + 1) / 2 : TI * TJ);

    if (SCHED == SCHED_STATIC || (SCHED == SCHED_BOTH && !p.sched)) {
        // static: one tile per block, tiles spread over the XCDs in contiguous ranges
        int I, J;
        tile_of(p.t0 + gemm_detail::xcd_tile(blockIdx.x, nt), p.tri, TJ, I, J);
        int kbeg = 0, kend = p.K;
        if (CM == C_PARTIAL) {
            kbeg = blockIdx.y * p.kchunk;
            kend = min(p.K, kbeg + p.kchunk);
        }
        gemm_tile<T, AOP, BOP, CM, PATH>(p, I, J, blockIdx.y, kbeg, kend, lds);
        return;
    }

    // dynamic: every block takes (split, tile) items until none are left, so a
    // block that shares its CU with other work simply takes fewer items
    __shared__ int s_item;
    const int splits = (CM == C_PARTIAL) ? p.splits : 1;
    const int items = nt * splits;
    for (;;) {
        if (threadIdx.x == 0)
            s_item = atomicAdd(p.sched, 1);
        __syncthreads();
        const int it = s_item;
        if (it >= items)
            break;
        const int split = it / nt;
        int I, J;
        tile_of(p.t0 + it % nt, p.tri, TJ, I, J);
        int kbeg = 0, kend = p.K;
        if (CM == C_PARTIAL) {
            kbeg = split * p.kchunk;
            kend = min(p.K, kbeg + p.kchunk);
        }
        gemm_tile<T, AOP, BOP, CM, PATH>(p, I, J, split, kbeg, kend, lds);
    }
    // the last block to finish returns the counters to zero for the next launch
    if (threadIdx.x == 0) {
        const int done = atomicAdd(p.sched + 1, 1);
        if (done == (int)gridDim.x - 1) {
            atomicExch(p.sched, 0);
            atomicExch(p.sched + 1, 0);
        }
    }
}

// host side -------------------------------------------------------------------

template <typename T>
static inline bool aligned16(const T *p, int64_t ld)
{
    constexpr int PER = 16 / sizeof(T);
    return ((uintptr_t)p % 16 == 0) && (ld % PER == 0);
}

template <typename T, int AOP, int BOP, int CM>
static chol_status gemm(GemmArgs<T> p, int splits, hipStream_t st)
{
    using namespace gemm_detail;
    if (p.M <= 0 || p.N <= 0)
        return CHOL_OK;
    p.vec = aligned16(p.a, p.lda) && aligned16(p.b, p.ldb);
    p.splits = splits;
    const int TI = (p.M + BM - 1) / BM, TJ = (p.N + BN - 1) / BN;
    const int nt_all = p.tri ? TI * (TI + 1) / 2 : TI * TJ;
    if (p.t0 < 0 || p.tn < 0 || p.t0 + (p.tn ? p.tn : nt_all) > nt_all)
        return CHOL_ERR_INVALID_VALUE;
    const int nt = p.tn ? p.tn : nt_all;
    if (nt == 0)
        return CHOL_OK;
    // which K-loop path the kernel carries: products of plain operands and
    // of the symmetric operand decide per tile which chunks take the
    // pipelined runs (all of them unless the tile has edges, diagonal
    // crossings or masks); the masked triangular operands take only the
    // general loop
    constexpr bool PLAIN_A = AOP == OP_MK || AOP == OP_KM;
    constexpr bool PLAIN_B = BOP == OP_MK || BOP == OP_KM;
    const bool all_fast = p.vec && p.M % BM == 0 && p.N % BN == 0 && p.K % BK == 0 &&
                          (CM != C_PARTIAL || p.kchunk % BK == 0);
    const dim3 sgrid((unsigned)nt, (unsigned)(CM == C_PARTIAL ? splits : 1));
    unsigned dgrid = 0;
    if (p.sched) {
        // persistent blocks, all resident at once (two per CU the stream may use)
        const int64_t items = (int64_t)nt * (CM == C_PARTIAL ? splits : 1);
        dgrid = (unsigned)std::min<int64_t>(items, p.cap > 0 ? p.cap : 2 * 240);
    }
    auto launch = [&](auto path_c) {
        constexpr int PATH = decltype(path_c)::value;
        if (p.sched && CM == C_SUB_LOWER)
            hipLaunchKernelGGL((k_gemm<T, AOP, BOP, CM, PATH, SCHED_DYN>), dim3(dgrid), dim3(NT), 0, st, p);
        else if (p.sched)
            hipLaunchKernelGGL((k_gemm<T, AOP, BOP, CM, PATH, SCHED_BOTH>), dim3(dgrid), dim3(NT), 0, st, p);
        else
            hipLaunchKernelGGL((k_gemm<T, AOP, BOP, CM, PATH, SCHED_BOTH>), sgrid, dim3(NT), 0, st, p);
    };
    if constexpr (PLAIN_A && PLAIN_B) {
        (void)all_fast;
        launch(std::integral_constant<int, PATH_MIXED>());
    } else if constexpr (AOP == OP_SYM && PLAIN_B) {
        launch(std::integral_constant<int, PATH_MIXED>());
    } else {
        launch(std::integral_constant<int, PATH_GENERAL>());
    }
    CHOL_LAUNCH_CHECK();
    return CHOL_OK;
}

} // namespace chol
