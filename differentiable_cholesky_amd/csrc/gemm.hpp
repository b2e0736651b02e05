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
//   OP_SYM_DG    OP_SYM whose 128 x 128 diagonal blocks are all read from a
//            dense copy (GemmArgs::dg); chosen by the host when every block
//            the product meets has one
//
// Design for gfx950: a 256-thread block computes a 128 x 128 tile as 2 x 2
// wavefronts of 64 x 64, each a 4 x 4 grid of 16x16x4 MFMA steps.  The
// contraction advances in chunks of BK (one 128-byte row segment per m: 16
// for fp64, 32 for fp32) staged in LDS, double-buffered.  A chunk is brought
// in by 16-byte global loads that write LDS directly (global_load_lds_dwordx4:
// lane i of a wave instruction fills bytes [16 i, 16 i + 16) of a 1 KB run),
// so staging costs no registers and no LDS write instructions; the loads of
// chunk c+1 are issued before the matrix-core steps of chunk c and waited for
// once, at the barrier that ends the chunk.  Two LDS layouts:
//   LAY_MK  [m][k] with the 16-byte slots of each row XOR-swizzled by m & 7,
//           so that the 16 lanes reading one k for 16 rows hit distinct banks
//           (a run of 8 rows is one wave instruction: the swizzle is applied
//           by choosing which global slot each lane fetches);
//   LAY_KM  [k][m] (128 contiguous m per k row, as k-major memory holds them).
// Chunks that are not whole 16-byte runs inside the operand (edges, the
// diagonal of a symmetric operand, an excluded block, unaligned operands) are
// fetched element by element with bounds and written to LDS in the same
// layout.  The lower mask of OP_KM_LOWER is applied when a fragment is read
// from LDS, so masked operands also take the direct loads.  Blocks are mapped
// to tiles so that each of the 8 XCDs receives a contiguous row-major range of
// tiles (rows of A and columns of B stay in one XCD's L2).
#pragma once

#include <algorithm>
#include <type_traits>

#include "common.hpp"

#include <hip/hip_ext.h>

namespace chol {

enum { OP_MK = 0, OP_KM = 1, OP_SYM = 2, OP_KM_LOWER = 3, OP_SYM_DG = 4 };
// contraction unit of the piece schedule: a whole number of fp32 (32) and
// fp64 (16) chunks
constexpr int SK_UNIT = 32;

enum { C_SUB = 0,        // C -= AB
       C_SUB_LOWER = 1,  // C -= AB where row >= col
       C_STORE = 2,      // C  = AB
       C_PARTIAL = 3 };  // part[split] = AB (row-major M x N)

template <typename T> struct GemmArgs {
    int M, N, K;
    const T *a; int64_t lda;
    const T *b; int64_t ldb;
    T *c; int64_t ldc;
    const T *cin; int64_t ldcin;  // C_SUB, C_SUB_LOWER, optional: C's values read
                         // from here (same shape) and the results written to c
    int kchunk;          // split-K: contraction length per split (multiple of 32)
    T *part;             // C_PARTIAL destination, splits * M * N
    int tri;             // 1: lower-triangular tile grid (M == N)
    int vec;             // bit 0 (A), bit 1 (B): 16-byte global loads are legal for that operand
    int splits;          // split count (C_PARTIAL)
    int excl;            // OP_SYM A operand: entries (m, k) with m < excl and
                         // k < excl read as zero (a block left out of the product)
    int t0, tn;          // tile window: tiles t0 .. t0 + tn - 1 of the (row-major
                         // or lower-triangular) tile grid; tn == 0: every tile
    int cap;             // persistent grid size with `sched` (0: two blocks per CU of 240)
    int *sched;          // non-null: blocks take (split, tile) items from this
                         // device counter pair (item, finished blocks), which
                         // must be zero at launch and is zero again afterwards
    int piece;           // C_PARTIAL with `sched`, optional: the tiles' contractions
                         // laid end to end in units of SK_UNIT elements and cut
                         // into pieces of `piece` units, one item each (a piece
                         // may end one tile's contraction and start the next
                         // one's); partial slot of a piece on a tile = the
                         // piece's index minus that of the first piece on the
                         // tile.  0: `splits` equal splits per tile
    const T *dg;         // OP_SYM A operand, optional: the symmetric 128 x 128
                         // diagonal blocks written whole (block I at dg + I*128*128,
                         // row-major), read by direct loads instead of
                         // assembling them from the lower triangle element by element
};

namespace gemm_detail {

constexpr int BM = 128;   // the large tile edge (the symmetric operand's diagonal blocks)
constexpr int NT = 256;

// Chunk geometry of one operand's TE x BK chunk (TE = 128, 64 or 32 rows
// along m).  An output tile is TM x TN (128 x 128, 64 x 128, 64 x 64, or
// 32 x 32 for the tile-sized products): A's chunks have TM rows, B's TN, and
// the 2 x 2 waves each own TM/2 x TN/2 of it, an FRM x FRN grid of 16 x 16
// MFMA tiles.  (A block always owns whole 128-column spans of its
// rows, so products computed in place over a 128-wide panel stay race-free.)
template <typename T, int TE = 128> struct Stage {
    static_assert(TE == 128 || TE == 64 || TE == 32, "tile edge 128, 64 or 32");
    static constexpr int PER = 16 / (int)sizeof(T);   // elements per 16-byte slot
    static constexpr int BK = 8 * PER;                 // chunk depth: 128 bytes of k per m
    static constexpr int TILE = TE * BK;               // elements of one staged operand chunk
    static constexpr int GEN = TILE / NT;              // elements per thread on the per-element path
    static constexpr int DPW = TE / 32;                // direct-load instructions per wave per chunk
};
template <int TM, int TN = 128> struct WaveTile {
    static constexpr int WM = TM / 2;                  // wave tile rows
    static constexpr int FRM = TM / 32;                // MFMA tiles along the wave tile's rows
    static constexpr int WN = TN / 2;                  // wave tile columns
    static constexpr int FRN = TN / 32;
};
// a wave's accumulators: FRM x FRN MFMA result tiles
template <typename T, int TM, int TN = 128>
using AccTile = typename Acc<T>::type[WaveTile<TM, TN>::FRM][WaveTile<TM, TN>::FRN];

// LDS a product needs: two buffers of A's (TM x BK) and B's (128 x BK) chunks
// (64 KB for 128-row tiles, 48 KB for 64-row tiles)
template <typename T, int TM = 128> constexpr int LDS_ELEMS = 2 * (Stage<T, TM>::TILE + Stage<T, 128>::TILE);

enum { LAY_MK = 0, LAY_KM = 1 };

typedef __attribute__((address_space(1))) void gvoid;
typedef __attribute__((address_space(3))) void lvoid;

// position of chunk element (m, k) in LDS
template <typename T, int TE>
__device__ __forceinline__ int lds_index(int lay, int m, int k)
{
    constexpr int PER = Stage<T, TE>::PER, BK = Stage<T, TE>::BK;
    return lay == LAY_MK ? m * BK + (((k / PER) ^ (m & 7)) * PER) + (k % PER) : k * TE + m;
}

// s_waitcnt vmcnt(0): this wave's global loads (and their LDS writes) are done
__device__ __forceinline__ void wait_loads() { __builtin_amdgcn_s_waitcnt(0x0F70); }
// s_waitcnt vmcnt(1): all but the wave's last load are done
__device__ __forceinline__ void wait_loads_but_1() { __builtin_amdgcn_s_waitcnt(0x0F71); }

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
    // OP_SYM, OP_SYM_DG
    if (m > k)
        return p[(int64_t)m * ld + k];
    if (m < k)
        return p[(int64_t)k * ld + m];
    return T(2) * p[(int64_t)m * ld + m];
}

template <typename T, int OP, int TS = 128>   // TS: the operand's chunk rows (along m)
struct Operand {
    const T *p;
    int64_t ld;
    int m0;      // tile origin along m
    int mlim;    // M (or N) bound
    int vec;     // 16-byte loads legal (base aligned, ld a multiple of 16 bytes)
    int excl;    // OP_SYM: leading excl x excl block left out

    // LDS layout of the operand's chunks: row panels keep rows, k-major
    // operands keep k rows (the symmetric operand is only ever staged by the
    // per-element path: its plain parts are handed over as row panels or
    // k-major panels by the tile body)
    static constexpr int LAY = (OP == OP_MK || OP == OP_SYM || OP == OP_SYM_DG) ? LAY_MK : LAY_KM;

    // can the chunk at k0 be staged by direct 16-byte loads?
    __device__ __forceinline__ bool direct(int k0, int klim) const
    {
        constexpr int BK = Stage<T, TS>::BK, PER = Stage<T, TS>::PER;
        if (OP == OP_SYM || OP == OP_SYM_DG)
            return false;
        return vec && m0 + TS <= mlim && k0 + BK <= klim && k0 % PER == 0 && m0 % PER == 0;
    }

    // direct loads of the chunk at k0 into S
    __device__ __forceinline__ void stage_direct(int k0, T *S) const
    {
        constexpr int PER = Stage<T, TS>::PER, BK = Stage<T, TS>::BK, DPW = Stage<T, TS>::DPW;
        const int lane = threadIdx.x % 64, w = threadIdx.x / 64;
        // the chunk's origin is uniform; a lane's element offset from it fits
        // 32 bits (at most 127 rows of ld elements, ld < 2^24)
        const int ld32 = (int)ld;
        if (LAY == LAY_MK) {
            // instruction q: rows 8q .. 8q+7; lane -> row r = lane / 8, LDS slot
            // lane % 8 of that row, which holds global slot (lane % 8) ^ r
            const T *base = p + (int64_t)m0 * ld + k0;
            const int r = lane / 8, sl = (lane % 8) ^ r;
            const int off = r * ld32 + sl * PER;
#pragma unroll
            for (int j = 0; j < DPW; ++j) {
                const int q = w + 4 * j;
                __builtin_amdgcn_global_load_lds((gvoid *)(base + (off + 8 * q * ld32)), (lvoid *)(S + 8 * q * BK),
                                                 16, 0, 0);
            }
        } else {
            // instruction q: elements [q * 64 PER, (q + 1) * 64 PER) of the [k][m] chunk
            const T *base = p + (int64_t)k0 * ld + m0;
#pragma unroll
            for (int j = 0; j < DPW; ++j) {
                const int q = w + 4 * j;
                const int e = q * 64 * PER + lane * PER;
                __builtin_amdgcn_global_load_lds((gvoid *)(base + ((e / TS) * ld32 + e % TS)), (lvoid *)(S + q * 64 * PER),
                                                 16, 0, 0);
            }
        }
    }

    // one element of one of the 128-byte lines of the chunk at k0 (a chunk
    // is TS such lines; thread l < TS takes line l), read only to bring the
    // line into L2 ahead of its direct load
    __device__ __forceinline__ T touch(int k0) const
    {
        constexpr int LPK = TS * (int)sizeof(T) / 128;   // lines per k row of a k-major chunk
        const int l = threadIdx.x % TS;
        if (LAY == LAY_MK)
            return p[(int64_t)(m0 + l) * ld + k0];
        return p[(int64_t)(k0 + l / LPK) * ld + m0 + (l % LPK) * (128 / (int)sizeof(T))];
    }

    // per-element path: bounds, masks, the symmetric diagonal; four
    // elements in flight per step, which keeps the path's registers few
    __device__ __forceinline__ void stage_elems(int k0, int klim, T *S) const
    {
        constexpr int BK = Stage<T, TS>::BK, GEN = Stage<T, TS>::GEN;
        constexpr int STEP = GEN < 4 ? GEN : 4;     // a 32-row fp64 chunk has 2 elements per thread
#pragma unroll 1
        for (int j0 = 0; j0 < GEN; j0 += STEP) {
            T v[STEP];
#pragma unroll
            for (int j = 0; j < STEP; ++j) {
                const int e = threadIdx.x + NT * (j0 + j);
                const int m = LAY == LAY_MK ? e / BK : e % TS, k = LAY == LAY_MK ? e % BK : e / TS;
                v[j] = elem<T, OP>(p, ld, m0 + m, k0 + k, mlim, klim, excl);
            }
#pragma unroll
            for (int j = 0; j < STEP; ++j) {
                const int e = threadIdx.x + NT * (j0 + j);
                const int m = LAY == LAY_MK ? e / BK : e % TS, k = LAY == LAY_MK ? e % BK : e / TS;
                S[lds_index<T, TS>(LAY, m, k)] = v[j];
            }
        }
    }

    __device__ __forceinline__ void stage(int k0, int klim, T *S) const
    {
        if (direct(k0, klim))
            stage_direct(k0, S);
        else
            stage_elems(k0, klim, S);
    }

    // fragment element (m, k) of the chunk at k0 staged in S
    __device__ __forceinline__ T frag(const T *S, int m, int k, int k0) const
    {
        const T x = S[lds_index<T, TS>(LAY, m, k)];
        if (OP == OP_KM_LOWER)
            return (k0 + k >= m0 + m) ? x : T(0);
        return x;
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

// acc += (NEG ? -A : A) B over one chunk at k0 staged at SA (A) and SB (B)
template <typename T, int AOP, int BOP, bool NEG, int TM, int TN = 128>
__device__ __forceinline__ void chunk_mma(AccTile<T, TM, TN> &acc, const Operand<T, AOP, TM> &A,
                                          const Operand<T, BOP, TN> &B, int k0, const T *SA, const T *SB)
{
    constexpr int BK = Stage<T, TM>::BK;
    constexpr int FRM = WaveTile<TM, TN>::FRM, FRN = WaveTile<TM, TN>::FRN;
    constexpr int WM = WaveTile<TM, TN>::WM, WN = WaveTile<TM, TN>::WN;
    const int lane = threadIdx.x % 64, wave = threadIdx.x / 64;
    const int wm = wave / 2, wn = wave % 2;
#pragma unroll
    for (int kk = 0; kk < BK; kk += 4) {
        const int kr = kk + lane / 16;
        T af[FRM], bf[FRN];
#pragma unroll
        for (int i = 0; i < FRM; ++i)
            af[i] = A.frag(SA, wm * WM + i * 16 + lane % 16, kr, k0);
#pragma unroll
        for (int j = 0; j < FRN; ++j)
            bf[j] = B.frag(SB, wn * WN + j * 16 + lane % 16, kr, k0);
#pragma unroll
        for (int i = 0; i < FRM; ++i)
#pragma unroll
            for (int j = 0; j < FRN; ++j)
                acc[i][j] = mfma16x16x4_s<NEG>(af[i], bf[j], acc[i][j]);
    }
}

} // namespace gemm_detail

// The K loop of one 128 x 128 tile: acc += (NEG ? -A : A) B over k in
// [kbeg, kend), operands staged through `lds` (LDS_ELEMS<T> elements).
// Called by all 256 threads of the block.  Software pipeline over chunks: the
// loads of chunk c+1 go out (directly into the free LDS buffers) before the
// matrix-core steps of chunk c; one wait and one barrier end each chunk.
// Each chunk of each operand is classified at run time (uniformly over the
// block): direct loads wherever the chunk allows them, the per-element path
// otherwise.  BOOST raises the waves' priority while they issue the next
// chunk's loads and the current chunk's matrix-core steps, so that on a SIMD
// shared by two blocks the block coming out of a barrier gets its memory
// traffic going first.  TOUCH (for an A streamed from HBM without reuse, as
// in the symmetric product): one load per 128-byte line of A's chunk c+2
// also goes out in iteration c (from waves 0 and 1), which brings the chunk
// into L2 before its direct loads are issued; the wait at the end of the
// chunk leaves that one load in flight.  (A second LDS buffer set for a
// two-chunk lookahead would take the block to 80 KB of LDS, and two blocks no
// longer fit a CU.)
template <typename T, int AOP, int BOP, bool NEG, bool BOOST = false, bool TOUCH = false, int TM = 128, int TN = 128>
__device__ __forceinline__ void tile_mma(gemm_detail::AccTile<T, TM, TN> &acc,
                                         const gemm_detail::Operand<T, AOP, TM> &A,
                                         const gemm_detail::Operand<T, BOP, TN> &B, int kbeg, int kend, T *lds)
{
    using namespace gemm_detail;
    constexpr int BK = Stage<T, TM>::BK, TA = Stage<T, TM>::TILE, SZ = TA + Stage<T, TN>::TILE;
    if (kend <= kbeg)
        return;
    const int nc = (kend - kbeg + BK - 1) / BK;
    __syncthreads();                      // earlier users of the LDS buffers are done
    A.stage(kbeg, kend, lds);
    B.stage(kbeg, kend, lds + TA);
    wait_loads();
    __syncthreads();
    const bool toucher = TOUCH && threadIdx.x < TM;
    T tsum = T(0), tprev = T(0);
    for (int c = 0; c < nc; ++c) {
        const int k0 = kbeg + c * BK;
        const T *S = lds + (c & 1) * SZ;
        if (BOOST)
            __builtin_amdgcn_s_setprio(2);
        if (c + 1 < nc) {
            T *D = lds + ((c + 1) & 1) * SZ;
            A.stage(k0 + BK, kend, D);
            B.stage(k0 + BK, kend, D + TA);
        }
        const bool touch = toucher && c + 2 < nc && A.direct(k0 + 2 * BK, kend);
        T tnext = T(0);
        if (touch)
            tnext = A.touch(k0 + 2 * BK);
        chunk_mma<T, AOP, BOP, NEG, TM, TN>(acc, A, B, k0, S, S + TA);
        if (BOOST)
            __builtin_amdgcn_s_setprio(0);
        if (touch)
            wait_loads_but_1();
        else
            wait_loads();
        __syncthreads();
        if (TOUCH) {
            tsum += tprev;                // loaded a chunk ago: complete by now
            tprev = tnext;
        }
    }
    if (TOUCH) {
        // the touched values are consumed here, so the loads are kept; they
        // carry nothing into the result
        tsum += tprev;
        __asm__ volatile("" : : "v"(tsum));
    }
}

// The same product without the software pipeline, for the few chunks of a
// symmetric operand that must be assembled element by element (the diagonal
// block when no dense copy of it exists): stage, wait, compute, one chunk at
// a time.  It keeps no state across chunks, which keeps the registers of the
// kernels that carry it within budget.
template <typename T, int AOP, int BOP, bool NEG, int TM = 128>
__device__ __forceinline__ void tile_mma_serial(gemm_detail::AccTile<T, TM> &acc,
                                                const gemm_detail::Operand<T, AOP, TM> &A,
                                                const gemm_detail::Operand<T, BOP, 128> &B, int kbeg, int kend,
                                                T *lds)
{
    using namespace gemm_detail;
    constexpr int BK = Stage<T, TM>::BK, TA = Stage<T, TM>::TILE;
#pragma unroll 1
    for (int k0 = kbeg; k0 < kend; k0 += BK) {
        __syncthreads();
        A.stage_elems(k0, kend, lds);
        B.stage(k0, kend, lds + TA);
        wait_loads();
        __syncthreads();
        chunk_mma<T, AOP, BOP, NEG, TM>(acc, A, B, k0, lds, lds + TA);
    }
}

// Position of accumulator element (i, j, v) of this thread inside the TM x 128 tile.
template <typename T, int TM = 128, int TN = 128>
__device__ __forceinline__ void acc_pos(int i, int j, int v, int &row, int &col)
{
    const int lane = threadIdx.x % 64, wave = threadIdx.x / 64;
    row = (wave / 2) * gemm_detail::WaveTile<TM, TN>::WM + i * 16 + Acc<T>::row(lane, v);
    col = (wave % 2) * gemm_detail::WaveTile<TM, TN>::WN + j * 16 + lane % 16;
}

// One TM x 128 output tile (I, J) over the contraction range [kbeg, kend).
template <typename T, int AOP, int BOP, int CM, bool BOOST = false, int TM = 128, int TN = 128>
__device__ __forceinline__ void gemm_tile(const GemmArgs<T> &p, int I, int J, int split, int kbeg, int kend, T *lds)
{
    using namespace gemm_detail;
    typedef typename Acc<T>::type acc_t;
    constexpr int FRM = WaveTile<TM, TN>::FRM, FRN = WaveTile<TM, TN>::FRN;
    static_assert((TM == BM && TN == BM) || (AOP != OP_SYM && AOP != OP_SYM_DG), "the symmetric operand takes 128 tiles");
    const int r0 = I * TM, c0 = J * TN;

    // C -= AB runs as acc = C, acc += (-A) B: the accumulators start from C,
    // so the epilogue is a plain store and no accumulator has to leave the
    // matrix-core registers for a read-modify-write.
    constexpr bool FROM_C = (CM == C_SUB || CM == C_SUB_LOWER);
    // a lower-only update has nothing to do on a tile above the diagonal (nor
    // on the lower half of a short last triangular tile that lies past M)
    if ((CM == C_SUB_LOWER && r0 + TM - 1 < c0) || r0 >= p.M)
        return;
    // a tile inside M x N needs no per-entry bounds test: its loads of C and
    // its stores are issued back to back, without a branch around each one
    const bool interior = r0 + TM <= p.M && c0 + TN <= p.N;
    const T *cin = p.cin ? p.cin : p.c;
    const int64_t ldcin = p.cin ? p.ldcin : p.ldc;
    acc_t acc[FRM][FRN];
    if (FROM_C && interior) {
#pragma unroll
        for (int i = 0; i < FRM; ++i)
#pragma unroll
            for (int j = 0; j < FRN; ++j)
#pragma unroll
                for (int v = 0; v < 4; ++v) {
                    int row, col;
                    acc_pos<T, TM, TN>(i, j, v, row, col);
                    acc[i][j][v] = cin[(int64_t)(row + r0) * ldcin + col + c0];
                }
    } else {
#pragma unroll
        for (int i = 0; i < FRM; ++i)
#pragma unroll
            for (int j = 0; j < FRN; ++j)
#pragma unroll
                for (int v = 0; v < 4; ++v) {
                    T x = T(0);
                    if (FROM_C) {
                        int row, col;
                        acc_pos<T, TM, TN>(i, j, v, row, col);
                        row += r0;
                        col += c0;
                        if (row < p.M && col < p.N)
                            x = cin[(int64_t)row * ldcin + col];
                    }
                    acc[i][j][v] = x;
                }
    }

    const int va = p.vec & 1, vb = (p.vec >> 1) & 1;
    Operand<T, AOP, TM> A{p.a, p.lda, r0, p.M, va, p.excl};
    Operand<T, BOP, TN> B{p.b, p.ldb, c0, p.N, vb, 0};
    if constexpr (AOP == OP_SYM || AOP == OP_SYM_DG) {
        // Sym(S)(m, k) for the tile's rows m in [r0, r0 + 128): left of the
        // diagonal block (k < r0) it is a row panel of S's lower triangle,
        // right of it (k >= r0 + 128) a k-major panel of it (S[k][m]); both
        // take the direct loads.  The diagonal block comes from its dense copy
        // with OP_SYM_DG (a plain row panel against B's rows shifted by r0),
        // else element by element.  The left-out leading block (at most 128
        // wide) can only meet the diagonal block of tile row 0, whose left
        // part is empty.
        const int b1 = min(kend, r0), d0 = max(kbeg, r0), d1 = min(kend, r0 + BM), a0 = max(kbeg, r0 + BM);
        if (b1 > kbeg) {
            Operand<T, OP_MK> Ab{p.a, p.lda, r0, p.M, va, 0};
            tile_mma<T, OP_MK, BOP, FROM_C, BOOST, true>(acc, Ab, B, kbeg, b1, lds);
        }
        if (d1 > d0 && !(r0 + BM <= p.excl)) {
            if constexpr (AOP == OP_SYM_DG) {
                Operand<T, OP_MK> D{p.dg + (int64_t)I * BM * BM, BM, 0, BM, 1, 0};
                Operand<T, BOP> B2{p.b + (int64_t)r0 * p.ldb, p.ldb, c0, p.N, vb, 0};
                tile_mma<T, OP_MK, BOP, FROM_C, BOOST>(acc, D, B2, d0 - r0, d1 - r0, lds);
            } else {
                tile_mma_serial<T, AOP, BOP, FROM_C>(acc, A, B, d0, d1, lds);
            }
        }
        if (kend > a0) {
            Operand<T, OP_KM> Aa{p.a, p.lda, r0, p.M, va, 0};
            tile_mma<T, OP_KM, BOP, FROM_C, BOOST, true>(acc, Aa, B, a0, kend, lds);
        }
    } else {
        tile_mma<T, AOP, BOP, FROM_C, BOOST, false, TM, TN>(acc, A, B, kbeg, kend, lds);
    }

    if (interior && (CM != C_SUB_LOWER || r0 >= c0 + TN - 1)) {
#pragma unroll
        for (int i = 0; i < FRM; ++i)
#pragma unroll
            for (int j = 0; j < FRN; ++j)
#pragma unroll
                for (int v = 0; v < 4; ++v) {
                    int row, col;
                    acc_pos<T, TM, TN>(i, j, v, row, col);
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
    for (int i = 0; i < FRM; ++i)
#pragma unroll
        for (int j = 0; j < FRN; ++j)
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                int row, col;
                acc_pos<T, TM, TN>(i, j, v, row, col);
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

// Waves per SIMD the register allocation aims for: two blocks of 128-row
// tiles per CU (256 registers each, 64 KB of LDS), or three of 64-row tiles
// (half the accumulators, 48 KB of LDS).
template <int TM> constexpr int gemm_waves() { return TM == 128 ? 2 : 3; }

template <typename T, int AOP, int BOP, int CM, int SCHED, int TM, int TN = 128>
__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(gemm_waves<TM>(), gemm_waves<TM>())))
k_gemm(GemmArgs<T> p)
{
    using namespace gemm_detail;
    __shared__ T lds[LDS_ELEMS<T, TM>];
    // tile grid: TM-row by 128-column tiles (the lower-triangular grid only
    // with square tiles, TM = 128)
    // a triangular grid counts 128 x 128 tiles; with 64-row tiles each of
    // them is two items (its upper and lower half), dynamic schedule only
    constexpr int HALVES = TM == 64 ? 2 : 1;
    const int TI = p.tri ? (p.M + 127) / 128 : (p.M + TM - 1) / TM, TJ = (p.N + TN - 1) / TN;
    const int nt = (p.tn ? p.tn : (p.tri ? TI * (TI + 1) / 2 : TI * TJ)) * (p.tri ? HALVES : 1);

    if (SCHED == SCHED_STATIC || (SCHED == SCHED_BOTH && !p.sched)) {
        // static: one tile per block, tiles spread over the XCDs in contiguous ranges
        int I, J;
        tile_of(p.t0 + gemm_detail::xcd_tile(blockIdx.x, nt), p.tri, TJ, I, J);
        int kbeg = 0, kend = p.K;
        if (CM == C_PARTIAL) {
            kbeg = blockIdx.y * p.kchunk;
            kend = min(p.K, kbeg + p.kchunk);
        }
        gemm_tile<T, AOP, BOP, CM, true, TM, TN>(p, I, J, blockIdx.y, kbeg, kend, lds);
        return;
    }

    // dynamic: every block takes (split, tile) items until none are left, so a
    // block that shares its CU with other work simply takes fewer items
    __shared__ int s_item;
    const int splits = (CM == C_PARTIAL) ? p.splits : 1;
    const int64_t nku = (p.K + SK_UNIT - 1) / SK_UNIT;            // units per tile (piece schedule)
    const bool pieces = CM == C_PARTIAL && p.piece > 0;
    const int items = pieces ? (int)(((int64_t)nt * nku + p.piece - 1) / p.piece) : nt * splits;
    for (;;) {
        if (threadIdx.x == 0)
            s_item = atomicAdd(p.sched, 1);
        __syncthreads();
        const int it = s_item;
        __syncthreads();                  // every thread holds the item before s_item is rewritten
        if (it >= items)
            break;
        if (pieces) {
            // piece it: units [lo, hi) of the contractions laid end to end,
            // over one tile or the end of one and the start of the next
            const int64_t total = (int64_t)nt * nku, lo = (int64_t)it * p.piece;
            const int64_t hi = lo + p.piece < total ? lo + p.piece : total;
            for (int64_t t = lo / nku; t * nku < hi; ++t) {
                const int64_t t0u = t * nku, t1u = t0u + nku;
                const int64_t a = (lo > t0u ? lo : t0u) - t0u, b = (hi < t1u ? hi : t1u) - t0u;
                const int slot = it - (int)(t0u / p.piece);
                const int64_t kend = b * SK_UNIT < p.K ? b * SK_UNIT : p.K;
                int I, J;
                tile_of(p.t0 + (int)t, p.tri, TJ, I, J);
                gemm_tile<T, AOP, BOP, CM, true, TM, TN>(p, I, J, slot, (int)(a * SK_UNIT), (int)kend, lds);
            }
            continue;
        }
        const int split = it / nt;
        int I, J;
        if (HALVES == 2 && p.tri) {
            const int t = it % nt;
            tile_of(p.t0 + t / 2, 1, TJ, I, J);
            I = 2 * I + (t & 1);
        } else {
            tile_of(p.t0 + it % nt, p.tri, TJ, I, J);
        }
        int kbeg = 0, kend = p.K;
        if (CM == C_PARTIAL) {
            kbeg = split * p.kchunk;
            kend = min(p.K, kbeg + p.kchunk);
        }
        gemm_tile<T, AOP, BOP, CM, true, TM, TN>(p, I, J, split, kbeg, kend, lds);
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

// direct 16-byte loads: aligned base and rows, and lane offsets within a tile
// (127 rows of ld elements) that fit 32 bits
template <typename T>
static inline bool aligned16(const T *p, int64_t ld)
{
    constexpr int PER = 16 / sizeof(T);
    return ((uintptr_t)p % 16 == 0) && (ld % PER == 0) && ld < ((int64_t)1 << 24);
}

namespace gemm_detail {
// a launch of the product kernel; with an event pair (a timed launch) the
// kernel's own start and end are stamped into it
template <typename T>
static void launch(void (*kern)(GemmArgs<T>), dim3 grid, hipStream_t st, const GemmArgs<T> &p, hipEvent_t ea,
                   hipEvent_t eb)
{
    if (ea && eb)
        hipExtLaunchKernelGGL(kern, grid, dim3(NT), 0, st, ea, eb, 0, p);
    else
        hipLaunchKernelGGL(kern, grid, dim3(NT), 0, st, p);
}
} // namespace gemm_detail

// C op= A B on the stream; TM x TN: output tile (128 x 128; 64 x 128 or
// 64 x 64 for short products whose 128 x 128 tiles would be too few, or too
// long each, to spread over the device; 32 x 128 for the in-place panel
// products, whose blocks must each own whole 128-wide rows; 32 x 32 for
// tile-sized products)
template <typename T, int AOP, int BOP, int CM, int TM = 128, int TN = 128>
static chol_status gemm(GemmArgs<T> p, int splits, hipStream_t st, hipEvent_t ea = nullptr, hipEvent_t eb = nullptr)
{
    using namespace gemm_detail;
    if (p.M <= 0 || p.N <= 0)
        return CHOL_OK;
    if (TM != BM && p.tri && !p.sched)
        return CHOL_ERR_INVALID_VALUE;           // halves of triangular tiles: dynamic schedule only
    if (TN != BM && (p.tri || p.sched))
        return CHOL_ERR_INVALID_VALUE;           // 64-column tiles: static rectangular grids only
    if (p.piece < 0 || (p.piece > 0 && (CM != C_PARTIAL || !p.sched)))
        return CHOL_ERR_INVALID_VALUE;           // pieces: persistent split-contraction products only
    p.vec = (aligned16(p.a, p.lda) ? 1 : 0) | (aligned16(p.b, p.ldb) ? 2 : 0);
    p.splits = splits;
    if constexpr (AOP == OP_SYM) {
        static_assert(TM == BM && TN == BM, "the symmetric operand takes 128 tiles");
        // the excluded block is at most one tile; with a dense copy of every
        // diagonal block the product meets, the kernel reads them from it
        if (p.excl < 0 || p.excl > BM)
            return CHOL_ERR_INVALID_VALUE;
        if (p.dg && p.vec == 3 && p.M % BM == 0 && (p.excl == 0 || p.excl == BM) && ((uintptr_t)p.dg % 16) == 0)
            return gemm<T, OP_SYM_DG, BOP, CM, TM>(p, splits, st, ea, eb);
    }
    const int TI = p.tri ? (p.M + BM - 1) / BM : (p.M + TM - 1) / TM, TJ = (p.N + TN - 1) / TN;
    const int nt_all = p.tri ? TI * (TI + 1) / 2 : TI * TJ;
    if (p.t0 < 0 || p.tn < 0 || p.t0 + (p.tn ? p.tn : nt_all) > nt_all)
        return CHOL_ERR_INVALID_VALUE;
    const int nt = p.tn ? p.tn : nt_all;
    if (nt == 0)
        return CHOL_OK;
    const dim3 sgrid((unsigned)nt, (unsigned)(CM == C_PARTIAL ? splits : 1));
    if (p.sched) {
        // persistent blocks, all resident at once (two per CU the stream may use)
        const int64_t nku = (p.K + SK_UNIT - 1) / SK_UNIT;
        const int64_t items = (CM == C_PARTIAL && p.piece > 0)
                                  ? ((int64_t)nt * nku + p.piece - 1) / p.piece
                                  : (int64_t)nt * (CM == C_PARTIAL ? splits : 1) * (TM != BM && p.tri ? 2 : 1);
        const unsigned dgrid = (unsigned)std::min<int64_t>(items, p.cap > 0 ? p.cap : 2 * 240);
        if (CM == C_SUB_LOWER)
            gemm_detail::launch(k_gemm<T, AOP, BOP, CM, SCHED_DYN, TM, TN>, dim3(dgrid), st, p, ea, eb);
        else
            gemm_detail::launch(k_gemm<T, AOP, BOP, CM, SCHED_BOTH, TM, TN>, dim3(dgrid), st, p, ea, eb);
    } else {
        gemm_detail::launch(k_gemm<T, AOP, BOP, CM, SCHED_BOTH, TM, TN>, sgrid, st, p, ea, eb);
    }
    CHOL_LAUNCH_CHECK();
    return CHOL_OK;
}

} // namespace chol
