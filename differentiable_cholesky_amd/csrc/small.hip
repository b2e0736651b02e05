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
// (a, b) fall out of the trailing work at compile time.  Each lane loads the
// entries it owns straight from global memory into registers (all loads in
// flight at once) and stores them back the same way, so a lane only ever
// writes entries it read itself (in-place calls need no ordering between
// lanes).  Per-step broadcasts -- a column of the trailing matrix, a row of L,
// a solved row or column -- go through small double-buffered LDS vectors in
// which column c of a row sits at (c % G) * (E + 1) + c / G, so that every lane
// reads the E entries it needs as one contiguous run; the one padding slot per
// lane column puts the runs of different lane columns (and, with the padded
// per-matrix stride, of different matrices in a wave) on different LDS banks.
#include "common.hpp"

namespace chol {

template <int G_, int E_> struct TileShape {
    static constexpr int G = G_;
    static constexpr int E = E_;
    static constexpr int NP = G * E;                      // padded edge
    static constexpr int LPM = G * G;                     // lanes per matrix
    static constexpr int THREADS = LPM < 64 ? 64 : LPM;   // one wavefront at least
    static constexpr int MPB = THREADS / LPM;             // matrices per block
    static constexpr int EP = E + 1;                      // LDS slots per lane column (one pad)
    static constexpr int VS = G * EP;                     // LDS vector stride per matrix
};

// Waves per SIMD the register allocation aims for (the scheduler otherwise
// trades occupancy for overlap of the fully unrolled steps): a tile's values
// take E*E/2 (factor) or about 2*E*E (adjoint) registers per lane.
template <typename T, int G, int E> struct TileWaves {
    static constexpr int words = (int)(sizeof(T) / 4);
    static constexpr int tile = E * E * words;
    static constexpr int factor = tile <= 32 ? 8 : (tile <= 64 ? 5 : 2);
    static constexpr int adjoint = tile <= 16 ? 8 : (tile <= 32 ? 4 : (tile <= 64 ? 3 : 1));
};

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

// Pivot arithmetic.  Every pivot step of the column loops waits on it, so it
// is kept short: 1 / sqrt(d) from the hardware reciprocal square root, and in
// fp64 one Newton step y += y (1 - d y^2) / 2 on it (which squares the
// approximation's relative error), then sqrt(d) = d / sqrt(d); the
// reciprocal likewise (hardware estimate, and in fp64 two Newton steps
// y += y (1 - x y)).  About one ulp either way -- far inside the parity
// tolerances -- against ~25 dependent instructions for the correctly rounded
// fp64 square root and reciprocal.
template <typename T> struct Piv;
template <> struct Piv<double> {
    static __device__ __forceinline__ void sqrt_rsqrt(double d, double &sq, double &rs)
    {
        const double y = __builtin_amdgcn_rsq(d);
        const double h = __builtin_fma(-d * y, y, 1.0);
        rs = __builtin_fma(0.5 * y, h, y);
        sq = d * rs;
    }
    static __device__ __forceinline__ double rcp(double x)
    {
        double y = __builtin_amdgcn_rcp(x);
        y = __builtin_fma(y, __builtin_fma(-x, y, 1.0), y);
        return __builtin_fma(y, __builtin_fma(-x, y, 1.0), y);
    }
};
template <> struct Piv<float> {
    static __device__ __forceinline__ void sqrt_rsqrt(float d, float &sq, float &rs)
    {
        rs = __builtin_amdgcn_rsqf(d);
        sq = d * rs;
    }
    static __device__ __forceinline__ float rcp(float x) { return __builtin_amdgcn_rcpf(x); }
};

// 16-byte global access for fp32 tiles whose edge is a multiple of 4 and whose
// rows and matrices start on 16-byte boundaries.  A quad of lanes (lc = 0..3,
// same lr) then moves one 64-byte run of a row per instruction: lane lc moves
// the 4 columns 4q .. 4q+3 with q = lc + 4q', and a 4 x 4 transpose across the
// quad turns that into the cyclic ownership above (lane lc holds columns
// lc + 4b, b = c + 4q', c = 0..3).
__device__ __forceinline__ float dpp_xor1(float v)
{
    return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0xB1, 0xF, 0xF, false));
}
__device__ __forceinline__ float dpp_xor2(float v)
{
    return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x4E, 0xF, 0xF, false));
}
// On entry lane l of the quad holds w[e] = M[l][e]; on exit w[e] = M[e][l].
// Two butterfly stages (partners l^1, then l^2); every lane of the quad must
// execute it.
__device__ __forceinline__ void quad_transpose(float (&w)[4], int l)
{
    const bool odd = (l & 1) != 0, hi = (l & 2) != 0;
    const float p1 = dpp_xor1(w[1]), p0 = dpp_xor1(w[0]), p3 = dpp_xor1(w[3]), p2 = dpp_xor1(w[2]);
    const float t0 = odd ? p1 : w[0];
    const float t1 = odd ? w[1] : p0;
    const float t2 = odd ? p3 : w[2];
    const float t3 = odd ? w[3] : p2;
    const float q2 = dpp_xor2(t2), q3 = dpp_xor2(t3), q0 = dpp_xor2(t0), q1 = dpp_xor2(t1);
    w[0] = hi ? q2 : t0;
    w[1] = hi ? q3 : t1;
    w[2] = hi ? t2 : q0;
    w[3] = hi ? t3 : q1;
}

// Load the lower blocks of one fp32 tile (edge 4E) into the cyclic layout:
// dst[a][b] for b <= a; entries right of the diagonal come back as zero.  All
// loads are issued before the first transpose needs one.
template <int E>
__device__ __forceinline__ void vec_load_lower(float (&dst)[E][E], const float *M, int64_t ld, bool mv, int lr,
                                               int lc)
{
    float4 raw[E][E / 4];
#pragma unroll
    for (int a = 0; a < E; ++a) {
        const int r = lr + 4 * a;
#pragma unroll
        for (int qq = 0; qq < E / 4; ++qq) {
            raw[a][qq] = make_float4(0.f, 0.f, 0.f, 0.f);
            const int q = lc + 4 * qq;
            if (16 * qq <= 4 * a + 3 && mv && 4 * q <= r)
                raw[a][qq] = *reinterpret_cast<const float4 *>(M + (int64_t)r * ld + 4 * q);
        }
    }
#pragma unroll
    for (int a = 0; a < E; ++a) {
#pragma unroll
        for (int qq = 0; qq < E / 4; ++qq) {
            if (16 * qq > 4 * a + 3)
                continue;                       // the whole group is right of the diagonal
            float w[4] = {raw[a][qq].x, raw[a][qq].y, raw[a][qq].z, raw[a][qq].w};
            quad_transpose(w, lc);
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                const int b = c + 4 * qq;
                if (b > a)
                    continue;
                // diagonal block: keep column lc + 4a <= row lr + 4a only
                dst[a][b] = (b < a || lc <= lr) ? w[c] : 0.f;
            }
        }
    }
}

// Store whole rows of one fp32 tile from the cyclic layout.  src(a, b) gives
// the value of entry (lr + 4a, lc + 4b); entries right of the diagonal must
// already be zero in src.
template <int E, typename F>
__device__ __forceinline__ void vec_store(float *M, int64_t ld, bool mv, int lr, int lc, F &&src)
{
#pragma unroll
    for (int a = 0; a < E; ++a) {
        const int r = lr + 4 * a;
#pragma unroll
        for (int qq = 0; qq < E / 4; ++qq) {
            const int q = lc + 4 * qq;
            if (16 * qq > 4 * a + 3) {
                if (mv)
                    *reinterpret_cast<float4 *>(M + (int64_t)r * ld + 4 * q) = make_float4(0.f, 0.f, 0.f, 0.f);
                continue;
            }
            float w[4];
#pragma unroll
            for (int c = 0; c < 4; ++c)
                w[c] = src(a, c + 4 * qq);
            quad_transpose(w, lc);
            if (mv)
                *reinterpret_cast<float4 *>(M + (int64_t)r * ld + 4 * q) = make_float4(w[0], w[1], w[2], w[3]);
        }
    }
}

// ------------------------------------------------------------------------
// Factor: right-looking column loop on register-resident tiles.
// ------------------------------------------------------------------------
template <typename T, int G, int E, bool VEC>
__global__ void __launch_bounds__((TileShape<G, E>::THREADS))
__attribute__((amdgpu_waves_per_eu(TileWaves<T, G, E>::factor)))
k_potrf_tile(int n, int64_t batch, const T *A, int64_t lda, int64_t sA,
             T *L, int64_t ldl, int64_t sL, int32_t *info, int info_mode, int64_t info_base)
{
    typedef TileShape<G, E> S;
    constexpr int MPB = S::MPB, EP = S::EP, VS = S::VS;
    __shared__ T colbuf[2 * MPB * VS];

    const int tid = threadIdx.x;
    const int g = tid / S::LPM;
    const int lr = (tid % S::LPM) / G;
    const int lc = tid % G;
    const int64_t mat = (int64_t)blockIdx.x * MPB + g;
    const bool mv = mat < batch;

    static_assert(!VEC || (G == 4 && E % 4 == 0 && sizeof(T) == 4), "16-byte path: fp32, G = 4");
    // global -> registers (lower blocks only; padding is the identity)
    T x[E][E];
    if constexpr (VEC) {
        vec_load_lower<E>(x, A + (mv ? mat * sA : 0), lda, mv, lr, lc);
    } else {
        const T *Am = A + (mv ? mat * sA : 0);
#pragma unroll
        for (int a = 0; a < E; ++a)
#pragma unroll
            for (int b = 0; b <= a; ++b) {
                const int i = lr + G * a, k = lc + G * b;
                x[a][b] = (i == k) ? T(1) : T(0);
                if (mv && i < n && k <= i)
                    x[a][b] = Am[(int64_t)i * lda + k];
            }
    }

    int fail = 0;
#pragma unroll
    for (int t_ = 0; t_ < E; ++t_) {
        const int jb = t_;
#pragma unroll 1
        for (int u_ = 0; u_ < G; ++u_) {
            const int jr = u_;
            const int j = jb * G + jr;
            T *cb = colbuf + ((j & 1) * MPB + g) * VS;
            // owners of column j publish it (unscaled); rows lr + G*a
            if (lc == jr) {
    #pragma unroll
                for (int a = jb; a < E; ++a)
                    cb[lr * EP + a] = x[a][jb];
            }
            __syncthreads();
            const T d = cb[jr * EP + jb];
            T u[E], v[E];
    #pragma unroll
            for (int a = jb; a < E; ++a)
                u[a] = cb[lr * EP + a];
    #pragma unroll
            for (int b = jb; b < E; ++b)
                v[b] = cb[lc * EP + b];
            if (!(d > T(0)) && fail == 0)
                fail = j + 1;
            T sq, rs;
            Piv<T>::sqrt_rsqrt(d, sq, rs);
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

    // registers -> global: lower triangle and zeroed upper triangle
    if constexpr (VEC) {
        vec_store<E>(L + (mv ? mat * sL : 0), ldl, mv, lr, lc, [&](int a, int b) {
            return (b < a || (b == a && lc <= lr)) ? x[a][b] : 0.f;
        });
        if (mv && lr == 0 && lc == 0)
            write_info(info, mat, fail, info_mode, info_base);
    } else if (mv) {
        T *Lm = L + mat * sL;
#pragma unroll
        for (int a = 0; a < E; ++a)
#pragma unroll
            for (int b = 0; b < E; ++b) {
                const int i = lr + G * a, k = lc + G * b;
                if (i < n && k < n)
                    Lm[(int64_t)i * ldl + k] = (b <= a && k <= i) ? x[a][b] : T(0);
            }
        if (lr == 0 && lc == 0)
            write_info(info, mat, fail, info_mode, info_base);
    }
}

// ------------------------------------------------------------------------
// Adjoint: M = L^T tril(adj_L) (lower part), Psi = P + P^T with P = Phi(M)
// (M's lower part mirrored, diagonal M_ii), V = Psi L^{-1}, Z = L^{-T} V
// (lower part), lower(adj_A) (+)= Phi(Z).  L and adj_L stay in registers; each
// step publishes the one row of L it needs and the vector it produces.
// adj_A may be adj_L itself when accumulate == 0.
// ------------------------------------------------------------------------
template <typename T, int G, int E>
__global__ void __launch_bounds__((TileShape<G, E>::THREADS))
__attribute__((amdgpu_waves_per_eu(TileWaves<T, G, E>::adjoint)))
k_potrf_adj_tile(int n, int64_t batch, const T *L, int64_t ldl, int64_t sL,
                 const T *adjL, int64_t ldal, int64_t sAL,
                 T *adjA, int64_t ldaa, int64_t sAA, int accumulate)
{
    typedef TileShape<G, E> S;
    // unpadded vectors (column c at (c % G) * E + c / G): the padded layout of
    // the factor measured slower here
    constexpr int NP = S::NP, MPB = S::MPB, EP = E, VS = NP;
    static_assert(S::LPM <= 64, "one matrix per wavefront at most (lane shuffles)");
    __shared__ T rowb[2 * MPB * VS];    // a row of L
    __shared__ T vecb[2 * MPB * VS];    // a row of adj_L, a column of V or a row of Z
    __shared__ T dinv[MPB * NP];        // 1 / L_jj

    const int tid = threadIdx.x;
    const int g = tid / S::LPM;
    const int lr = (tid % S::LPM) / G;
    const int lc = tid % G;
    const int64_t mat = (int64_t)blockIdx.x * MPB + g;
    const bool mv = mat < batch;

    // global -> registers: L (identity padding) and tril(adj_L) (zero padding)
    T lw[E][E], bw[E][E];
    {
        const T *Lm = L + (mv ? mat * sL : 0);
        const T *Bm = adjL + (mv ? mat * sAL : 0);
#pragma unroll
        for (int a = 0; a < E; ++a)
#pragma unroll
            for (int b = 0; b <= a; ++b) {
                const int i = lr + G * a, k = lc + G * b;
                const bool in = mv && i < n && k <= i;
                lw[a][b] = (i == k) ? T(1) : T(0);
                bw[a][b] = T(0);
                if (in) {
                    lw[a][b] = Lm[(int64_t)i * ldl + k];
                    bw[a][b] = Bm[(int64_t)i * ldal + k];
                }
            }
    }
    if (lr == lc) {
#pragma unroll
        for (int a = 0; a < E; ++a)
            dinv[g * NP + lr + G * a] = Piv<T>::rcp(lw[a][a]);
    }

    T p[E][E];
#pragma unroll
    for (int a = 0; a < E; ++a)
#pragma unroll
        for (int b = 0; b < E; ++b)
            p[a][b] = T(0);

    // M_ij = sum_{k >= i} L_ki adjL_kj (i >= j): row k of L and of adj_L per step
#pragma unroll
    for (int t_ = 0; t_ < E; ++t_) {
        const int kb = t_;
#pragma unroll 1
        for (int u_ = 0; u_ < G; ++u_) {
            const int kr = u_;
            const int k = kb * G + kr;
            T *rb = rowb + ((k & 1) * MPB + g) * VS;
            T *vb = vecb + ((k & 1) * MPB + g) * VS;
            if (lr == kr) {
    #pragma unroll
                for (int b = 0; b < E; ++b) {
                    rb[lc * EP + b] = (b <= kb) ? lw[kb][b] : T(0);
                    vb[lc * EP + b] = (b <= kb) ? bw[kb][b] : T(0);
                }
            }
            __syncthreads();
            T lk[E], ak[E];
    #pragma unroll
            for (int a = 0; a <= kb; ++a)
                lk[a] = rb[lr * EP + a];          // L[k][lr + G a]
    #pragma unroll
            for (int b = 0; b <= kb; ++b)
                ak[b] = vb[lc * EP + b];          // adjL[k][lc + G b]
    #pragma unroll
            for (int a = 0; a <= kb; ++a)
    #pragma unroll
                for (int b = 0; b <= a; ++b)
                    p[a][b] += lk[a] * ak[b];
        }
    }

    // Psi: the upper entries are M's transposed lower entries, held by lane
    // (lc, lr) of the same matrix at block (b, a)
    {
        const int src = (tid / S::LPM) * S::LPM % 64 + lc * G + lr;
#pragma unroll
        for (int a = 0; a < E; ++a) {
#pragma unroll
            for (int b = a + 1; b < E; ++b)
                p[a][b] = __shfl(p[b][a], src, 64);
            const T t = __shfl(p[a][a], src, 64);
            if (lr < lc)
                p[a][a] = t;
        }
    }
    __syncthreads();

    // V = Psi L^{-1}  (V L = Psi), columns j = NP-1 .. 0:
    //   V[:, j] = R[:, j] / L_jj ;  R[:, k] -= V[:, j] L_jk  (k < j)
#pragma unroll
    for (int t_ = 0; t_ < E; ++t_) {
        const int jb = E - 1 - t_;
#pragma unroll 1
        for (int u_ = 0; u_ < G; ++u_) {
            const int jr = G - 1 - u_;
            const int j = jb * G + jr;
            T *rb = rowb + ((j & 1) * MPB + g) * VS;
            T *vb = vecb + ((j & 1) * MPB + g) * VS;
            if (lc == jr) {
                const T r = dinv[g * NP + j];
    #pragma unroll
                for (int a = 0; a < E; ++a) {
                    p[a][jb] *= r;
                    vb[lr * EP + a] = p[a][jb];
                }
            }
            if (lr == jr) {
    #pragma unroll
                for (int b = 0; b <= jb; ++b)
                    rb[lc * EP + b] = lw[jb][b];
            }
            __syncthreads();
            T u[E], lj[E];
    #pragma unroll
            for (int a = 0; a < E; ++a)
                u[a] = vb[lr * EP + a];           // V[lr + G a][j]
    #pragma unroll
            for (int b = 0; b <= jb; ++b)
                lj[b] = rb[lc * EP + b];          // L[j][lc + G b]; zero right of j
            if (lc == jr)
                lj[jb] = T(0);                   // the solved column itself
    #pragma unroll
            for (int a = 0; a < E; ++a)
    #pragma unroll
                for (int b = 0; b <= jb; ++b)
                    p[a][b] -= u[a] * lj[b];
        }
    }
    __syncthreads();

    // the accumulated output is read while Z is solved
    T acc[E][E];
    if (accumulate && mv) {
        const T *Gm = adjA + mat * sAA;
#pragma unroll
        for (int a = 0; a < E; ++a)
#pragma unroll
            for (int b = 0; b <= a; ++b) {
                const int i = lr + G * a, k = lc + G * b;
                acc[a][b] = (i < n && k <= i) ? Gm[(int64_t)i * ldaa + k] : T(0);
            }
    }

    // Z = L^{-T} V (L^T Z = V), lower part, rows i = NP-1 .. 0:
    //   Z[i, :] = R[i, :] / L_ii ;  R[t, :] -= L_it Z[i, :]  (t < i)
#pragma unroll
    for (int t_ = 0; t_ < E; ++t_) {
        const int ib = E - 1 - t_;
#pragma unroll 1
        for (int u_ = 0; u_ < G; ++u_) {
            const int ir = G - 1 - u_;
            const int i = ib * G + ir;
            T *rb = rowb + ((i & 1) * MPB + g) * VS;
            T *vb = vecb + ((i & 1) * MPB + g) * VS;
            if (lr == ir) {
                const T r = dinv[g * NP + i];
    #pragma unroll
                for (int b = 0; b <= ib; ++b) {
                    p[ib][b] *= r;
                    vb[lc * EP + b] = p[ib][b];
                    rb[lc * EP + b] = lw[ib][b];
                }
            }
            __syncthreads();
            T w[E], li[E];
    #pragma unroll
            for (int b = 0; b <= ib; ++b)
                w[b] = vb[lc * EP + b];           // Z[i][lc + G b]
    #pragma unroll
            for (int a = 0; a <= ib; ++a)
                li[a] = rb[lr * EP + a];          // L[i][lr + G a]; zero right of i
            if (lr == ir)
                li[ib] = T(0);                   // the solved row itself
    #pragma unroll
            for (int a = 0; a <= ib; ++a)
    #pragma unroll
                for (int b = 0; b <= a; ++b)
                    p[a][b] -= li[a] * w[b];
        }
    }

    // G = Phi(Z): halve the diagonal; lower triangle only
    if (mv) {
        T *Gm = adjA + mat * sAA;
#pragma unroll
        for (int a = 0; a < E; ++a)
#pragma unroll
            for (int b = 0; b <= a; ++b) {
                const int i = lr + G * a, k = lc + G * b;
                if (i < n && k <= i) {
                    const T gv = (i == k) ? p[a][b] * T(0.5) : p[a][b];
                    Gm[(int64_t)i * ldaa + k] = accumulate ? acc[a][b] + gv : gv;
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

// The sum reduction with the same ownership: y = sum_k a_k, written by lane
// 0 only; reverse: a_bar_k += y_bar for every k, with y_bar read by lane 0 and
// published to every lane first (the tile_sum adjoint's broadcast of the
// upstream gradient through shared scratch that Warp issue #1374 describes).
template <typename T>
__global__ void __launch_bounds__(64)
k_wave_sum(int n, const T *a, T *y, const T *ybar, T *abar, int staging)
{
    __shared__ T sa[64], sy[1];
    const int l = threadIdx.x;
    T av = T(0);
    if (staging) {
        sa[l] = l < n ? a[l] : T(0);
        __syncthreads();
        av = sa[l];
    } else if (l < n) {
        av = a[l];
    }
    T s = av;
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1)
        s += __shfl_xor(s, off, 64);
    if (l == 0)
        y[0] = s;
    T yb = (l == 0) ? ybar[0] : T(0);
    if (staging) {
        if (l == 0)
            sy[0] = yb;
        __syncthreads();
        yb = sy[0];
    } else {
        yb = __shfl(yb, 0, 64);
    }
    if (l < n)
        abar[l] += yb;
}

// ------------------------------------------------------------------------
// Diagonal tile of the blocked factor with its inverse (one 128-edge tile per
// 256-thread block, lane grid 16 x 16).  The inverse X = L^{-1} is built row
// by row alongside the factor: once L_jj is known, the lanes of row j of X
// scale it by 1 / L_jj and publish it, and every row t > j takes
// R_t -= L_tj X_j, with L_tj kept in registers from factor step j.  The
// inverse runs one step behind the factor, so that the column of factor step
// j and the row j-1 of X are published together and each step needs one
// barrier.  No tile-sized LDS buffer is needed, so the kernel fits beside the
// blocks of a running matrix-core product.  X is written whole (n x n, zeros
// above its diagonal) to Xo, where the panel solve of the blocked
// factorisation reads it as a plain operand.
template <typename T>
__global__ void __launch_bounds__(256)
k_potrf_inv_tile(int n, T *W, int64_t ld, int32_t *info, int info_mode, int64_t info_base, T *Xo, int64_t ldx)
{
    constexpr int G = 16, E = 8, EP = E + 1, VS = G * EP;
    // on the critical path of the factorisation, beside blocks of the trailing
    // update: its waves win instruction arbitration on their SIMDs
    __builtin_amdgcn_s_setprio(3);
    __shared__ T colbuf[2 * VS];
    __shared__ T rowbuf[2 * VS];
    const int tid = threadIdx.x, lr = tid / G, lc = tid % G;

    T x[E][E], y[E][E];
#pragma unroll
    for (int a = 0; a < E; ++a)
#pragma unroll
        for (int b = 0; b <= a; ++b) {
            const int i = lr + G * a, k = lc + G * b;
            x[a][b] = (i == k) ? T(1) : T(0);
            if (i < n && k <= i)
                x[a][b] = W[(int64_t)i * ld + k];
            y[a][b] = (i == k) ? T(1) : T(0);
        }

    // row p of X (block pb, lane row pr): X_p = R_p / L_pp, published at the
    // lane columns; after the barrier every row t > p takes R_t -= L_tp X_p
    T lt[E];                  // L_tp for this lane's rows t = lr + G a (zero for t <= p)
    T rs_p = T(0);            // 1 / L_pp
#pragma unroll
    for (int a = 0; a < E; ++a)
        lt[a] = T(0);
    auto publish_row = [&](int pb, int pr, T *rb) {
        if (lr == pr) {
#pragma unroll
            for (int b = 0; b <= pb; ++b) {
                y[pb][b] *= rs_p;
                rb[lc * EP + b] = y[pb][b];
            }
        }
    };
    auto apply_row = [&](int pb, const T *rb) {
        T w[E];
#pragma unroll
        for (int b = 0; b <= pb; ++b)
            w[b] = rb[lc * EP + b];
#pragma unroll
        for (int a = pb; a < E; ++a)
#pragma unroll
            for (int b = 0; b <= pb; ++b)
                y[a][b] -= lt[a] * w[b];
    };

    int fail = 0;
#pragma unroll
    for (int jb = 0; jb < E; ++jb) {
#pragma unroll 1
        for (int jr = 0; jr < G; ++jr) {
            const int j = jb * G + jr;
            T *cb = colbuf + (j & 1) * VS;
            T *rb = rowbuf + ((j + 1) & 1) * VS;   // row j - 1 of X
            if (lc == jr) {
#pragma unroll
                for (int a = jb; a < E; ++a)
                    cb[lr * EP + a] = x[a][jb];
            }
            // row j - 1 of X: in block jb - 1 at lane row G - 1 when jr == 0
            if (jr > 0)
                publish_row(jb, jr - 1, rb);
            else if (jb > 0)
                publish_row(jb - 1, G - 1, rb);
            __syncthreads();
            if (jr > 0)
                apply_row(jb, rb);
            else if (jb > 0)
                apply_row(jb - 1, rb);
            const T d = cb[jr * EP + jb];
            T u[E], v[E];
#pragma unroll
            for (int a = jb; a < E; ++a)
                u[a] = cb[lr * EP + a];
#pragma unroll
            for (int b = jb; b < E; ++b)
                v[b] = cb[lc * EP + b];
            if (!(d > T(0)) && fail == 0)
                fail = j + 1;
            T sq, rs;
            Piv<T>::sqrt_rsqrt(d, sq, rs);
            const T rd = rs * rs;
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
            // L_tj for the inverse step of row j (next iteration)
#pragma unroll
            for (int a = jb; a < E; ++a)
                lt[a] = u[a] * rs;
            rs_p = rs;
        }
    }
    // the last row of X has no rows below it: only its scaling is left
    if (lr == G - 1) {
#pragma unroll
        for (int b = 0; b < E; ++b)
            y[E - 1][b] *= rs_p;
    }

    // L (lower triangle of the tile) and X (whole, to Xo)
#pragma unroll
    for (int a = 0; a < E; ++a)
#pragma unroll
        for (int b = 0; b < E; ++b) {
            const int i = lr + G * a, k = lc + G * b;
            if (i >= n || k >= n)
                continue;
            const bool low = b <= a && k <= i;
            if (low)
                W[(int64_t)i * ld + k] = x[a][b];
            Xo[(int64_t)i * ldx + k] = low ? y[a][b] : T(0);
        }
    if (tid == 0)
        write_info(info, 0, fail, info_mode, info_base);
}

// ------------------------------------------------------------------ hosts ----
// The 16-byte path needs every row start of every matrix on a 16-byte boundary.
static inline bool rows_aligned16(const void *p, int64_t ld, int64_t stride)
{
    return ((uintptr_t)p % 16) == 0 && ld % 4 == 0 && stride % 4 == 0;
}

template <typename T, int G, int E>
static chol_status launch_potrf_tile(int n, int64_t batch, const T *A, int64_t lda, int64_t sA,
                                     T *L, int64_t ldl, int64_t sL, int32_t *info, int info_mode,
                                     int64_t info_base, hipStream_t st)
{
    typedef TileShape<G, E> S;
    const int64_t blocks = (batch + S::MPB - 1) / S::MPB;
    if constexpr (sizeof(T) == 4 && G == 4 && E % 4 == 0) {
        if (n == S::NP && rows_aligned16(A, lda, sA) && rows_aligned16(L, ldl, sL)) {
            hipLaunchKernelGGL((k_potrf_tile<T, G, E, true>), dim3((unsigned)blocks), dim3(S::THREADS), 0, st,
                               n, batch, A, lda, sA, L, ldl, sL, info, info_mode, info_base);
            CHOL_LAUNCH_CHECK();
            return CHOL_OK;
        }
    }
    hipLaunchKernelGGL((k_potrf_tile<T, G, E, false>), dim3((unsigned)blocks), dim3(S::THREADS), 0, st,
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

// Diagonal tile of the blocked factor: n <= 128, one 256-thread block; with
// `inv`, the tile's inverse is also formed, whole (zeros above its diagonal),
// into inv with leading dimension ldinv.
template <typename T>
chol_status diag_potrf(int n, T *W, int64_t ld, int32_t *info, int info_mode, int64_t info_base, T *inv,
                       int64_t ldinv, hipStream_t st)
{
    if (inv) {
        hipLaunchKernelGGL((k_potrf_inv_tile<T>), dim3(1), dim3(256), 0, st, n, W, ld, info, info_mode, info_base,
                           inv, ldinv);
        CHOL_LAUNCH_CHECK();
        return CHOL_OK;
    }
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

template <typename T>
chol_status wave_sum(int n, const T *a, T *y, const T *ybar, T *abar, int staging, hipStream_t st)
{
    hipLaunchKernelGGL((k_wave_sum<T>), dim3(1), dim3(64), 0, st, n, a, y, ybar, abar, staging);
    CHOL_LAUNCH_CHECK();
    return CHOL_OK;
}

// Loads this file's kernels on the current device (their code object is
// otherwise loaded on first launch).
chol_status small_load()
{
    hipFuncAttributes a;
    if (hip_failed(hipFuncGetAttributes(&a, reinterpret_cast<const void *>(&k_potrf_tile<float, 4, 8, true>))))
        return CHOL_ERR_HIP;
    return CHOL_OK;
}

#define CHOL_INST(T)                                                                                      \
    template chol_status small_potrf<T>(int, int64_t, const T *, int64_t, int64_t, T *, int64_t, int64_t, \
                                        int32_t *, int, int64_t, hipStream_t);                            \
    template chol_status diag_potrf<T>(int, T *, int64_t, int32_t *, int, int64_t, T *, int64_t,          \
                                       hipStream_t);                                                      \
    template chol_status small_potrf_adjoint<T>(int, int64_t, const T *, int64_t, int64_t, const T *,     \
                                                int64_t, int64_t, T *, int64_t, int64_t, int, hipStream_t); \
    template chol_status wave_dot<T>(int, const T *, const T *, T *, const T *, T *, T *, int, hipStream_t); \
    template chol_status wave_sum<T>(int, const T *, T *, const T *, T *, int, hipStream_t);
CHOL_INST(float)
CHOL_INST(double)
#undef CHOL_INST

} // namespace chol
