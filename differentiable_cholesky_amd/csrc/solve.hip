// Solve with the factor for n <= 64, batched: X = (L L^T)^{-1} B by forward
// and back substitution against L, and its adjoint
//   adj_B = (L L^T)^{-1} adj_X,   adj_L (+)= -tril((adj_B X^T + X adj_B^T) L).
// (The factor is returned without a solve -- jaxmg documentation, "Cholesky
// factorization"; this is the solve it is computed for, made of the two
// triangular solves against L that Warp issue #1316's resolution comment
// names for the adjoint.)
//
// Design: one matrix per wavefront, lane i owning row i (n <= 64).  L's lower
// triangle is staged in LDS (rows padded by one element); the right-hand side
// is taken CH columns at a time, lane i holding row i of the chunk in
// registers.  Substitution step j: lane j scales its row by 1 / L_jj, the
// row is made uniform with readlane (every lane then reads the value lane j
// produced, in a scalar register), and the lanes it concerns subtract their
// L entry times it.
#include <hip/hip_runtime.h>

#include <algorithm>

#include "common.hpp"
#include "profile.hpp"

namespace chol {
namespace {

constexpr int CH = 8;   // right-hand-side columns per pass

template <int N, typename T> constexpr int waves_per_block() { return (sizeof(T) == 8 && N == 64) ? 2 : 4; }

// value of v in lane j (j uniform), in every lane
__device__ __forceinline__ float from_lane(float v, int j)
{
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), j));
}
__device__ __forceinline__ double from_lane(double v, int j)
{
    const long long b = __double_as_longlong(v);
    const int lo = __builtin_amdgcn_readlane((int)(b & 0xffffffffll), j);
    const int hi = __builtin_amdgcn_readlane((int)(b >> 32), j);
    return __longlong_as_double(((long long)hi << 32) | (unsigned int)lo);
}

// the wave's LDS writes are complete and visible to all of its lanes (one
// wavefront per matrix: no barrier with the block's other waves is needed)
__device__ __forceinline__ void wave_lds_sync()
{
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "workgroup");
    __builtin_amdgcn_wave_barrier();
}

// lower triangle of the wave's L into S (row pitch N + 1), zeros elsewhere
template <typename T, int N>
__device__ __forceinline__ void stage_lower(int n, const T *Lb, int64_t ldl, T *S)
{
    constexpr int LP = N + 1;
    const int lane = threadIdx.x % 64;
    for (int e = lane; e < N * N; e += 64) {
        const int i = e / N, j = e % N;
        S[i * LP + j] = (i < n && j <= i) ? Lb[(int64_t)i * ldl + j] : T(0);
    }
}

// x (lane i: row i of a chunk of cw columns) <- (L L^T)^{-1} x, with rd = 1 / L_ii
template <typename T, int N>
__device__ __forceinline__ void substitute(int n, int cw, const T *S, T rd, T (&x)[CH])
{
    constexpr int LP = N + 1;
    const int lane = threadIdx.x % 64;
    // forward: L y = x
    for (int j = 0; j < n; ++j) {
        if (lane == j) {
#pragma unroll
            for (int c = 0; c < CH; ++c)
                x[c] *= rd;
        }
        const T l = lane > j && lane < n ? S[lane * LP + j] : T(0);
#pragma unroll
        for (int c = 0; c < CH; ++c) {
            if (c < cw) {
                const T y = from_lane(x[c], j);
                x[c] -= l * y;
            }
        }
    }
    // backward: L^T x = y
    for (int j = n - 1; j >= 0; --j) {
        if (lane == j) {
#pragma unroll
            for (int c = 0; c < CH; ++c)
                x[c] *= rd;
        }
        const T l = lane < j ? S[j * LP + lane] : T(0);
#pragma unroll
        for (int c = 0; c < CH; ++c) {
            if (c < cw) {
                const T y = from_lane(x[c], j);
                x[c] -= l * y;
            }
        }
    }
}

template <typename T, int N>
__global__ void __launch_bounds__(256)
k_potrs_small(int n, int nrhs, int64_t batch, const T *L, int64_t ldl, int64_t sL, const T *B, int64_t ldb,
              int64_t sB, T *X, int64_t ldx, int64_t sX)
{
    constexpr int WPB = waves_per_block<N, T>(), LP = N + 1;
    __shared__ T lds[WPB * N * LP];
    const int lane = threadIdx.x % 64, w = threadIdx.x / 64;
    if (w >= WPB)
        return;
    const int64_t b = (int64_t)blockIdx.x * WPB + w;
    if (b >= batch)
        return;            // one wave per matrix, no barrier between waves
    T *S = lds + w * N * LP;
    stage_lower<T, N>(n, L + b * sL, ldl, S);
    wave_lds_sync();
    const T rd = lane < n ? T(1) / S[lane * LP + lane] : T(0);
    const T *Bb = B + b * sB;
    T *Xb = X + b * sX;
    for (int c0 = 0; c0 < nrhs; c0 += CH) {
        const int cw = min(CH, nrhs - c0);
        T x[CH];
#pragma unroll
        for (int c = 0; c < CH; ++c)
            x[c] = (lane < n && c < cw) ? Bb[(int64_t)lane * ldb + c0 + c] : T(0);
        substitute<T, N>(n, cw, S, rd, x);
        if (lane < n) {
#pragma unroll
            for (int c = 0; c < CH; ++c)
                if (c < cw)
                    Xb[(int64_t)lane * ldx + c0 + c] = x[c];
        }
    }
}

// lower(adj_L) (+)= -tril(S P + X Q) with P = X^T L, Q = S^T L (S = adj_B),
// i.e. G_ij = -sum_c (S_ic P_cj + X_ic Q_cj) for j <= i.  Lane i accumulates
// row i of G in registers over chunks of columns c; per chunk, lane j forms
// P_cj and Q_cj (sums over t >= j of X_tc L_tj, S_tc L_tj) and publishes them.
template <typename T, int N>
__global__ void __launch_bounds__(256)
k_potrs_adj_small(int n, int nrhs, int64_t batch, const T *L, int64_t ldl, int64_t sL, const T *X, int64_t ldx,
                  int64_t sX, const T *Sg, int64_t lds_, int64_t sS, T *adjL, int64_t ldal, int64_t sAL,
                  int accumulate)
{
    constexpr int WPB = waves_per_block<N, T>(), LP = N + 1;
    constexpr int PER_WAVE = N * LP + 4 * N * CH;
    __shared__ T lds[WPB * PER_WAVE];
    const int lane = threadIdx.x % 64, w = threadIdx.x / 64;
    if (w >= WPB)
        return;
    const int64_t b = (int64_t)blockIdx.x * WPB + w;
    if (b >= batch)
        return;
    T *Ls = lds + w * PER_WAVE;
    T *Xs = Ls + N * LP;            // [t][c]
    T *Ss = Xs + N * CH;
    T *Ps = Ss + N * CH;            // [c][j]
    T *Qs = Ps + N * CH;
    stage_lower<T, N>(n, L + b * sL, ldl, Ls);
    const T *Xb = X + b * sX, *Sb = Sg + b * sS;
    T g[N];
#pragma unroll
    for (int j = 0; j < N; ++j)
        g[j] = T(0);
    for (int c0 = 0; c0 < nrhs; c0 += CH) {
        const int cw = min(CH, nrhs - c0);
        T xr[CH], sr[CH];
#pragma unroll
        for (int c = 0; c < CH; ++c) {
            const bool in = lane < n && c < cw;
            xr[c] = in ? Xb[(int64_t)lane * ldx + c0 + c] : T(0);
            sr[c] = in ? Sb[(int64_t)lane * lds_ + c0 + c] : T(0);
        }
        if (lane < N) {
#pragma unroll
            for (int c = 0; c < CH; ++c) {
                Xs[lane * CH + c] = xr[c];
                Ss[lane * CH + c] = sr[c];
            }
        }
        wave_lds_sync();
        // lane j: P_cj, Q_cj
        T pc[CH], qc[CH];
#pragma unroll
        for (int c = 0; c < CH; ++c)
            pc[c] = qc[c] = T(0);
        if (lane < n) {
            for (int t = lane; t < n; ++t) {
                const T l = Ls[t * LP + lane];
#pragma unroll
                for (int c = 0; c < CH; ++c) {
                    pc[c] += Xs[t * CH + c] * l;
                    qc[c] += Ss[t * CH + c] * l;
                }
            }
        }
        wave_lds_sync();
        if (lane < N) {
#pragma unroll
            for (int c = 0; c < CH; ++c) {
                Ps[c * N + lane] = pc[c];
                Qs[c * N + lane] = qc[c];
            }
        }
        wave_lds_sync();
        // lane i: g_ij += sum_c S_ic P_cj + X_ic Q_cj
#pragma unroll
        for (int c = 0; c < CH; ++c) {
            if (c < cw) {
#pragma unroll
                for (int j = 0; j < N; ++j)
                    g[j] += sr[c] * Ps[c * N + j] + xr[c] * Qs[c * N + j];
            }
        }
        wave_lds_sync();   // Xs / Ps are rewritten by the next chunk
    }
    if (lane < n) {
        T *row = adjL + b * sAL + (int64_t)lane * ldal;
#pragma unroll
        for (int j = 0; j < N; ++j) {
            if (j <= lane && j < n)
                row[j] = accumulate ? row[j] - g[j] : -g[j];
        }
    }
}

template <int N, typename T>
chol_status launch_potrs(int n, int nrhs, int64_t batch, const T *L, int64_t ldl, int64_t sL, const T *B, int64_t ldb,
                         int64_t sB, T *X, int64_t ldx, int64_t sX, hipStream_t st)
{
    constexpr int WPB = waves_per_block<N, T>();
    const int64_t blocks = (batch + WPB - 1) / WPB;
    hipLaunchKernelGGL((k_potrs_small<T, N>), dim3((unsigned)blocks), dim3(64 * WPB), 0, st, n, nrhs, batch, L, ldl,
                       sL, B, ldb, sB, X, ldx, sX);
    CHOL_LAUNCH_CHECK();
    return CHOL_OK;
}

template <int N, typename T>
chol_status launch_potrs_adj(int n, int nrhs, int64_t batch, const T *L, int64_t ldl, int64_t sL, const T *X,
                             int64_t ldx, int64_t sX, const T *S, int64_t lds_, int64_t sS, T *adjL, int64_t ldal,
                             int64_t sAL, int accumulate, hipStream_t st)
{
    constexpr int WPB = waves_per_block<N, T>();
    const int64_t blocks = (batch + WPB - 1) / WPB;
    hipLaunchKernelGGL((k_potrs_adj_small<T, N>), dim3((unsigned)blocks), dim3(64 * WPB), 0, st, n, nrhs, batch, L,
                       ldl, sL, X, ldx, sX, S, lds_, sS, adjL, ldal, sAL, accumulate);
    CHOL_LAUNCH_CHECK();
    return CHOL_OK;
}

} // namespace

template <typename T>
static chol_status potrs_dispatch(int n, int nrhs, int64_t batch, const T *L, int64_t ldl, int64_t sL, const T *B,
                                  int64_t ldb, int64_t sB, T *X, int64_t ldx, int64_t sX, hipStream_t st)
{
    if (n <= 8)
        return launch_potrs<8, T>(n, nrhs, batch, L, ldl, sL, B, ldb, sB, X, ldx, sX, st);
    if (n <= 16)
        return launch_potrs<16, T>(n, nrhs, batch, L, ldl, sL, B, ldb, sB, X, ldx, sX, st);
    if (n <= 32)
        return launch_potrs<32, T>(n, nrhs, batch, L, ldl, sL, B, ldb, sB, X, ldx, sX, st);
    return launch_potrs<64, T>(n, nrhs, batch, L, ldl, sL, B, ldb, sB, X, ldx, sX, st);
}

template <typename T>
chol_status small_potrs(int n, int nrhs, int64_t batch, const T *L, int64_t ldl, int64_t sL, const T *B, int64_t ldb,
                        int64_t sB, T *X, int64_t ldx, int64_t sX, hipStream_t st)
{
    prof::Scope ps(CHOL_K_SOLVE, st, 2.0 * batch * n * n * nrhs);
    return potrs_dispatch<T>(n, nrhs, batch, L, ldl, sL, B, ldb, sB, X, ldx, sX, st);
}

// adj_B = (L L^T)^{-1} adj_X (into adjB, which may be adj_X), then the adj_L term
template <typename T>
chol_status small_potrs_adjoint(int n, int nrhs, int64_t batch, const T *L, int64_t ldl, int64_t sL, const T *X,
                                int64_t ldx, int64_t sX, const T *adjX, int64_t ldax, int64_t saX, T *adjB,
                                int64_t ldab, int64_t saB, T *adjL, int64_t ldal, int64_t saL, int accumulate,
                                hipStream_t st)
{
    {
        prof::Scope ps(CHOL_K_SOLVE, st, 2.0 * batch * n * n * nrhs);
        chol_status s = potrs_dispatch<T>(n, nrhs, batch, L, ldl, sL, adjX, ldax, saX, adjB, ldab, saB, st);
        if (s != CHOL_OK)
            return s;
    }
    prof::Scope ps(CHOL_K_SOLVE_ADJOINT, st, 4.0 * batch * n * n * nrhs);
    if (n <= 8)
        return launch_potrs_adj<8, T>(n, nrhs, batch, L, ldl, sL, X, ldx, sX, adjB, ldab, saB, adjL, ldal, saL,
                                      accumulate, st);
    if (n <= 16)
        return launch_potrs_adj<16, T>(n, nrhs, batch, L, ldl, sL, X, ldx, sX, adjB, ldab, saB, adjL, ldal, saL,
                                       accumulate, st);
    if (n <= 32)
        return launch_potrs_adj<32, T>(n, nrhs, batch, L, ldl, sL, X, ldx, sX, adjB, ldab, saB, adjL, ldal, saL,
                                       accumulate, st);
    return launch_potrs_adj<64, T>(n, nrhs, batch, L, ldl, sL, X, ldx, sX, adjB, ldab, saB, adjL, ldal, saL,
                                   accumulate, st);
}

// lower triangle (diagonal included) of `batch` n x n matrices set to zero
template <typename T>
__global__ void __launch_bounds__(256) k_zero_lower(int64_t n, int64_t batch, T *p, int64_t ld, int64_t stride)
{
    const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (idx >= batch * n * n)
        return;
    const int64_t b = idx / (n * n), r = (idx / n) % n, c = idx % n;
    if (c <= r)
        p[b * stride + r * ld + c] = T(0);
}

chol_status zero_lower_batched(size_t es, int64_t n, int64_t batch, void *p, int64_t ld, int64_t stride, hipStream_t st)
{
    const int64_t tot = batch * n * n;
    if (tot <= 0)
        return CHOL_OK;
    const unsigned blocks = (unsigned)((tot + 255) / 256);
    if (es == 8)
        hipLaunchKernelGGL((k_zero_lower<double>), dim3(blocks), dim3(256), 0, st, n, batch, (double *)p, ld, stride);
    else
        hipLaunchKernelGGL((k_zero_lower<float>), dim3(blocks), dim3(256), 0, st, n, batch, (float *)p, ld, stride);
    CHOL_LAUNCH_CHECK();
    return CHOL_OK;
}

#define CHOL_INST(T)                                                                                          \
    template chol_status small_potrs<T>(int, int, int64_t, const T *, int64_t, int64_t, const T *, int64_t,   \
                                        int64_t, T *, int64_t, int64_t, hipStream_t);                         \
    template chol_status small_potrs_adjoint<T>(int, int, int64_t, const T *, int64_t, int64_t, const T *,    \
                                                int64_t, int64_t, const T *, int64_t, int64_t, T *, int64_t,  \
                                                int64_t, T *, int64_t, int64_t, int, hipStream_t);
CHOL_INST(float)
CHOL_INST(double)
#undef CHOL_INST

} // namespace chol
