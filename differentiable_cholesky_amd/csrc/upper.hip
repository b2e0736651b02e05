// Upper-factor form (uplo = U): A = U^T U with U upper triangular, the
// row-major layout of a column-major caller's lower factor.  U = L^T for the
// lower factor L of the same symmetric matrix, so the upper entry points run
// the lower-form kernels on transposed copies: the upper triangle of A is
// brought into the lower triangle of the output transposed, factored there
// in place, and transposed back into the upper triangle (zeros below); the
// adjoint transposes U and adj_U into a workspace, runs the lower-form
// adjoint there and adds (or writes) the result transposed into adj_A's
// upper triangle.
//
// The transpositions go through 32 x 32 tiles in LDS (rows of 32 elements
// read and written whole), one workgroup per tile pair (I, J), J <= I, of
// each matrix of the batch; a pair's two tiles are only ever touched by its
// own workgroup, which makes the in-place forms race-free.
#include <hip/hip_runtime.h>

#include "common.hpp"
#include "profile.hpp"

namespace chol {
namespace {

constexpr int TT = 32;

__device__ __forceinline__ void pair_of(int64_t t, int64_t &I, int64_t &J)
{
    int64_t r = (int64_t)((sqrt(8.0 * (double)t + 1.0) - 1.0) * 0.5);
    while (r * (r + 1) / 2 > t)
        --r;
    while ((r + 1) * (r + 2) / 2 <= t)
        ++r;
    I = r;
    J = t - r * (r + 1) / 2;
}

// MODE 0: lower(dst) = upper(src)^T            (dst may be src)
// MODE 1: upper(p) = lower(p)^T, strict lower(p) = 0   (in place, src unused)
// MODE 2: upper(dst) (+)= lower(src)^T          (accumulate: add)
template <typename T, int MODE>
__global__ void __launch_bounds__(256)
k_transpose_tri(int64_t n, int64_t pairs, const T *src, int64_t lds, int64_t ss, T *dst, int64_t ldd, int64_t sd,
                int accumulate)
{
    __shared__ T tile[TT][TT + 1];
    const int64_t b = (int64_t)blockIdx.x / pairs;
    int64_t I, J;
    pair_of((int64_t)blockIdx.x % pairs, I, J);
    const int tx = threadIdx.x % TT, ty = threadIdx.x / TT;   // 32 x 8 threads
    const int64_t r0 = I * TT, c0 = J * TT;                  // the lower tile (I, J)
    if (MODE == 0) {
        // read the upper tile (J, I) of src: element (c0 + y, r0 + x)
        const T *s = src + b * ss;
        for (int y = ty; y < TT; y += 8) {
            const int64_t row = c0 + y, col = r0 + tx;
            tile[y][tx] = (row < n && col < n && col >= row) ? s[row * lds + col] : T(0);
        }
        __syncthreads();
        T *d = dst + b * sd;
        for (int y = ty; y < TT; y += 8) {
            const int64_t row = r0 + y, col = c0 + tx;         // lower element (row, col) = src (col, row)
            if (row < n && col < n && col <= row)
                d[row * ldd + col] = tile[tx][y];
        }
    } else if (MODE == 1) {
        T *p = dst + b * sd;
        for (int y = ty; y < TT; y += 8) {
            const int64_t row = r0 + y, col = c0 + tx;
            tile[y][tx] = (row < n && col < n && col <= row) ? p[row * ldd + col] : T(0);
        }
        __syncthreads();
        for (int y = ty; y < TT; y += 8) {
            // upper element (c0 + y, r0 + x) = lower (r0 + x, c0 + y)
            const int64_t row = c0 + y, col = r0 + tx;
            if (row < n && col < n && col >= row)
                p[row * ldd + col] = tile[tx][y];
        }
        __syncthreads();   // the diagonal tile's reads and writes cover the same rows
        for (int y = ty; y < TT; y += 8) {
            const int64_t row = r0 + y, col = c0 + tx;
            if (row < n && col < n && col < row)
                p[row * ldd + col] = T(0);
        }
    } else {
        const T *s = src + b * ss;
        for (int y = ty; y < TT; y += 8) {
            const int64_t row = r0 + y, col = c0 + tx;
            tile[y][tx] = (row < n && col < n && col <= row) ? s[row * lds + col] : T(0);
        }
        __syncthreads();
        T *d = dst + b * sd;
        for (int y = ty; y < TT; y += 8) {
            const int64_t row = c0 + y, col = r0 + tx;
            if (row < n && col < n && col >= row) {
                const T g = tile[tx][y];
                d[row * ldd + col] = accumulate ? d[row * ldd + col] + g : g;
            }
        }
    }
}

template <typename T, int MODE>
chol_status launch_transpose(int64_t n, int64_t batch, const T *src, int64_t lds, int64_t ss, T *dst, int64_t ldd,
                             int64_t sd, int accumulate, hipStream_t st)
{
    if (n <= 0 || batch <= 0)
        return CHOL_OK;
    const int64_t tiles = (n + TT - 1) / TT, pairs = tiles * (tiles + 1) / 2;
    const int64_t blocks = pairs * batch;
    if (blocks > 0x7fffffff)
        return CHOL_ERR_NOT_SUPPORTED;
    const double tri = (double)n * (n + 1) / 2 * batch * sizeof(T);
    prof::Scope ps(CHOL_K_ELEMENTWISE, st, MODE == 1 ? 3 * tri : (MODE == 2 && accumulate ? 3 * tri : 2 * tri));
    hipLaunchKernelGGL((k_transpose_tri<T, MODE>), dim3((unsigned)blocks), dim3(256), 0, st, n, pairs, src, lds, ss,
                       dst, ldd, sd, accumulate);
    CHOL_LAUNCH_CHECK();
    return CHOL_OK;
}

} // namespace

template <typename T>
chol_status upper_to_lower(int64_t n, int64_t batch, const T *src, int64_t lds, int64_t ss, T *dst, int64_t ldd,
                           int64_t sd, hipStream_t st)
{
    return launch_transpose<T, 0>(n, batch, src, lds, ss, dst, ldd, sd, 0, st);
}

template <typename T>
chol_status lower_to_upper(int64_t n, int64_t batch, T *p, int64_t ld, int64_t stride, hipStream_t st)
{
    return launch_transpose<T, 1>(n, batch, nullptr, 0, 0, p, ld, stride, 0, st);
}

template <typename T>
chol_status add_upper_from_lower(int64_t n, int64_t batch, const T *G, int64_t ldg, int64_t sg, T *A, int64_t lda,
                                 int64_t sa, int accumulate, hipStream_t st)
{
    return launch_transpose<T, 2>(n, batch, G, ldg, sg, A, lda, sa, accumulate, st);
}

#define CHOL_INST(T)                                                                                          \
    template chol_status upper_to_lower<T>(int64_t, int64_t, const T *, int64_t, int64_t, T *, int64_t,       \
                                           int64_t, hipStream_t);                                             \
    template chol_status lower_to_upper<T>(int64_t, int64_t, T *, int64_t, int64_t, hipStream_t);             \
    template chol_status add_upper_from_lower<T>(int64_t, int64_t, const T *, int64_t, int64_t, T *, int64_t, \
                                                 int64_t, int, hipStream_t);
CHOL_INST(float)
CHOL_INST(double)
#undef CHOL_INST

} // namespace chol
