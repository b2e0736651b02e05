// Hermitian complex factor A = L L^H and its adjoint through the real
// embedding.  Each complex entry z = x + iy becomes the 2 x 2 real block
// [[x, -y], [y, x]]; a Hermitian A becomes a symmetric 2n x 2n matrix M, and
// a lower factor L with real positive diagonal becomes E(L), which is lower
// triangular with positive diagonal (its diagonal blocks are [[l, 0], [0, l]])
// and satisfies E(L) E(L)^T = E(L L^H) = M.  The real factor being unique,
// the real Cholesky factor of M is E(L): the complex factor is read back from
// the first column of each 2 x 2 block.  The adjoint runs the real adjoint on
// (E(L), adj_E), where adj_E holds dloss/dRe L_ij and dloss/dIm L_ij at the
// two entries the read-back takes L_ij from, and folds the real gradient of
// M's lower entries back onto the complex entries: Re A_ij sits at (2i, 2j)
// and (2i+1, 2j+1), Im A_ij at (2i+1, 2j) and, negated, at (2i, 2j+1).
// The embedding costs twice the real flops of a native complex factor; it
// keeps every step on the real kernels (register tiles for 2n <= 64, the
// blocked matrix-core path above).
//
// Complex arrays are interleaved (re, im) pairs of the real type T, row-major,
// leading dimensions and batch strides counted in complex elements.
#include <hip/hip_runtime.h>

#include "common.hpp"
#include "profile.hpp"

namespace chol {
namespace {

// MODE 0: M (2n x 2n, lower blocks) = E(A) from A's lower triangle (the
//         diagonal's imaginary part is not read);
// MODE 1: adj_E from adj_L: (2i, 2j) = Re, (2i+1, 2j) = Im (0 on the
//         diagonal), the block's second column 0.
template <typename T, int MODE>
__global__ void __launch_bounds__(256)
k_embed(int64_t n, int64_t batch, const T *A, int64_t lda, int64_t sA, T *M, int64_t ldm, int64_t sM)
{
    const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (idx >= batch * n * n)
        return;
    const int64_t b = idx / (n * n), i = (idx / n) % n, j = idx % n;
    if (j > i)
        return;
    const T *a = A + 2 * (b * sA + i * lda + j);
    const T x = a[0], y = (i == j) ? T(0) : a[1];
    T *m0 = M + b * sM + (2 * i) * ldm + 2 * j;
    T *m1 = m0 + ldm;
    if (MODE == 0) {
        m0[0] = x;
        m1[0] = y;
        m1[1] = x;
        if (i != j)
            m0[1] = -y;
    } else {
        m0[0] = x;
        m1[0] = y;
        m1[1] = T(0);
        if (i != j)
            m0[1] = T(0);
    }
}

// L (complex, n x n) from the real factor E: L_ij = E(2i, 2j) + i E(2i+1, 2j)
// below the diagonal, L_ii = E(2i, 2i), zeros above
template <typename T>
__global__ void __launch_bounds__(256)
k_read_back(int64_t n, int64_t batch, const T *E, int64_t lde, int64_t sE, T *L, int64_t ldl, int64_t sL)
{
    const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (idx >= batch * n * n)
        return;
    const int64_t b = idx / (n * n), i = (idx / n) % n, j = idx % n;
    T *l = L + 2 * (b * sL + i * ldl + j);
    if (j > i) {
        l[0] = T(0);
        l[1] = T(0);
        return;
    }
    const T *e = E + b * sE + (2 * i) * lde + 2 * j;
    l[0] = e[0];
    l[1] = (i == j) ? T(0) : e[lde];
}

// lower(adj_A) (+)= G folded from the real gradient GM of M's lower entries
template <typename T>
__global__ void __launch_bounds__(256)
k_fold(int64_t n, int64_t batch, const T *GM, int64_t ldg, int64_t sG, T *adjA, int64_t lda, int64_t sA,
       int accumulate)
{
    const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (idx >= batch * n * n)
        return;
    const int64_t b = idx / (n * n), i = (idx / n) % n, j = idx % n;
    if (j > i)
        return;
    const T *g0 = GM + b * sG + (2 * i) * ldg + 2 * j;
    const T *g1 = g0 + ldg;
    const T re = g0[0] + g1[1];
    const T im = (i == j) ? T(0) : g1[0] - g0[1];
    T *a = adjA + 2 * (b * sA + i * lda + j);
    if (accumulate) {
        a[0] += re;
        a[1] += im;
    } else {
        a[0] = re;
        a[1] = im;
    }
}

// a failing real column 2c or 2c+1 (info 2c+1 or 2c+2) is complex column c
__global__ void k_info_to_complex(int64_t batch, int32_t *info)
{
    const int64_t b = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (b < batch && info[b] > 0)
        info[b] = (info[b] + 1) / 2;
}

template <typename K, typename... Args>
chol_status launch_elem(K kernel, int64_t n, int64_t batch, hipStream_t st, Args... args)
{
    const int64_t tot = batch * n * n;
    if (tot <= 0)
        return CHOL_OK;
    hipLaunchKernelGGL(kernel, dim3((unsigned)((tot + 255) / 256)), dim3(256), 0, st, n, batch, args...);
    CHOL_LAUNCH_CHECK();
    return CHOL_OK;
}

} // namespace

template <typename T>
chol_status herm_embed(int64_t n, int64_t batch, const T *A, int64_t lda, int64_t sA, T *M, int64_t ldm, int64_t sM,
                       hipStream_t st)
{
    prof::Scope ps(CHOL_K_ELEMENTWISE, st, (double)batch * n * (n + 1) * 3 * sizeof(T));
    return launch_elem(k_embed<T, 0>, n, batch, st, A, lda, sA, M, ldm, sM);
}

template <typename T>
chol_status herm_embed_adjoint(int64_t n, int64_t batch, const T *adjL, int64_t ldal, int64_t sAL, T *M,
                               int64_t ldm, int64_t sM, hipStream_t st)
{
    prof::Scope ps(CHOL_K_ELEMENTWISE, st, (double)batch * n * (n + 1) * 3 * sizeof(T));
    return launch_elem(k_embed<T, 1>, n, batch, st, adjL, ldal, sAL, M, ldm, sM);
}

template <typename T>
chol_status herm_read_back(int64_t n, int64_t batch, const T *E, int64_t lde, int64_t sE, T *L, int64_t ldl,
                           int64_t sL, hipStream_t st)
{
    prof::Scope ps(CHOL_K_ELEMENTWISE, st, (double)batch * n * n * 3 * sizeof(T));
    return launch_elem(k_read_back<T>, n, batch, st, E, lde, sE, L, ldl, sL);
}

template <typename T>
chol_status herm_fold(int64_t n, int64_t batch, const T *GM, int64_t ldg, int64_t sG, T *adjA, int64_t lda,
                      int64_t sA, int accumulate, hipStream_t st)
{
    prof::Scope ps(CHOL_K_ELEMENTWISE, st, (double)batch * n * (n + 1) * (accumulate ? 4 : 3) * sizeof(T));
    return launch_elem(k_fold<T>, n, batch, st, GM, ldg, sG, adjA, lda, sA, accumulate);
}

chol_status herm_info(int64_t batch, int32_t *info, hipStream_t st)
{
    if (!info || batch <= 0)
        return CHOL_OK;
    hipLaunchKernelGGL(k_info_to_complex, dim3((unsigned)((batch + 255) / 256)), dim3(256), 0, st, batch, info);
    CHOL_LAUNCH_CHECK();
    return CHOL_OK;
}

#define CHOL_INST(T)                                                                                          \
    template chol_status herm_embed<T>(int64_t, int64_t, const T *, int64_t, int64_t, T *, int64_t, int64_t, \
                                       hipStream_t);                                                          \
    template chol_status herm_embed_adjoint<T>(int64_t, int64_t, const T *, int64_t, int64_t, T *, int64_t,   \
                                               int64_t, hipStream_t);                                         \
    template chol_status herm_read_back<T>(int64_t, int64_t, const T *, int64_t, int64_t, T *, int64_t,       \
                                           int64_t, hipStream_t);                                             \
    template chol_status herm_fold<T>(int64_t, int64_t, const T *, int64_t, int64_t, T *, int64_t, int64_t,   \
                                      int, hipStream_t);
CHOL_INST(float)
CHOL_INST(double)
#undef CHOL_INST

} // namespace chol
