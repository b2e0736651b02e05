// Shared device helpers for libchol's gfx950 kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <atomic>

#include "../../include/libchol.h"

namespace chol {

// ---------------------------------------------------------------- math ----
// Division and square root use HIP's IEEE routines for both precisions.
template <typename T> __device__ __forceinline__ T dsqrt(T x);
template <> __device__ __forceinline__ float dsqrt<float>(float x) { return __fsqrt_rn(x); }
template <> __device__ __forceinline__ double dsqrt<double>(double x) { return __dsqrt_rn(x); }

template <typename T> __device__ __forceinline__ T drcp(T x);
template <> __device__ __forceinline__ float drcp<float>(float x) { return __fdiv_rn(1.0f, x); }
template <> __device__ __forceinline__ double drcp<double>(double x) { return __drcp_rn(x); }

// ---------------------------------------------------------------- MFMA ----
// One 16x16x4 matrix-core step: acc(16x16) += a(16x4) * b(4x16).
// Operand layout of v_mfma_{f32,f64}_16x16x4 on a 64-lane wavefront (checked
// on gfx950 with one-hot inputs):
//   a: lane l holds A[l % 16][l / 16]      (row, k)
//   b: lane l holds B[l / 16][l % 16]      (k, col)
//   acc[v], f32: lane l holds C[4 * (l / 16) + v][l % 16]
//   acc[v], f64: lane l holds C[(l / 16) + 4 * v][l % 16]
typedef double d4_t __attribute__((ext_vector_type(4)));
typedef float f4_t __attribute__((ext_vector_type(4)));

template <typename T> struct Acc;
template <> struct Acc<double> {
    typedef d4_t type;
    static __device__ __forceinline__ int row(int lane, int v) { return lane / 16 + 4 * v; }
};
template <> struct Acc<float> {
    typedef f4_t type;
    static __device__ __forceinline__ int row(int lane, int v) { return 4 * (lane / 16) + v; }
};

__device__ __forceinline__ d4_t mfma16x16x4(double a, double b, d4_t c)
{
    return __builtin_amdgcn_mfma_f64_16x16x4f64(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f4_t mfma16x16x4(float a, float b, f4_t c)
{
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}
// acc += (NEG ? -a : a) b.  The f64 instruction carries negate modifiers for
// its operands (its last field; neg:[1,0,0] negates a), so the negation costs
// no vector instruction; in the f32 instruction that field selects a lane
// broadcast instead, so a is negated by hand there.
template <bool NEG>
__device__ __forceinline__ d4_t mfma16x16x4_s(double a, double b, d4_t c)
{
    return __builtin_amdgcn_mfma_f64_16x16x4f64(a, b, c, 0, 0, NEG ? 1 : 0);
}
template <bool NEG>
__device__ __forceinline__ f4_t mfma16x16x4_s(float a, float b, f4_t c)
{
    return __builtin_amdgcn_mfma_f32_16x16x4f32(NEG ? -a : a, b, c, 0, 0, 0);
}

// ------------------------------------------------------ launch checking ----
// The HIP error behind the most recent CHOL_ERR_HIP (process-wide, for
// diagnostics: chol_last_hip_error()).
inline std::atomic<int> g_last_hip_error{0};

// Records e if it is an error; true if it is.
inline bool hip_failed(hipError_t e)
{
    if (e == hipSuccess)
        return false;
    g_last_hip_error.store((int)e, std::memory_order_relaxed);
    return true;
}

#define CHOL_LAUNCH_CHECK()                                  \
    do {                                                     \
        if (chol::hip_failed(hipGetLastError()))             \
            return CHOL_ERR_HIP;                             \
    } while (0)

} // namespace chol
