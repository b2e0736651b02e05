// Plain streaming kernels: the HBM ceiling that the bandwidth-bound kernels
// (the batched small tiles) are measured against.  Each block walks the
// buffer in 16-byte elements with a grid-stride loop, four loads or stores
// in flight per thread per iteration.
#include "common.hpp"

namespace chol {

namespace {

__global__ void __launch_bounds__(256) k_stream_read(const float4 *src, int64_t n, float *sink)
{
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    for (; i + 3 * stride < n; i += 4 * stride) {
        const float4 a = src[i], b = src[i + stride], c = src[i + 2 * stride], d = src[i + 3 * stride];
        acc.x += a.x + b.x + c.x + d.x;
        acc.y += a.y + b.y + c.y + d.y;
        acc.z += a.z + b.z + c.z + d.z;
        acc.w += a.w + b.w + c.w + d.w;
    }
    for (; i < n; i += stride) {
        const float4 a = src[i];
        acc.x += a.x; acc.y += a.y; acc.z += a.z; acc.w += a.w;
    }
    // one value per thread goes out (keeps every load); the buffer holds
    // gridDim.x * blockDim.x floats
    sink[(int64_t)blockIdx.x * blockDim.x + threadIdx.x] = acc.x + acc.y + acc.z + acc.w;
}

__global__ void __launch_bounds__(256) k_stream_write(float4 *dst, int64_t n, float value)
{
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    const float4 v = make_float4(value, value, value, value);
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride)
        dst[i] = v;
}

__global__ void __launch_bounds__(256) k_stream_copy(const float4 *src, float4 *dst, int64_t n)
{
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    for (; i + 3 * stride < n; i += 4 * stride) {
        const float4 a = src[i], b = src[i + stride], c = src[i + 2 * stride], d = src[i + 3 * stride];
        dst[i] = a;
        dst[i + stride] = b;
        dst[i + 2 * stride] = c;
        dst[i + 3 * stride] = d;
    }
    for (; i < n; i += stride)
        dst[i] = src[i];
}

} // namespace

// blocks of the streaming grid (8 per CU of a 256-CU device); the read
// kernel's sink holds one float per thread
constexpr int STREAM_BLOCKS = CHOL_HBM_READ_SINK_FLOATS / 256;

chol_status hbm_stream(int mode, const void *src, void *dst, size_t bytes, hipStream_t st)
{
    const int64_t n = (int64_t)(bytes / 16);
    if (mode == 0)
        hipLaunchKernelGGL(k_stream_read, dim3(STREAM_BLOCKS), dim3(256), 0, st, (const float4 *)src, n,
                           (float *)dst);
    else if (mode == 1)
        hipLaunchKernelGGL(k_stream_write, dim3(STREAM_BLOCKS), dim3(256), 0, st, (float4 *)dst, n, 1.0f);
    else
        hipLaunchKernelGGL(k_stream_copy, dim3(STREAM_BLOCKS), dim3(256), 0, st, (const float4 *)src,
                           (float4 *)dst, n);
    CHOL_LAUNCH_CHECK();
    return CHOL_OK;
}

} // namespace chol
