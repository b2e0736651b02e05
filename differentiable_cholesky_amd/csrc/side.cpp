#include "side.hpp"

#include "common.hpp"

namespace chol {

// Device storage of the blocked calls (one copy per device, allocated with the
// library's code object when it is loaded on that device).
__device__ __align__(256) int g_sched_counters[SCHED_INTS];
__device__ __align__(256) double g_fwd_inverse_slots[2 * CHOL_MAX_NB * CHOL_MAX_NB];

namespace {
constexpr int MAX_DEVICES = 64;
Side g_side[MAX_DEVICES];
std::mutex g_init_mu[MAX_DEVICES];

__global__ void k_zero_ints(int *p, int count)
{
    for (int i = threadIdx.x + blockIdx.x * blockDim.x; i < count; i += blockDim.x * gridDim.x)
        p[i] = 0;
}

void release(Side &s)
{
    for (auto &e : s.ev)
        if (e) {
            (void)hipEventDestroy(e);
            e = nullptr;
        }
    if (s.x) {
        (void)hipStreamDestroy(s.x);
        s.x = nullptr;
    }
    if (s.chain) {
        (void)hipStreamDestroy(s.chain);
        s.chain = nullptr;
    }
    s.sched = nullptr;
    s.fwd_inv = nullptr;
}

bool create(Side &s, int dev)
{
    int cus = 0;
    if (hip_failed(hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev)))
        return false;
    if (cus <= 0) {
        hip_failed(hipErrorInvalidDevice);
        return false;
    }
    // persistent grids of the wide stream leave RESERVED_CUS CUs' worth of
    // block slots free (restricting the stream with a CU mask instead was
    // measured slower: its launches cost more)
    s.wide_cus = cus > 4 * RESERVED_CUS ? cus - RESERVED_CUS : cus;
    if (hip_failed(hipGetSymbolAddress((void **)&s.sched, HIP_SYMBOL(g_sched_counters))) ||
        hip_failed(hipGetSymbolAddress(&s.fwd_inv, HIP_SYMBOL(g_fwd_inverse_slots))))
        return false;
    if (hip_failed(hipStreamCreateWithFlags(&s.chain, hipStreamNonBlocking)) ||
        hip_failed(hipStreamCreateWithFlags(&s.x, hipStreamNonBlocking)))
        return false;
    for (auto &e : s.ev)
        if (hip_failed(hipEventCreateWithFlags(&e, hipEventDisableTiming)))
            return false;
    return true;
}
} // namespace

Side *side_resources()
{
    int dev = 0;
    if (hip_failed(hipGetDevice(&dev)))
        return nullptr;
    if (dev < 0 || dev >= MAX_DEVICES) {
        hip_failed(hipErrorInvalidDevice);
        return nullptr;
    }
    Side &s = g_side[dev];
    std::lock_guard<std::mutex> lk(g_init_mu[dev]);
    if (!s.ok) {
        if (!create(s, dev)) {
            release(s);
            return nullptr;
        }
        s.ok = true;
    }
    return &s;
}

hipError_t stream_join(hipStream_t waiter, hipStream_t src, hipEvent_t ev)
{
    hipError_t e = hipEventRecord(ev, src);
    if (hip_failed(e))
        return e;
    e = hipStreamWaitEvent(waiter, ev, 0);
    hip_failed(e);
    return e;
}

hipError_t zero_ints(int *p, int count, hipStream_t st)
{
    hipLaunchKernelGGL(k_zero_ints, dim3(1), dim3(64), 0, st, p, count);
    const hipError_t e = hipGetLastError();
    hip_failed(e);
    return e;
}

} // namespace chol
