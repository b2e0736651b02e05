#include "side.hpp"

#include "common.hpp"

namespace chol {

// Device storage of the blocked calls (one copy per device, allocated with the
// library's code object when it is loaded on that device).
__device__ __align__(256) int g_sched_counters[SCHED_INTS];
__device__ __align__(256) double g_fwd_inverse_slots[2 * CHOL_MAX_NB * CHOL_MAX_NB];

// Workspace of the allocation-free adjoint (chol_potrf_adjoint_noalloc), one
// copy per device.  In host code its name is only a handle for the symbol
// lookup below; every use goes through the device address resolved there.
static __device__ __align__(256) unsigned char scratch[CHOL_NOALLOC_SCRATCH_BYTES];

namespace {
constexpr int MAX_DEVICES = 64;
Side g_side[MAX_DEVICES];
std::mutex g_init_mu[MAX_DEVICES];

struct NoAllocSlot {
    NoAlloc r{};
    bool ok = false;
};
NoAllocSlot g_noalloc[MAX_DEVICES];
std::mutex g_noalloc_mu[MAX_DEVICES];

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

bool noalloc_resources(NoAlloc &out)
{
    int dev = 0;
    if (hip_failed(hipGetDevice(&dev)))
        return false;
    if (dev < 0 || dev >= MAX_DEVICES) {
        hip_failed(hipErrorInvalidDevice);
        return false;
    }
    NoAllocSlot &s = g_noalloc[dev];
    std::lock_guard<std::mutex> lk(g_noalloc_mu[dev]);
    if (!s.ok) {
        NoAlloc r{};
        int *counters = nullptr;
        if (hip_failed(hipGetSymbolAddress(&r.scratch, HIP_SYMBOL(scratch))) ||
            hip_failed(hipGetSymbolAddress((void **)&counters, HIP_SYMBOL(g_sched_counters))) ||
            hip_failed(hipDeviceGetAttribute(&r.cus, hipDeviceAttributeMultiprocessorCount, dev)))
            return false;
        if (r.cus <= 0) {
            hip_failed(hipErrorInvalidDevice);
            return false;
        }
        r.sched = counters + SCHED_STRIDE;   // slot 1; slot 0 belongs to the calls on the library streams
        s.r = r;
        s.ok = true;
    }
    out = s.r;
    return true;
}

hipError_t stream_join(hipStream_t waiter, hipStream_t src, hipEvent_t ev)
{
    if (waiter == src)
        return hipSuccess;              // one stream: already in order
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
