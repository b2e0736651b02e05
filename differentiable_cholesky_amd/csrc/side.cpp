#include "side.hpp"

#include "common.hpp"


namespace chol {

namespace {
constexpr int MAX_DEVICES = 64;
Side g_side[MAX_DEVICES];
std::once_flag g_once[MAX_DEVICES];
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
    std::call_once(g_once[dev], [&s, dev]() {
        if (hip_failed(hipStreamCreateWithFlags(&s.chain, hipStreamNonBlocking)))
            return;
        int cus = 0;
        if (hip_failed(hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev)))
            return;
        if (cus <= 0) {
            hip_failed(hipErrorInvalidDevice);
            return;
        }
        if (hip_failed(hipStreamCreateWithFlags(&s.x, hipStreamNonBlocking)))
            return;
        // persistent grids of the wide stream leave RESERVED_CUS CUs' worth of
        // block slots free (restricting the stream with a CU mask instead was
        // measured slower: its launches cost more)
        s.wide_cus = cus > 4 * RESERVED_CUS ? cus - RESERVED_CUS : cus;
        for (auto &e : s.ev)
            if (hip_failed(hipEventCreateWithFlags(&e, hipEventDisableTiming)))
                return;
        const size_t bytes = sizeof(int) * SCHED_SLOTS * SCHED_STRIDE;
        if (hip_failed(hipMalloc((void **)&s.sched, bytes)))
            return;
        if (hip_failed(hipMalloc(&s.fwd_inv, 2 * CHOL_MAX_NB * CHOL_MAX_NB * sizeof(double))))
            return;
        if (hip_failed(hipMemset(s.sched, 0, bytes)) || hip_failed(hipDeviceSynchronize()))
            return;
        s.ok = true;
    });
    return s.ok ? &s : nullptr;
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

} // namespace chol
