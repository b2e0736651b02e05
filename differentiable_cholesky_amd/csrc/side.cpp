#include "side.hpp"


namespace chol {

namespace {
constexpr int MAX_DEVICES = 64;
Side g_side[MAX_DEVICES];
std::once_flag g_once[MAX_DEVICES];
} // namespace

Side *side_resources()
{
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= MAX_DEVICES)
        return nullptr;
    Side &s = g_side[dev];
    std::call_once(g_once[dev], [&s, dev]() {
        if (hipStreamCreateWithFlags(&s.chain, hipStreamNonBlocking) != hipSuccess)
            return;
        int cus = 0;
        if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
            return;
        if (hipStreamCreateWithFlags(&s.x, hipStreamNonBlocking) != hipSuccess)
            return;
        // persistent grids of the wide stream leave RESERVED_CUS CUs' worth of
        // block slots free (restricting the stream with a CU mask instead was
        // measured slower: its launches cost more)
        s.wide_cus = cus > 4 * RESERVED_CUS ? cus - RESERVED_CUS : cus;
        for (auto &e : s.ev)
            if (hipEventCreateWithFlags(&e, hipEventDisableTiming) != hipSuccess)
                return;
        const size_t bytes = sizeof(int) * SCHED_SLOTS * SCHED_STRIDE;
        if (hipMalloc((void **)&s.sched, bytes) != hipSuccess)
            return;
        if (hipMemset(s.sched, 0, bytes) != hipSuccess || hipDeviceSynchronize() != hipSuccess)
            return;
        s.ok = true;
    });
    return s.ok ? &s : nullptr;
}

hipError_t stream_join(hipStream_t waiter, hipStream_t src, hipEvent_t ev)
{
    hipError_t e = hipEventRecord(ev, src);
    if (e != hipSuccess)
        return e;
    return hipStreamWaitEvent(waiter, ev, 0);
}

} // namespace chol
