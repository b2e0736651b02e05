// Optional per-kernel-family timing with HIP events on the launching stream.
// Disabled by default; when disabled a scope costs one relaxed atomic load.
#pragma once

#include <hip/hip_runtime.h>

#include <atomic>

#include "../../include/libchol.h"

namespace chol {
namespace prof {

extern std::atomic<uint32_t> g_mask;   // families being timed, 0: timing off

struct Scope {
    int id;
    hipStream_t st;
    double work;
    hipEvent_t a = nullptr, b = nullptr;
    Scope(int id_, hipStream_t st_, double work_);
    ~Scope();
};

// The same timing for one kernel launch that carries the events itself
// (hipExtLaunchKernel): the pair, when the family is being timed, is handed to
// the launch, which stamps the kernel's own start and end into it, so that no
// marker enters the stream between this kernel and its neighbours.
struct LaunchEvents {
    int id;
    double work;
    hipEvent_t a = nullptr, b = nullptr;
    LaunchEvents(int id_, double work_);
    ~LaunchEvents();
};

} // namespace prof
} // namespace chol
