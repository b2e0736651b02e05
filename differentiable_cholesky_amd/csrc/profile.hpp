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

} // namespace prof
} // namespace chol
