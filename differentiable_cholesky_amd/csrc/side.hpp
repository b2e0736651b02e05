// Streams on which the blocked factor and adjoint run, so that the large
// trailing products (wide stream `x`) overlap the one-block kernels of the
// next tile column (stream `chain`).  Both are created on first use per
// device and kept for the life of the process, at default priority and
// non-blocking with respect to the null stream; work is ordered against the
// caller's stream and between the two streams by events only.  The large
// products on the wide stream run as persistent grids of two blocks per CU on
// all but RESERVED_CUS compute units' worth of block slots, which stay free
// for the chain's one-block kernels.  A small device buffer of zeroed work
// counters is allocated with them (once per device).
#pragma once

#include <hip/hip_runtime.h>

#include <mutex>

namespace chol {

constexpr int RESERVED_CUS = 16;

struct Side {
    hipStream_t chain = nullptr;   // one-block kernels
    hipStream_t x = nullptr;       // kernels that span the matrix
    hipEvent_t ev[6] = {};
    int *sched = nullptr;          // device counters of dynamically scheduled products
                                   // (SCHED_SLOTS slots of 2 ints, 64 bytes apart)
    void *fwd_inv = nullptr;       // two CHOL_MAX_NB-edge fp64 tiles: inverses of the factor's
                                   // diagonal tiles, alternating between tile columns
    int wide_cus = 0;              // CUs' worth of block slots the persistent grids use
    std::mutex mu;                 // one blocked call enqueues on these resources at a time
    bool ok = false;
};
constexpr int SCHED_SLOTS = 4;
constexpr int SCHED_STRIDE = 16;   // ints between slots

// Resources of the current device, or nullptr if they could not be created.
Side *side_resources();

// Enqueue-side helpers: make `waiter` wait for everything enqueued so far on `src`.
hipError_t stream_join(hipStream_t waiter, hipStream_t src, hipEvent_t ev);

} // namespace chol
