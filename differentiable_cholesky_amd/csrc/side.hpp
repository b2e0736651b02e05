// Per-device resources of the blocked calls.
//
// Streams: the large trailing products (wide stream `x`) overlap the
// one-block kernels of the next tile column (stream `chain`).  Both streams
// are created on first use per device (or by chol_init) and kept for the life
// of the process, at default priority and non-blocking with respect to the
// null stream; work is ordered against the caller's stream and between the
// two streams by events only.  The large products on the wide stream run as
// persistent grids of two blocks per CU on all but RESERVED_CUS compute
// units' worth of block slots, which stay free for the chain's one-block
// kernels.
//
// Device memory: the work counters of the persistent grids and the forward's
// two diagonal-tile inverse slots are file-scope device arrays of the
// library's code object, so the calls allocate nothing; their per-device
// addresses are resolved once.
// Blocked calls on one device are serialised through these streams and
// buffers (the mutex covers enqueueing; stream order covers execution).
#pragma once

#include <hip/hip_runtime.h>

#include <mutex>

#include "../../include/libchol.h"

namespace chol {

constexpr int RESERVED_CUS = 16;
constexpr int SCHED_SLOTS = 4;
constexpr int SCHED_STRIDE = 16;   // ints between slots (64 bytes)
constexpr int SCHED_INTS = SCHED_SLOTS * SCHED_STRIDE;

struct Side {
    hipStream_t chain = nullptr;   // one-block kernels
    hipStream_t x = nullptr;       // kernels that span the matrix
    hipEvent_t ev[6] = {};
    int *sched = nullptr;          // device counters of dynamically scheduled products
                                   // (SCHED_SLOTS slots of 2 ints, SCHED_STRIDE ints apart);
                                   // zeroed in stream order at the entry of every blocked call
    void *fwd_inv = nullptr;       // two CHOL_MAX_NB-edge fp64 tiles: inverses of the factor's
                                   // diagonal tiles, alternating between tile columns
    int wide_cus = 0;              // CUs' worth of block slots the persistent grids use
    std::mutex mu;                 // one blocked call enqueues on these resources at a time
    bool ok = false;
};

// Resources of the current device, created on first use; nullptr (and the
// HIP error recorded) if they could not be created -- a later call retries.
Side *side_resources();

// Split cap of the symmetric product in the allocation-free adjoint, whose
// workspace lives in the library's static `scratch` array.
constexpr int NOALLOC_SPLIT_MAX = 4;

// The allocation-free adjoint's device storage on the current device: the
// address of the static `scratch` array (CHOL_NOALLOC_SCRATCH_BYTES) and of
// its own work-counter slot, and the device's CU count.  Resolved once per
// device (symbol lookups only: nothing is allocated or created); false (and
// the HIP error recorded) on failure.
struct NoAlloc {
    void *scratch;
    int *sched;
    int cus;
};
bool noalloc_resources(NoAlloc &out);

// Enqueue-side helpers: make `waiter` wait for everything enqueued so far on `src`.
hipError_t stream_join(hipStream_t waiter, hipStream_t src, hipEvent_t ev);

// Zero `count` ints at p in stream order (a fill kernel, so that it is an
// ordinary kernel node under stream capture).
hipError_t zero_ints(int *p, int count, hipStream_t st);

} // namespace chol
