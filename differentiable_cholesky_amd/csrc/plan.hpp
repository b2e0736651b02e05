// Host-side schedule of the blocked factorisation: the operations the forward
// sweep enqueues, in order, each on one of the two library streams, with the
// joins between the streams made explicit.  The executor in blocked.hip
// launches exactly this list; chol_potrf_plan exposes it so that the schedule
// can be checked on the host (panel bookkeeping, ordering of every pair of
// operations that touch the same data).
#pragma once

#include <stdint.h>

#include <vector>

namespace chol {

enum FwdKind {
    FWD_COPY = 0,        // chain: lower part of columns 0 .. w-1 of A into L
    FWD_DIAG = 1,        // chain (or wide, with nothing beside it): factor tile column k's diagonal
                         // tile; slot >= 0: its inverse into slot
    FWD_PANEL = 2,       // wide: panel solve of tile column k (rows below its tile), reading slot
    FWD_UPDATE = 3,      // wide: lower part of W[c:, c:c+w] -= Q[c:] Q[c:c+w]^T, Q = panels f .. f+np-1
    FWD_TRI = 4,         // wide: lower tiles t0 .. t0+tn-1 (128 x 128, row-major) of W[c:, c:] -= Q Q^T
                         // (slot 1: W read from A, the tiles' first update)
    FWD_JOIN = 5,        // `stream` waits for everything enqueued so far on the other stream (event ev)
    FWD_ZERO_UPPER = 6   // chain: strict upper triangle of L set to zero
};
enum FwdStream { FWD_CHAIN = 0, FWD_WIDE = 1 };

struct FwdOp {
    int32_t kind, stream;
    int64_t k;           // FWD_DIAG, FWD_PANEL: tile column
    int64_t c, w, f;     // FWD_UPDATE, FWD_TRI (w unused for FWD_TRI)
    int32_t np, t0, tn;  // panels; FWD_TRI tile window
    int32_t slot;        // FWD_DIAG: inverse slot written (-1: none); FWD_PANEL: slot read;
                         // FWD_JOIN: event index; FWD_TRI: 1 if the tiles are read from A
};

// depth of the deferred trailing update: the far triangle is updated with
// DEFER panels at once (at n = 16384 the factor took 42.7, 41.9, 41.4, 43.9
// and 45.9 ms with depths 2, 3, 4, 6 and 8: deeper groups add narrow
// 128-deep updates of the columns inside the group)
constexpr int FWD_DEFER = 4;

// The operations for an n x n factor with tile size nb (copy: A is not L);
// slots: block slots of the persistent grid that runs the FWD_TRI updates
// (0: the far triangle is cut into equal parts).
std::vector<FwdOp> forward_plan(int64_t n, int nb, bool copy, int slots);

} // namespace chol
