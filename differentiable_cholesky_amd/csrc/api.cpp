// libchol C-ABI: argument validation and dispatch to the two kernel families.
// Every check here runs on the host before anything is launched; a failed
// check launches nothing.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdint>

#include "../../include/libchol.h"
#include "common.hpp"
#include "plan.hpp"
#include "profile.hpp"
#include "side.hpp"

namespace chol {
template <typename T>
chol_status small_potrf(int n, int64_t batch, const T *A, int64_t lda, int64_t sA, T *L, int64_t ldl,
                        int64_t sL, int32_t *info, int info_mode, int64_t info_base, hipStream_t st);
template <typename T>
chol_status small_potrf_adjoint(int n, int64_t batch, const T *L, int64_t ldl, int64_t sL,
                                const T *adjL, int64_t ldal, int64_t sAL, T *adjA, int64_t ldaa,
                                int64_t sAA, int accumulate, hipStream_t st);
template <typename T>
chol_status blocked_potrf(int64_t n, const T *A, int64_t lda, T *L, int64_t ldl, int32_t *info, int nb,
                          hipStream_t st);
template <typename T>
chol_status blocked_adjoint(int64_t n, const T *L, int64_t ldl, const T *adjL, int64_t ldal, T *adjA,
                            int64_t ldaa, int accumulate, int nb, void *ws, hipStream_t st);
size_t blocked_adjoint_workspace(int64_t n, int nb, size_t esize, bool need_wb);
size_t blocked_adjoint_workspace(int64_t n, int nb, size_t esize, bool need_wb, int max_splits);
template <typename T>
chol_status blocked_adjoint_single_stream(int64_t n, const T *L, int64_t ldl, const T *adjL, int64_t ldal, T *adjA,
                                          int64_t ldaa, int accumulate, int nb, void *ws, int *sched, int cus,
                                          hipStream_t st);
chol_status hbm_stream(int mode, const void *src, void *dst, size_t bytes, hipStream_t st);
template <typename T>
chol_status small_potrs(int n, int nrhs, int64_t batch, const T *L, int64_t ldl, int64_t sL, const T *B, int64_t ldb,
                        int64_t sB, T *X, int64_t ldx, int64_t sX, hipStream_t st);
template <typename T>
chol_status small_potrs_adjoint(int n, int nrhs, int64_t batch, const T *L, int64_t ldl, int64_t sL, const T *X,
                                int64_t ldx, int64_t sX, const T *adjX, int64_t ldax, int64_t saX, T *adjB,
                                int64_t ldab, int64_t saB, T *adjL, int64_t ldal, int64_t saL, int accumulate,
                                hipStream_t st);
template <typename T>
chol_status blocked_potrs(int64_t n, int64_t nrhs, const T *L, int64_t ldl, const T *B, int64_t ldb, T *X,
                          int64_t ldx, int nb, void *ws, hipStream_t st);
template <typename T>
chol_status blocked_potrs_adjoint(int64_t n, int64_t nrhs, const T *L, int64_t ldl, const T *X, int64_t ldx,
                                  const T *adjX, int64_t ldax, T *adjB, int64_t ldab, T *adjL, int64_t ldal,
                                  int accumulate, int nb, void *ws, hipStream_t st);
size_t blocked_solve_workspace(int64_t n, int64_t nrhs, int nb, size_t es);
chol_status zero_lower_batched(size_t es, int64_t n, int64_t batch, void *p, int64_t ld, int64_t stride, hipStream_t st);
template <typename T>
chol_status herm_embed(int64_t n, int64_t batch, const T *A, int64_t lda, int64_t sA, T *M, int64_t ldm, int64_t sM,
                       hipStream_t st);
template <typename T>
chol_status herm_embed_adjoint(int64_t n, int64_t batch, const T *adjL, int64_t ldal, int64_t sAL, T *M,
                               int64_t ldm, int64_t sM, hipStream_t st);
template <typename T>
chol_status herm_read_back(int64_t n, int64_t batch, const T *E, int64_t lde, int64_t sE, T *L, int64_t ldl,
                           int64_t sL, hipStream_t st);
template <typename T>
chol_status herm_fold(int64_t n, int64_t batch, const T *GM, int64_t ldg, int64_t sG, T *adjA, int64_t lda,
                      int64_t sA, int accumulate, hipStream_t st);
chol_status herm_info(int64_t batch, int32_t *info, hipStream_t st);
template <typename T>
chol_status upper_to_lower(int64_t n, int64_t batch, const T *src, int64_t lds, int64_t ss, T *dst, int64_t ldd,
                           int64_t sd, hipStream_t st);
template <typename T>
chol_status lower_to_upper(int64_t n, int64_t batch, T *p, int64_t ld, int64_t stride, hipStream_t st);
template <typename T>
chol_status add_upper_from_lower(int64_t n, int64_t batch, const T *G, int64_t ldg, int64_t sg, T *A, int64_t lda,
                                 int64_t sa, int accumulate, hipStream_t st);
size_t blocked_solve_adjoint_workspace(int64_t n, int64_t nrhs, int nb, size_t es);
chol_status small_load();
chol_status blocked_load();
template <typename T>
chol_status wave_dot(int n, const T *a, const T *b, T *y, const T *ybar, T *abar, T *bbar, int staging,
                     hipStream_t st);
template <typename T>
chol_status wave_sum(int n, const T *a, T *y, const T *ybar, T *abar, int staging, hipStream_t st);
} // namespace chol

namespace {

const int DEFAULT_NB = 128;
// Index arithmetic inside the kernels uses 32-bit row/column counts.
const int64_t MAX_N = (int64_t)1 << 30;

struct Extent {
    uintptr_t lo, hi; // [lo, hi) in bytes; empty when lo == hi
};

bool valid_dtype(chol_dtype dt) { return dt == CHOL_F32 || dt == CHOL_F64; }
size_t esize(chol_dtype dt) { return dt == CHOL_F64 ? 8 : 4; }

Extent extent(const void *p, int64_t n, int64_t ld, int64_t batch, int64_t stride, size_t es)
{
    Extent e{(uintptr_t)p, (uintptr_t)p};
    if (n > 0 && batch > 0)
        e.hi = e.lo + (size_t)((batch - 1) * stride + (n - 1) * ld + n) * es;
    return e;
}

bool overlap(const Extent &a, const Extent &b) { return a.lo < b.hi && b.lo < a.hi; }

// Output `o` may be exactly the same buffer as input `i` (same base, ld and
// stride) or disjoint from it; any other overlap is rejected.
bool alias_ok(const void *i, int64_t ldi, int64_t si, const void *o, int64_t ldo, int64_t so, int64_t n,
              int64_t batch, size_t es)
{
    if (i == o)
        return ldi == ldo && (batch <= 1 || si == so);
    return !overlap(extent(i, n, ldi, batch, si, es), extent(o, n, ldo, batch, so, es));
}

// rows x cols blocks (right-hand sides of the solve)
Extent rect_extent(const void *p, int64_t rows, int64_t cols, int64_t ld, int64_t batch, int64_t stride, size_t es)
{
    Extent e{(uintptr_t)p, (uintptr_t)p};
    if (rows > 0 && cols > 0 && batch > 0)
        e.hi = e.lo + (size_t)((batch - 1) * stride + (rows - 1) * ld + cols) * es;
    return e;
}

bool rect_alias_ok(const void *i, int64_t ldi, int64_t si, const void *o, int64_t ldo, int64_t so, int64_t rows,
                   int64_t cols, int64_t batch, size_t es)
{
    if (i == o)
        return ldi == ldo && (batch <= 1 || si == so);
    return !overlap(rect_extent(i, rows, cols, ldi, batch, si, es), rect_extent(o, rows, cols, ldo, batch, so, es));
}

bool ld_ok(int64_t ld, int64_t n) { return ld >= std::max<int64_t>(1, n); }
bool stride_ok(int64_t stride, int64_t ld, int64_t n, int64_t batch)
{
    return batch <= 1 || stride >= ld * n;
}
bool nb_ok(int64_t nb) { return nb >= 0 && nb <= CHOL_MAX_NB; }

} // namespace

// The library checks each launch with hipGetLastError(), whose status is
// sticky per host thread: a status left by unrelated HIP calls made earlier on
// this thread (for example an event query that found work still pending) would
// be taken for a failed launch.  Every entry point that launches clears it
// first.
static inline void clear_stale_status() { (void)hipGetLastError(); }

extern "C" {

int chol_abi_version(void) { return LIBCHOL_ABI_VERSION; }

chol_status chol_init(void)
{
    clear_stale_status();
    if (chol::small_load() != CHOL_OK || chol::blocked_load() != CHOL_OK)
        return CHOL_ERR_HIP;
    chol::NoAlloc na;
    if (!chol::noalloc_resources(na))
        return CHOL_ERR_HIP;
    return chol::side_resources() ? CHOL_OK : CHOL_ERR_HIP;
}

const char *chol_status_string(chol_status s)
{
    switch (s) {
    case CHOL_OK: return "CHOL_OK";
    case CHOL_ERR_INVALID_VALUE: return "CHOL_ERR_INVALID_VALUE: an argument is out of range or buffers overlap";
    case CHOL_ERR_NOT_SUPPORTED: return "CHOL_ERR_NOT_SUPPORTED: size outside what this entry point handles";
    case CHOL_ERR_WORKSPACE: return "CHOL_ERR_WORKSPACE: workspace missing or too small";
    case CHOL_ERR_HIP: return "CHOL_ERR_HIP: a HIP launch failed";
    }
    return "unknown chol_status";
}

int64_t chol_potrf_plan(int64_t n, int64_t nb, int copy, int64_t slots, int64_t *ops, int64_t cap)
{
    if (n < 0 || !nb_ok(nb) || slots < 0 || slots > INT32_MAX || cap < 0 || (cap > 0 && !ops))
        return -1;
    const std::vector<chol::FwdOp> plan =
        chol::forward_plan(n, nb ? (int)nb : DEFAULT_NB, copy != 0, (int)slots);
    const int64_t count = (int64_t)plan.size();
    for (int64_t i = 0; i < count && i < cap; ++i) {
        const chol::FwdOp &o = plan[(size_t)i];
        int64_t *r = ops + i * CHOL_PLAN_FIELDS;
        r[0] = o.kind; r[1] = o.stream; r[2] = o.k; r[3] = o.c; r[4] = o.w;
        r[5] = o.f; r[6] = o.np; r[7] = o.t0; r[8] = o.tn; r[9] = o.slot;
    }
    return count;
}

// ------------------------------------------------------------------ solve ----

namespace {
// shared checks of the solve entry points; returns CHOL_OK to go on, or the
// status to return (CHOL_OK with *noop for empty problems)
chol_status potrs_args(chol_dtype dt, int64_t n, int64_t nrhs, int64_t batch, const void *L, int64_t ldl,
                       int64_t sL, const void *B, int64_t ldb, int64_t sB, const void *X, int64_t ldx, int64_t sX,
                       bool *noop)
{
    *noop = false;
    if (!valid_dtype(dt) || n < 0 || nrhs < 0 || batch < 0)
        return CHOL_ERR_INVALID_VALUE;
    if (n == 0 || nrhs == 0 || batch == 0) {
        *noop = true;
        return CHOL_OK;
    }
    if (!L || !B || !X || !ld_ok(ldl, n) || !ld_ok(ldb, nrhs) || !ld_ok(ldx, nrhs) ||
        !stride_ok(sL, ldl, n, batch) || !stride_ok(sB, ldb, n, batch) || !stride_ok(sX, ldx, n, batch))
        return CHOL_ERR_INVALID_VALUE;
    if (n > MAX_N || nrhs > INT32_MAX || batch > ((int64_t)1 << 31) - 1)
        return CHOL_ERR_NOT_SUPPORTED;
    const size_t es = esize(dt);
    if (!rect_alias_ok(B, ldb, sB, X, ldx, sX, n, nrhs, batch, es) ||
        overlap(extent(L, n, ldl, batch, sL, es), rect_extent(X, n, nrhs, ldx, batch, sX, es)))
        return CHOL_ERR_INVALID_VALUE;
    return CHOL_OK;
}
} // namespace

chol_status chol_potrs_workspace_size(chol_dtype dt, int64_t n, int64_t nrhs, int64_t nb, size_t *bytes)
{
    if (!bytes || !valid_dtype(dt) || n < 0 || nrhs < 0 || !nb_ok(nb))
        return CHOL_ERR_INVALID_VALUE;
    *bytes = 0;
    if (n <= CHOL_SMALL_MAX_N || nrhs == 0)
        return CHOL_OK;
    if (n > MAX_N)
        return CHOL_ERR_NOT_SUPPORTED;
    *bytes = chol::blocked_solve_workspace(n, nrhs, nb ? (int)nb : DEFAULT_NB, esize(dt));
    return CHOL_OK;
}

chol_status chol_potrs(chol_dtype dt, int64_t n, int64_t nrhs, const void *L, int64_t ldl, const void *B,
                       int64_t ldb, void *X, int64_t ldx, int64_t nb, void *workspace, size_t workspace_bytes,
                       void *stream)
{
    if (!nb_ok(nb))
        return CHOL_ERR_INVALID_VALUE;
    bool noop;
    chol_status s = potrs_args(dt, n, nrhs, 1, L, ldl, 0, B, ldb, 0, X, ldx, 0, &noop);
    if (s != CHOL_OK || noop)
        return s;
    const size_t es = esize(dt);
    hipStream_t st = (hipStream_t)stream;
    clear_stale_status();
    if (n <= CHOL_SMALL_MAX_N) {
        if (dt == CHOL_F64)
            return chol::small_potrs<double>((int)n, (int)nrhs, 1, (const double *)L, ldl, 0, (const double *)B, ldb,
                                             0, (double *)X, ldx, 0, st);
        return chol::small_potrs<float>((int)n, (int)nrhs, 1, (const float *)L, ldl, 0, (const float *)B, ldb, 0,
                                        (float *)X, ldx, 0, st);
    }
    const int b = nb ? (int)nb : DEFAULT_NB;
    const size_t need = chol::blocked_solve_workspace(n, nrhs, b, es);
    if (!workspace || workspace_bytes < need)
        return CHOL_ERR_WORKSPACE;
    const Extent ws{(uintptr_t)workspace, (uintptr_t)workspace + need};
    if (overlap(ws, extent(L, n, ldl, 1, 0, es)) || overlap(ws, rect_extent(B, n, nrhs, ldb, 1, 0, es)) ||
        overlap(ws, rect_extent(X, n, nrhs, ldx, 1, 0, es)))
        return CHOL_ERR_INVALID_VALUE;
    if (dt == CHOL_F64)
        return chol::blocked_potrs<double>(n, nrhs, (const double *)L, ldl, (const double *)B, ldb, (double *)X, ldx,
                                           b, workspace, st);
    return chol::blocked_potrs<float>(n, nrhs, (const float *)L, ldl, (const float *)B, ldb, (float *)X, ldx, b,
                                      workspace, st);
}

chol_status chol_potrs_batched(chol_dtype dt, int64_t n, int64_t nrhs, int64_t batch, const void *L, int64_t ldl,
                               int64_t strideL, const void *B, int64_t ldb, int64_t strideB, void *X, int64_t ldx,
                               int64_t strideX, void *stream)
{
    if (n > CHOL_SMALL_MAX_N && valid_dtype(dt) && nrhs >= 0 && batch >= 0)
        return CHOL_ERR_NOT_SUPPORTED;
    bool noop;
    chol_status s = potrs_args(dt, n, nrhs, batch, L, ldl, strideL, B, ldb, strideB, X, ldx, strideX, &noop);
    if (s != CHOL_OK || noop)
        return s;
    hipStream_t st = (hipStream_t)stream;
    clear_stale_status();
    if (dt == CHOL_F64)
        return chol::small_potrs<double>((int)n, (int)nrhs, batch, (const double *)L, ldl, strideL,
                                         (const double *)B, ldb, strideB, (double *)X, ldx, strideX, st);
    return chol::small_potrs<float>((int)n, (int)nrhs, batch, (const float *)L, ldl, strideL, (const float *)B, ldb,
                                    strideB, (float *)X, ldx, strideX, st);
}

namespace {
chol_status potrs_adjoint_args(chol_dtype dt, int64_t n, int64_t nrhs, int64_t batch, const void *L, int64_t ldl,
                               int64_t sL, const void *X, int64_t ldx, int64_t sX, const void *adjX, int64_t ldax,
                               int64_t saX, const void *adjB, int64_t ldab, int64_t saB, const void *adjL,
                               int64_t ldal, int64_t saL, bool *noop)
{
    // adj_B = solve(adj_X): the solve's own rules (adj_B may be adj_X)
    chol_status s = potrs_args(dt, n, nrhs, batch, L, ldl, sL, adjX, ldax, saX, adjB, ldab, saB, noop);
    if (s != CHOL_OK)
        return s;
    if (*noop) {
        // no right-hand side: adj_L's term is zero, and only adj_L is touched
        if (n == 0 || batch == 0)
            return CHOL_OK;
        if (!adjL || !ld_ok(ldal, n) || !stride_ok(saL, ldal, n, batch))
            return CHOL_ERR_INVALID_VALUE;
        return CHOL_OK;
    }
    if (!X || !adjL || !ld_ok(ldx, nrhs) || !ld_ok(ldal, n) || !stride_ok(sX, ldx, n, batch) ||
        !stride_ok(saL, ldal, n, batch))
        return CHOL_ERR_INVALID_VALUE;
    const size_t es = esize(dt);
    const Extent eB = rect_extent(adjB, n, nrhs, ldab, batch, saB, es);
    const Extent eL = extent(adjL, n, ldal, batch, saL, es);
    // outputs (adj_B, adj_L) apart from each other and from the inputs they do not replace
    if (overlap(eB, eL) || overlap(eB, rect_extent(X, n, nrhs, ldx, batch, sX, es)) ||
        overlap(eL, extent(L, n, ldl, batch, sL, es)) || overlap(eL, rect_extent(X, n, nrhs, ldx, batch, sX, es)) ||
        overlap(eL, rect_extent(adjX, n, nrhs, ldax, batch, saX, es)))
        return CHOL_ERR_INVALID_VALUE;
    return CHOL_OK;
}
} // namespace

chol_status chol_potrs_adjoint_workspace_size(chol_dtype dt, int64_t n, int64_t nrhs, int64_t nb, size_t *bytes)
{
    if (!bytes || !valid_dtype(dt) || n < 0 || nrhs < 0 || !nb_ok(nb))
        return CHOL_ERR_INVALID_VALUE;
    *bytes = 0;
    if (n <= CHOL_SMALL_MAX_N || nrhs == 0)
        return CHOL_OK;
    if (n > MAX_N || nrhs > INT32_MAX / 2)
        return CHOL_ERR_NOT_SUPPORTED;
    *bytes = chol::blocked_solve_adjoint_workspace(n, nrhs, nb ? (int)nb : DEFAULT_NB, esize(dt));
    return CHOL_OK;
}

chol_status chol_potrs_adjoint(chol_dtype dt, int64_t n, int64_t nrhs, const void *L, int64_t ldl, const void *X,
                               int64_t ldx, const void *adjX, int64_t ldax, void *adjB, int64_t ldab, void *adjL,
                               int64_t ldal, int accumulate, int64_t nb, void *workspace, size_t workspace_bytes,
                               void *stream)
{
    if (!nb_ok(nb))
        return CHOL_ERR_INVALID_VALUE;
    bool noop;
    chol_status s = potrs_adjoint_args(dt, n, nrhs, 1, L, ldl, 0, X, ldx, 0, adjX, ldax, 0, adjB, ldab, 0, adjL,
                                       ldal, 0, &noop);
    if (s != CHOL_OK)
        return s;
    hipStream_t st = (hipStream_t)stream;
    if (noop) {
        // nrhs == 0: adj_L's term is zero (overwrite mode clears its lower triangle)
        if (n == 0 || accumulate)
            return CHOL_OK;
        clear_stale_status();
        return chol::zero_lower_batched(esize(dt), n, 1, adjL, ldal, 0, st);
    }
    const size_t es = esize(dt);
    clear_stale_status();
    if (n <= CHOL_SMALL_MAX_N) {
        if (dt == CHOL_F64)
            return chol::small_potrs_adjoint<double>((int)n, (int)nrhs, 1, (const double *)L, ldl, 0,
                                                     (const double *)X, ldx, 0, (const double *)adjX, ldax, 0,
                                                     (double *)adjB, ldab, 0, (double *)adjL, ldal, 0, accumulate,
                                                     st);
        return chol::small_potrs_adjoint<float>((int)n, (int)nrhs, 1, (const float *)L, ldl, 0, (const float *)X,
                                                ldx, 0, (const float *)adjX, ldax, 0, (float *)adjB, ldab, 0,
                                                (float *)adjL, ldal, 0, accumulate, st);
    }
    if (nrhs > INT32_MAX / 2)
        return CHOL_ERR_NOT_SUPPORTED;
    const int b = nb ? (int)nb : DEFAULT_NB;
    const size_t need = chol::blocked_solve_adjoint_workspace(n, nrhs, b, es);
    if (!workspace || workspace_bytes < need)
        return CHOL_ERR_WORKSPACE;
    const Extent ws{(uintptr_t)workspace, (uintptr_t)workspace + need};
    if (overlap(ws, extent(L, n, ldl, 1, 0, es)) || overlap(ws, rect_extent(X, n, nrhs, ldx, 1, 0, es)) ||
        overlap(ws, rect_extent(adjX, n, nrhs, ldax, 1, 0, es)) ||
        overlap(ws, rect_extent(adjB, n, nrhs, ldab, 1, 0, es)) || overlap(ws, extent(adjL, n, ldal, 1, 0, es)))
        return CHOL_ERR_INVALID_VALUE;
    if (dt == CHOL_F64)
        return chol::blocked_potrs_adjoint<double>(n, nrhs, (const double *)L, ldl, (const double *)X, ldx,
                                                   (const double *)adjX, ldax, (double *)adjB, ldab, (double *)adjL,
                                                   ldal, accumulate, b, workspace, st);
    return chol::blocked_potrs_adjoint<float>(n, nrhs, (const float *)L, ldl, (const float *)X, ldx,
                                              (const float *)adjX, ldax, (float *)adjB, ldab, (float *)adjL, ldal,
                                              accumulate, b, workspace, st);
}

chol_status chol_potrs_adjoint_batched(chol_dtype dt, int64_t n, int64_t nrhs, int64_t batch, const void *L,
                                       int64_t ldl, int64_t strideL, const void *X, int64_t ldx, int64_t strideX,
                                       const void *adjX, int64_t ldax, int64_t strideAX, void *adjB, int64_t ldab,
                                       int64_t strideAB, void *adjL, int64_t ldal, int64_t strideAL, int accumulate,
                                       void *stream)
{
    if (n > CHOL_SMALL_MAX_N && valid_dtype(dt) && nrhs >= 0 && batch >= 0)
        return CHOL_ERR_NOT_SUPPORTED;
    bool noop;
    chol_status s = potrs_adjoint_args(dt, n, nrhs, batch, L, ldl, strideL, X, ldx, strideX, adjX, ldax, strideAX,
                                       adjB, ldab, strideAB, adjL, ldal, strideAL, &noop);
    if (s != CHOL_OK)
        return s;
    hipStream_t st = (hipStream_t)stream;
    if (noop) {
        if (n == 0 || batch == 0 || accumulate)
            return CHOL_OK;
        clear_stale_status();
        return chol::zero_lower_batched(esize(dt), n, batch, adjL, ldal, strideAL, st);
    }
    clear_stale_status();
    if (dt == CHOL_F64)
        return chol::small_potrs_adjoint<double>((int)n, (int)nrhs, batch, (const double *)L, ldl, strideL,
                                                 (const double *)X, ldx, strideX, (const double *)adjX, ldax,
                                                 strideAX, (double *)adjB, ldab, strideAB, (double *)adjL, ldal,
                                                 strideAL, accumulate, st);
    return chol::small_potrs_adjoint<float>((int)n, (int)nrhs, batch, (const float *)L, ldl, strideL,
                                            (const float *)X, ldx, strideX, (const float *)adjX, ldax, strideAX,
                                            (float *)adjB, ldab, strideAB, (float *)adjL, ldal, strideAL,
                                            accumulate, st);
}

// ------------------------------------------------------------ upper form ----

extern "C++" {
namespace {
template <typename T>
chol_status potrf_upper_t(int64_t n, int64_t batch, const T *A, int64_t lda, int64_t sA, T *U, int64_t ldu,
                          int64_t sU, int32_t *info, int nb, hipStream_t st)
{
    chol_status s = chol::upper_to_lower<T>(n, batch, A, lda, sA, U, ldu, sU, st);
    if (s != CHOL_OK)
        return s;
    if (n <= CHOL_SMALL_MAX_N)
        s = chol::small_potrf<T>((int)n, batch, U, ldu, sU, U, ldu, sU, info, 0, 0, st);
    else
        s = chol::blocked_potrf<T>(n, U, ldu, U, ldu, info, nb, st);
    if (s != CHOL_OK)
        return s;
    return chol::lower_to_upper<T>(n, batch, U, ldu, sU, st);
}

// workspace of the upper adjoint: U^T and adj_U^T (n x n each, per matrix),
// then the lower-form adjoint's own (single matrix, n > CHOL_SMALL_MAX_N)
size_t upper_adjoint_workspace(int64_t n, int64_t batch, int nb, size_t es)
{
    const size_t mat = ((size_t)batch * n * n * es + 255) & ~(size_t)255;
    size_t bytes = 2 * mat;
    if (n > CHOL_SMALL_MAX_N)
        bytes += chol::blocked_adjoint_workspace(n, nb, es, false);
    return bytes;
}

template <typename T>
chol_status potrf_adjoint_upper_t(int64_t n, int64_t batch, const T *U, int64_t ldu, int64_t sU, const T *adjU,
                                  int64_t ldau, int64_t sAU, T *adjA, int64_t ldaa, int64_t sAA, int accumulate,
                                  int nb, void *ws, hipStream_t st)
{
    const size_t mat = ((size_t)batch * n * n * sizeof(T) + 255) & ~(size_t)255;
    T *Lt = (T *)ws;
    T *Gt = (T *)((char *)ws + mat);
    void *inner = (char *)ws + 2 * mat;
    const int64_t nn = n * n;
    chol_status s = chol::upper_to_lower<T>(n, batch, U, ldu, sU, Lt, n, nn, st);
    if (s == CHOL_OK)
        s = chol::upper_to_lower<T>(n, batch, adjU, ldau, sAU, Gt, n, nn, st);
    if (s != CHOL_OK)
        return s;
    // G (lower form) written over adj_L's transposed copy
    if (n <= CHOL_SMALL_MAX_N)
        s = chol::small_potrf_adjoint<T>((int)n, batch, Lt, n, nn, Gt, n, nn, Gt, n, nn, 0, st);
    else
        s = chol::blocked_adjoint<T>(n, Lt, n, Gt, n, Gt, n, 0, nb, inner, st);
    if (s != CHOL_OK)
        return s;
    return chol::add_upper_from_lower<T>(n, batch, Gt, n, nn, adjA, ldaa, sAA, accumulate, st);
}
} // namespace
} // extern "C++"

chol_status chol_potrf_upper(chol_dtype dt, int64_t n, const void *A, int64_t lda, void *U, int64_t ldu,
                             int32_t *info, int64_t nb, void *stream)
{
    if (!valid_dtype(dt) || n < 0 || !nb_ok(nb))
        return CHOL_ERR_INVALID_VALUE;
    if (n == 0)
        return CHOL_OK;
    if (!A || !U || !ld_ok(lda, n) || !ld_ok(ldu, n))
        return CHOL_ERR_INVALID_VALUE;
    if (n > MAX_N)
        return CHOL_ERR_NOT_SUPPORTED;
    const size_t es = esize(dt);
    if (!alias_ok(A, lda, 0, U, ldu, 0, n, 1, es))
        return CHOL_ERR_INVALID_VALUE;
    if (info && overlap(extent(info, 1, 1, 1, 0, 4), extent(U, n, ldu, 1, 0, es)))
        return CHOL_ERR_INVALID_VALUE;
    hipStream_t st = (hipStream_t)stream;
    clear_stale_status();
    const int b = nb ? (int)nb : DEFAULT_NB;
    if (dt == CHOL_F64)
        return potrf_upper_t<double>(n, 1, (const double *)A, lda, 0, (double *)U, ldu, 0, info, b, st);
    return potrf_upper_t<float>(n, 1, (const float *)A, lda, 0, (float *)U, ldu, 0, info, b, st);
}

chol_status chol_potrf_upper_batched(chol_dtype dt, int64_t n, int64_t batch, const void *A, int64_t lda,
                                     int64_t strideA, void *U, int64_t ldu, int64_t strideU, int32_t *info,
                                     void *stream)
{
    if (!valid_dtype(dt) || n < 0 || batch < 0)
        return CHOL_ERR_INVALID_VALUE;
    if (n > CHOL_SMALL_MAX_N)
        return CHOL_ERR_NOT_SUPPORTED;
    if (n == 0 || batch == 0)
        return CHOL_OK;
    if (!A || !U || !ld_ok(lda, n) || !ld_ok(ldu, n) || !stride_ok(strideA, lda, n, batch) ||
        !stride_ok(strideU, ldu, n, batch))
        return CHOL_ERR_INVALID_VALUE;
    if (batch > ((int64_t)1 << 31) - 1)
        return CHOL_ERR_NOT_SUPPORTED;
    const size_t es = esize(dt);
    if (!alias_ok(A, lda, strideA, U, ldu, strideU, n, batch, es))
        return CHOL_ERR_INVALID_VALUE;
    if (info && overlap(extent(info, 1, 1, batch, 1, 4), extent(U, n, ldu, batch, strideU, es)))
        return CHOL_ERR_INVALID_VALUE;
    hipStream_t st = (hipStream_t)stream;
    clear_stale_status();
    if (dt == CHOL_F64)
        return potrf_upper_t<double>(n, batch, (const double *)A, lda, strideA, (double *)U, ldu, strideU, info,
                                     DEFAULT_NB, st);
    return potrf_upper_t<float>(n, batch, (const float *)A, lda, strideA, (float *)U, ldu, strideU, info,
                                DEFAULT_NB, st);
}

chol_status chol_potrf_adjoint_upper_workspace_size(chol_dtype dt, int64_t n, int64_t batch, int64_t nb,
                                                    size_t *bytes)
{
    if (!bytes || !valid_dtype(dt) || n < 0 || batch < 0 || !nb_ok(nb))
        return CHOL_ERR_INVALID_VALUE;
    *bytes = 0;
    if (n == 0 || batch == 0)
        return CHOL_OK;
    if (n > MAX_N || (batch > 1 && n > CHOL_SMALL_MAX_N))
        return CHOL_ERR_NOT_SUPPORTED;
    *bytes = upper_adjoint_workspace(n, batch, nb ? (int)nb : DEFAULT_NB, esize(dt));
    return CHOL_OK;
}

namespace {
chol_status adjoint_upper_entry(chol_dtype dt, int64_t n, int64_t batch, const void *U, int64_t ldu, int64_t sU,
                                const void *adjU, int64_t ldau, int64_t sAU, void *adjA, int64_t ldaa, int64_t sAA,
                                int accumulate, int64_t nb, void *workspace, size_t workspace_bytes, void *stream)
{
    if (!valid_dtype(dt) || n < 0 || batch < 0 || !nb_ok(nb))
        return CHOL_ERR_INVALID_VALUE;
    if (batch > 1 && n > CHOL_SMALL_MAX_N)
        return CHOL_ERR_NOT_SUPPORTED;
    if (n == 0 || batch == 0)
        return CHOL_OK;
    if (!U || !adjU || !adjA || !ld_ok(ldu, n) || !ld_ok(ldau, n) || !ld_ok(ldaa, n) ||
        !stride_ok(sU, ldu, n, batch) || !stride_ok(sAU, ldau, n, batch) || !stride_ok(sAA, ldaa, n, batch))
        return CHOL_ERR_INVALID_VALUE;
    if (n > MAX_N || batch > ((int64_t)1 << 31) - 1)
        return CHOL_ERR_NOT_SUPPORTED;
    const size_t es = esize(dt);
    // adj_A may be adj_U itself (it is read into the workspace first), not U
    if (!alias_ok(adjU, ldau, sAU, adjA, ldaa, sAA, n, batch, es) ||
        overlap(extent(U, n, ldu, batch, sU, es), extent(adjA, n, ldaa, batch, sAA, es)))
        return CHOL_ERR_INVALID_VALUE;
    const int b = nb ? (int)nb : DEFAULT_NB;
    const size_t need = upper_adjoint_workspace(n, batch, b, es);
    if (!workspace || workspace_bytes < need)
        return CHOL_ERR_WORKSPACE;
    const Extent ws{(uintptr_t)workspace, (uintptr_t)workspace + need};
    if (overlap(ws, extent(U, n, ldu, batch, sU, es)) || overlap(ws, extent(adjU, n, ldau, batch, sAU, es)) ||
        overlap(ws, extent(adjA, n, ldaa, batch, sAA, es)))
        return CHOL_ERR_INVALID_VALUE;
    hipStream_t st = (hipStream_t)stream;
    clear_stale_status();
    if (dt == CHOL_F64)
        return potrf_adjoint_upper_t<double>(n, batch, (const double *)U, ldu, sU, (const double *)adjU, ldau, sAU,
                                             (double *)adjA, ldaa, sAA, accumulate, b, workspace, st);
    return potrf_adjoint_upper_t<float>(n, batch, (const float *)U, ldu, sU, (const float *)adjU, ldau, sAU,
                                        (float *)adjA, ldaa, sAA, accumulate, b, workspace, st);
}
} // namespace

chol_status chol_potrf_adjoint_upper(chol_dtype dt, int64_t n, const void *U, int64_t ldu, const void *adjU,
                                     int64_t ldau, void *adjA, int64_t ldaa, int accumulate, int64_t nb,
                                     void *workspace, size_t workspace_bytes, void *stream)
{
    return adjoint_upper_entry(dt, n, 1, U, ldu, 0, adjU, ldau, 0, adjA, ldaa, 0, accumulate, nb, workspace,
                               workspace_bytes, stream);
}

chol_status chol_potrf_adjoint_upper_batched(chol_dtype dt, int64_t n, int64_t batch, const void *U, int64_t ldu,
                                             int64_t strideU, const void *adjU, int64_t ldau, int64_t strideAU,
                                             void *adjA, int64_t ldaa, int64_t strideAA, int accumulate,
                                             void *workspace, size_t workspace_bytes, void *stream)
{
    if (valid_dtype(dt) && n > CHOL_SMALL_MAX_N && batch >= 0)
        return CHOL_ERR_NOT_SUPPORTED;
    return adjoint_upper_entry(dt, n, batch, U, ldu, strideU, adjU, ldau, strideAU, adjA, ldaa, strideAA, accumulate,
                               0, workspace, workspace_bytes, stream);
}

// ------------------------------------------------------ Hermitian complex ----

extern "C++" {
namespace {
bool complex_dtype(chol_dtype dt) { return dt == CHOL_C64 || dt == CHOL_C128; }
size_t real_esize(chol_dtype dt) { return dt == CHOL_C128 ? 8 : 4; }
size_t align_up(size_t x) { return (x + 255) & ~(size_t)255; }

// the real 2n x 2n embedding of each matrix (per matrix 4 n^2 reals)
size_t herm_embedding_bytes(int64_t n, int64_t batch, size_t res)
{
    return align_up((size_t)batch * 4 * n * n * res);
}

template <typename T>
chol_status herm_potrf_t(int64_t n, int64_t batch, const T *A, int64_t lda, int64_t sA, T *L, int64_t ldl,
                         int64_t sL, int32_t *info, int nb, void *ws, hipStream_t st)
{
    T *M = (T *)ws;
    const int64_t m = 2 * n, mm = m * m;
    chol_status s = chol::herm_embed<T>(n, batch, A, lda, sA, M, m, mm, st);
    if (s != CHOL_OK)
        return s;
    if (m <= CHOL_SMALL_MAX_N)
        s = chol::small_potrf<T>((int)m, batch, M, m, mm, M, m, mm, info, 0, 0, st);
    else
        s = chol::blocked_potrf<T>(m, M, m, M, m, info, nb, st);
    if (s == CHOL_OK)
        s = chol::herm_read_back<T>(n, batch, M, m, mm, L, ldl, sL, st);
    if (s == CHOL_OK)
        s = chol::herm_info(batch, info, st);
    return s;
}

size_t herm_adjoint_bytes(int64_t n, int64_t batch, int nb, size_t res)
{
    size_t bytes = 2 * herm_embedding_bytes(n, batch, res);
    if (2 * n > CHOL_SMALL_MAX_N)
        bytes += chol::blocked_adjoint_workspace(2 * n, nb, res, false);
    return bytes;
}

template <typename T>
chol_status herm_adjoint_t(int64_t n, int64_t batch, const T *L, int64_t ldl, int64_t sL, const T *adjL, int64_t ldal,
                           int64_t sAL, T *adjA, int64_t ldaa, int64_t sAA, int accumulate, int nb, void *ws,
                           hipStream_t st)
{
    const size_t emb = herm_embedding_bytes(n, batch, sizeof(T));
    T *E = (T *)ws;
    T *aE = (T *)((char *)ws + emb);
    void *inner = (char *)ws + 2 * emb;
    const int64_t m = 2 * n, mm = m * m;
    chol_status s = chol::herm_embed<T>(n, batch, L, ldl, sL, E, m, mm, st);
    if (s == CHOL_OK)
        s = chol::herm_embed_adjoint<T>(n, batch, adjL, ldal, sAL, aE, m, mm, st);
    if (s != CHOL_OK)
        return s;
    // the real gradient of M's lower entries, written over adj_E
    if (m <= CHOL_SMALL_MAX_N)
        s = chol::small_potrf_adjoint<T>((int)m, batch, E, m, mm, aE, m, mm, aE, m, mm, 0, st);
    else
        s = chol::blocked_adjoint<T>(m, E, m, aE, m, aE, m, 0, nb, inner, st);
    if (s != CHOL_OK)
        return s;
    return chol::herm_fold<T>(n, batch, aE, m, mm, adjA, ldaa, sAA, accumulate, st);
}

// argument checks shared by the Hermitian entry points (sizes in complex
// elements); CHOL_OK with *noop for empty problems
chol_status herm_args(chol_dtype dt, int64_t n, int64_t batch, const void *X, int64_t ldx, int64_t sX, const void *Y,
                      int64_t ldy, int64_t sY, bool *noop)
{
    *noop = false;
    if (!complex_dtype(dt) || n < 0 || batch < 0)
        return CHOL_ERR_INVALID_VALUE;
    if (n == 0 || batch == 0) {
        *noop = true;
        return CHOL_OK;
    }
    if (!X || !Y || !ld_ok(ldx, n) || !ld_ok(ldy, n) || !stride_ok(sX, ldx, n, batch) || !stride_ok(sY, ldy, n, batch))
        return CHOL_ERR_INVALID_VALUE;
    if (n > MAX_N / 2 || batch > ((int64_t)1 << 31) - 1)
        return CHOL_ERR_NOT_SUPPORTED;
    return CHOL_OK;
}
} // namespace
} // extern "C++"

chol_status chol_potrf_hermitian_workspace_size(chol_dtype dt, int64_t n, int64_t batch, int64_t nb, int adjoint,
                                                size_t *bytes)
{
    if (!bytes || !complex_dtype(dt) || n < 0 || batch < 0 || !nb_ok(nb))
        return CHOL_ERR_INVALID_VALUE;
    *bytes = 0;
    if (n == 0 || batch == 0)
        return CHOL_OK;
    if (n > MAX_N / 2 || (batch > 1 && 2 * n > CHOL_SMALL_MAX_N))
        return CHOL_ERR_NOT_SUPPORTED;
    const int b = nb ? (int)nb : DEFAULT_NB;
    *bytes = adjoint ? herm_adjoint_bytes(n, batch, b, real_esize(dt)) : herm_embedding_bytes(n, batch, real_esize(dt));
    return CHOL_OK;
}

namespace {
chol_status herm_potrf_entry(chol_dtype dt, int64_t n, int64_t batch, const void *A, int64_t lda, int64_t sA, void *L,
                             int64_t ldl, int64_t sL, int32_t *info, int64_t nb, void *workspace,
                             size_t workspace_bytes, void *stream)
{
    if (!nb_ok(nb))
        return CHOL_ERR_INVALID_VALUE;
    bool noop;
    chol_status s = herm_args(dt, n, batch, A, lda, sA, L, ldl, sL, &noop);
    if (s != CHOL_OK || noop)
        return s;
    if (batch > 1 && 2 * n > CHOL_SMALL_MAX_N)
        return CHOL_ERR_NOT_SUPPORTED;
    const size_t ce = 2 * real_esize(dt);
    if (!alias_ok(A, lda, sA, L, ldl, sL, n, batch, ce))
        return CHOL_ERR_INVALID_VALUE;
    if (info && overlap(extent(info, 1, 1, batch, 1, 4), extent(L, n, ldl, batch, sL, ce)))
        return CHOL_ERR_INVALID_VALUE;
    const size_t need = herm_embedding_bytes(n, batch, real_esize(dt));
    if (!workspace || workspace_bytes < need)
        return CHOL_ERR_WORKSPACE;
    const Extent ws{(uintptr_t)workspace, (uintptr_t)workspace + need};
    if (overlap(ws, extent(A, n, lda, batch, sA, ce)) || overlap(ws, extent(L, n, ldl, batch, sL, ce)) ||
        (info && overlap(ws, extent(info, 1, 1, batch, 1, 4))))
        return CHOL_ERR_INVALID_VALUE;
    hipStream_t st = (hipStream_t)stream;
    clear_stale_status();
    const int b = nb ? (int)nb : DEFAULT_NB;
    if (dt == CHOL_C128)
        return herm_potrf_t<double>(n, batch, (const double *)A, lda, sA, (double *)L, ldl, sL, info, b, workspace, st);
    return herm_potrf_t<float>(n, batch, (const float *)A, lda, sA, (float *)L, ldl, sL, info, b, workspace, st);
}

chol_status herm_adjoint_entry(chol_dtype dt, int64_t n, int64_t batch, const void *L, int64_t ldl, int64_t sL,
                               const void *adjL, int64_t ldal, int64_t sAL, void *adjA, int64_t ldaa, int64_t sAA,
                               int accumulate, int64_t nb, void *workspace, size_t workspace_bytes, void *stream)
{
    if (!nb_ok(nb))
        return CHOL_ERR_INVALID_VALUE;
    bool noop;
    chol_status s = herm_args(dt, n, batch, L, ldl, sL, adjL, ldal, sAL, &noop);
    if (s != CHOL_OK || noop)
        return s;
    if (!adjA || !ld_ok(ldaa, n) || !stride_ok(sAA, ldaa, n, batch))
        return CHOL_ERR_INVALID_VALUE;
    if (batch > 1 && 2 * n > CHOL_SMALL_MAX_N)
        return CHOL_ERR_NOT_SUPPORTED;
    const size_t ce = 2 * real_esize(dt);
    // adj_A may be adj_L itself (adj_L is embedded first), not L
    if (!alias_ok(adjL, ldal, sAL, adjA, ldaa, sAA, n, batch, ce) ||
        overlap(extent(L, n, ldl, batch, sL, ce), extent(adjA, n, ldaa, batch, sAA, ce)))
        return CHOL_ERR_INVALID_VALUE;
    const int b = nb ? (int)nb : DEFAULT_NB;
    const size_t need = herm_adjoint_bytes(n, batch, b, real_esize(dt));
    if (!workspace || workspace_bytes < need)
        return CHOL_ERR_WORKSPACE;
    const Extent ws{(uintptr_t)workspace, (uintptr_t)workspace + need};
    if (overlap(ws, extent(L, n, ldl, batch, sL, ce)) || overlap(ws, extent(adjL, n, ldal, batch, sAL, ce)) ||
        overlap(ws, extent(adjA, n, ldaa, batch, sAA, ce)))
        return CHOL_ERR_INVALID_VALUE;
    hipStream_t st = (hipStream_t)stream;
    clear_stale_status();
    if (dt == CHOL_C128)
        return herm_adjoint_t<double>(n, batch, (const double *)L, ldl, sL, (const double *)adjL, ldal, sAL,
                                      (double *)adjA, ldaa, sAA, accumulate, b, workspace, st);
    return herm_adjoint_t<float>(n, batch, (const float *)L, ldl, sL, (const float *)adjL, ldal, sAL, (float *)adjA,
                                 ldaa, sAA, accumulate, b, workspace, st);
}
} // namespace

chol_status chol_potrf_hermitian(chol_dtype dt, int64_t n, const void *A, int64_t lda, void *L, int64_t ldl,
                                 int32_t *info, int64_t nb, void *workspace, size_t workspace_bytes, void *stream)
{
    return herm_potrf_entry(dt, n, 1, A, lda, 0, L, ldl, 0, info, nb, workspace, workspace_bytes, stream);
}

chol_status chol_potrf_hermitian_batched(chol_dtype dt, int64_t n, int64_t batch, const void *A, int64_t lda,
                                         int64_t strideA, void *L, int64_t ldl, int64_t strideL, int32_t *info,
                                         void *workspace, size_t workspace_bytes, void *stream)
{
    if (complex_dtype(dt) && 2 * n > CHOL_SMALL_MAX_N && batch >= 0)
        return CHOL_ERR_NOT_SUPPORTED;
    return herm_potrf_entry(dt, n, batch, A, lda, strideA, L, ldl, strideL, info, 0, workspace, workspace_bytes,
                            stream);
}

chol_status chol_potrf_adjoint_hermitian(chol_dtype dt, int64_t n, const void *L, int64_t ldl, const void *adjL,
                                         int64_t ldal, void *adjA, int64_t ldaa, int accumulate, int64_t nb,
                                         void *workspace, size_t workspace_bytes, void *stream)
{
    return herm_adjoint_entry(dt, n, 1, L, ldl, 0, adjL, ldal, 0, adjA, ldaa, 0, accumulate, nb, workspace,
                              workspace_bytes, stream);
}

chol_status chol_potrf_adjoint_hermitian_batched(chol_dtype dt, int64_t n, int64_t batch, const void *L, int64_t ldl,
                                                 int64_t strideL, const void *adjL, int64_t ldal, int64_t strideAL,
                                                 void *adjA, int64_t ldaa, int64_t strideAA, int accumulate,
                                                 void *workspace, size_t workspace_bytes, void *stream)
{
    if (complex_dtype(dt) && 2 * n > CHOL_SMALL_MAX_N && batch >= 0)
        return CHOL_ERR_NOT_SUPPORTED;
    return herm_adjoint_entry(dt, n, batch, L, ldl, strideL, adjL, ldal, strideAL, adjA, ldaa, strideAA, accumulate,
                              0, workspace, workspace_bytes, stream);
}

int chol_last_hip_error(void) { return chol::g_last_hip_error.load(std::memory_order_relaxed); }

const char *chol_last_hip_error_string(void)
{
    return hipGetErrorString((hipError_t)chol::g_last_hip_error.load(std::memory_order_relaxed));
}

chol_status chol_potrf(chol_dtype dt, int64_t n, const void *A, int64_t lda, void *L, int64_t ldl,
                       int32_t *info, int64_t nb, void *stream)
{
    if (!valid_dtype(dt) || n < 0 || !nb_ok(nb))
        return CHOL_ERR_INVALID_VALUE;
    if (n == 0)
        return CHOL_OK;
    if (!A || !L || !ld_ok(lda, n) || !ld_ok(ldl, n))
        return CHOL_ERR_INVALID_VALUE;
    if (n > MAX_N)
        return CHOL_ERR_NOT_SUPPORTED;
    const size_t es = esize(dt);
    if (!alias_ok(A, lda, 0, L, ldl, 0, n, 1, es))
        return CHOL_ERR_INVALID_VALUE;
    if (info && overlap(extent(info, 1, 1, 1, 0, 4), extent(L, n, ldl, 1, 0, es)))
        return CHOL_ERR_INVALID_VALUE;
    hipStream_t st = (hipStream_t)stream;
    clear_stale_status();
    const int b = nb ? (int)nb : DEFAULT_NB;
    if (dt == CHOL_F64) {
        if (n <= CHOL_SMALL_MAX_N)
            return chol::small_potrf<double>((int)n, 1, (const double *)A, lda, 0, (double *)L, ldl, 0, info, 0, 0, st);
        return chol::blocked_potrf<double>(n, (const double *)A, lda, (double *)L, ldl, info, b, st);
    }
    if (n <= CHOL_SMALL_MAX_N)
        return chol::small_potrf<float>((int)n, 1, (const float *)A, lda, 0, (float *)L, ldl, 0, info, 0, 0, st);
    return chol::blocked_potrf<float>(n, (const float *)A, lda, (float *)L, ldl, info, b, st);
}

chol_status chol_potrf_batched(chol_dtype dt, int64_t n, int64_t batch, const void *A, int64_t lda,
                               int64_t strideA, void *L, int64_t ldl, int64_t strideL, int32_t *info,
                               void *stream)
{
    if (!valid_dtype(dt) || n < 0 || batch < 0)
        return CHOL_ERR_INVALID_VALUE;
    if (n > CHOL_SMALL_MAX_N)
        return CHOL_ERR_NOT_SUPPORTED;
    if (n == 0 || batch == 0)
        return CHOL_OK;
    if (!A || !L || !ld_ok(lda, n) || !ld_ok(ldl, n) || !stride_ok(strideA, lda, n, batch) ||
        !stride_ok(strideL, ldl, n, batch))
        return CHOL_ERR_INVALID_VALUE;
    if (batch > ((int64_t)1 << 31) - 1)
        return CHOL_ERR_NOT_SUPPORTED;
    const size_t es = esize(dt);
    if (!alias_ok(A, lda, strideA, L, ldl, strideL, n, batch, es))
        return CHOL_ERR_INVALID_VALUE;
    if (info && overlap(extent(info, 1, 1, batch, 1, 4), extent(L, n, ldl, batch, strideL, es)))
        return CHOL_ERR_INVALID_VALUE;
    hipStream_t st = (hipStream_t)stream;
    clear_stale_status();
    chol::prof::Scope ps(CHOL_K_SMALL_FACTOR, st, 2.0 * batch * ((double)n * (n + 1) / 2) * es);
    if (dt == CHOL_F64)
        return chol::small_potrf<double>((int)n, batch, (const double *)A, lda, strideA, (double *)L, ldl,
                                         strideL, info, 0, 0, st);
    return chol::small_potrf<float>((int)n, batch, (const float *)A, lda, strideA, (float *)L, ldl, strideL,
                                    info, 0, 0, st);
}

chol_status chol_potrf_adjoint_workspace_size(chol_dtype dt, int64_t n, int64_t nb, int accumulate,
                                              int in_place, size_t *bytes)
{
    if (!bytes || !valid_dtype(dt) || n < 0 || !nb_ok(nb) || (in_place && accumulate))
        return CHOL_ERR_INVALID_VALUE;
    *bytes = 0;
    if (n <= CHOL_SMALL_MAX_N)
        return CHOL_OK;
    if (n > MAX_N)
        return CHOL_ERR_NOT_SUPPORTED;
    *bytes = chol::blocked_adjoint_workspace(n, nb ? (int)nb : DEFAULT_NB, esize(dt), accumulate != 0);
    return CHOL_OK;
}

chol_status chol_potrf_adjoint(chol_dtype dt, int64_t n, const void *L, int64_t ldl, const void *adjL,
                               int64_t ldal, void *adjA, int64_t ldaa, int accumulate, int64_t nb,
                               void *workspace, size_t workspace_bytes, void *stream)
{
    if (!valid_dtype(dt) || n < 0 || !nb_ok(nb))
        return CHOL_ERR_INVALID_VALUE;
    if (n == 0)
        return CHOL_OK;
    if (!L || !adjL || !adjA || !ld_ok(ldl, n) || !ld_ok(ldal, n) || !ld_ok(ldaa, n))
        return CHOL_ERR_INVALID_VALUE;
    if (n > MAX_N)
        return CHOL_ERR_NOT_SUPPORTED;
    const size_t es = esize(dt);
    const bool in_place = adjA == adjL;
    if (in_place && accumulate)
        return CHOL_ERR_INVALID_VALUE;
    if (!alias_ok(adjL, ldal, 0, adjA, ldaa, 0, n, 1, es))
        return CHOL_ERR_INVALID_VALUE;
    if (overlap(extent(L, n, ldl, 1, 0, es), extent(adjA, n, ldaa, 1, 0, es)))
        return CHOL_ERR_INVALID_VALUE;
    hipStream_t st = (hipStream_t)stream;
    clear_stale_status();
    if (n <= CHOL_SMALL_MAX_N) {
        if (dt == CHOL_F64)
            return chol::small_potrf_adjoint<double>((int)n, 1, (const double *)L, ldl, 0, (const double *)adjL,
                                                     ldal, 0, (double *)adjA, ldaa, 0, accumulate, st);
        return chol::small_potrf_adjoint<float>((int)n, 1, (const float *)L, ldl, 0, (const float *)adjL, ldal,
                                                0, (float *)adjA, ldaa, 0, accumulate, st);
    }
    const int b = nb ? (int)nb : DEFAULT_NB;
    const size_t need = chol::blocked_adjoint_workspace(n, b, es, accumulate != 0);
    if (!workspace || workspace_bytes < need)
        return CHOL_ERR_WORKSPACE;
    const Extent ws{(uintptr_t)workspace, (uintptr_t)workspace + need};
    if (overlap(ws, extent(L, n, ldl, 1, 0, es)) || overlap(ws, extent(adjL, n, ldal, 1, 0, es)) ||
        overlap(ws, extent(adjA, n, ldaa, 1, 0, es)))
        return CHOL_ERR_INVALID_VALUE;
    if (dt == CHOL_F64)
        return chol::blocked_adjoint<double>(n, (const double *)L, ldl, (const double *)adjL, ldal,
                                             (double *)adjA, ldaa, accumulate, b, workspace, st);
    return chol::blocked_adjoint<float>(n, (const float *)L, ldl, (const float *)adjL, ldal, (float *)adjA,
                                        ldaa, accumulate, b, workspace, st);
}

chol_status chol_potrf_adjoint_noalloc(chol_dtype dt, int64_t n, const void *L, int64_t ldl, const void *adjL,
                                       int64_t ldal, void *adjA, int64_t ldaa, int accumulate, int64_t nb,
                                       void *stream)
{
    if (!valid_dtype(dt) || n < 0 || !nb_ok(nb))
        return CHOL_ERR_INVALID_VALUE;
    if (n == 0)
        return CHOL_OK;
    if (!L || !adjL || !adjA || !ld_ok(ldl, n) || !ld_ok(ldal, n) || !ld_ok(ldaa, n))
        return CHOL_ERR_INVALID_VALUE;
    if (n > CHOL_NOALLOC_MAX_N)
        return CHOL_ERR_NOT_SUPPORTED;
    const size_t es = esize(dt);
    const bool in_place = adjA == adjL;
    if (in_place && accumulate)
        return CHOL_ERR_INVALID_VALUE;
    if (!alias_ok(adjL, ldal, 0, adjA, ldaa, 0, n, 1, es))
        return CHOL_ERR_INVALID_VALUE;
    if (overlap(extent(L, n, ldl, 1, 0, es), extent(adjA, n, ldaa, 1, 0, es)))
        return CHOL_ERR_INVALID_VALUE;
    hipStream_t st = (hipStream_t)stream;
    clear_stale_status();
    if (n <= CHOL_SMALL_MAX_N) {
        if (dt == CHOL_F64)
            return chol::small_potrf_adjoint<double>((int)n, 1, (const double *)L, ldl, 0, (const double *)adjL,
                                                     ldal, 0, (double *)adjA, ldaa, 0, accumulate, st);
        return chol::small_potrf_adjoint<float>((int)n, 1, (const float *)L, ldl, 0, (const float *)adjL, ldal,
                                                0, (float *)adjA, ldaa, 0, accumulate, st);
    }
    const int b = nb ? (int)nb : DEFAULT_NB;
    if (chol::blocked_adjoint_workspace(n, b, es, accumulate != 0, chol::NOALLOC_SPLIT_MAX) >
        (size_t)CHOL_NOALLOC_SCRATCH_BYTES)
        return CHOL_ERR_NOT_SUPPORTED;
    chol::NoAlloc na;
    if (!chol::noalloc_resources(na))
        return CHOL_ERR_HIP;
    if (dt == CHOL_F64)
        return chol::blocked_adjoint_single_stream<double>(n, (const double *)L, ldl, (const double *)adjL, ldal,
                                                           (double *)adjA, ldaa, accumulate, b, na.scratch,
                                                           na.sched, na.cus, st);
    return chol::blocked_adjoint_single_stream<float>(n, (const float *)L, ldl, (const float *)adjL, ldal,
                                                      (float *)adjA, ldaa, accumulate, b, na.scratch, na.sched,
                                                      na.cus, st);
}

chol_status chol_potrf_adjoint_batched(chol_dtype dt, int64_t n, int64_t batch, const void *L, int64_t ldl,
                                       int64_t strideL, const void *adjL, int64_t ldal, int64_t strideAL,
                                       void *adjA, int64_t ldaa, int64_t strideAA, int accumulate,
                                       void *stream)
{
    if (!valid_dtype(dt) || n < 0 || batch < 0)
        return CHOL_ERR_INVALID_VALUE;
    if (n > CHOL_SMALL_MAX_N)
        return CHOL_ERR_NOT_SUPPORTED;
    if (n == 0 || batch == 0)
        return CHOL_OK;
    if (!L || !adjL || !adjA || !ld_ok(ldl, n) || !ld_ok(ldal, n) || !ld_ok(ldaa, n) ||
        !stride_ok(strideL, ldl, n, batch) || !stride_ok(strideAL, ldal, n, batch) ||
        !stride_ok(strideAA, ldaa, n, batch))
        return CHOL_ERR_INVALID_VALUE;
    if (batch > ((int64_t)1 << 31) - 1)
        return CHOL_ERR_NOT_SUPPORTED;
    const size_t es = esize(dt);
    if (adjA == adjL && accumulate)
        return CHOL_ERR_INVALID_VALUE;
    if (!alias_ok(adjL, ldal, strideAL, adjA, ldaa, strideAA, n, batch, es))
        return CHOL_ERR_INVALID_VALUE;
    if (overlap(extent(L, n, ldl, batch, strideL, es), extent(adjA, n, ldaa, batch, strideAA, es)))
        return CHOL_ERR_INVALID_VALUE;
    hipStream_t st = (hipStream_t)stream;
    clear_stale_status();
    chol::prof::Scope ps(CHOL_K_SMALL_ADJOINT, st,
                         (accumulate ? 4.0 : 3.0) * batch * ((double)n * (n + 1) / 2) * es);
    if (dt == CHOL_F64)
        return chol::small_potrf_adjoint<double>((int)n, batch, (const double *)L, ldl, strideL,
                                                 (const double *)adjL, ldal, strideAL, (double *)adjA, ldaa,
                                                 strideAA, accumulate, st);
    return chol::small_potrf_adjoint<float>((int)n, batch, (const float *)L, ldl, strideL, (const float *)adjL,
                                            ldal, strideAL, (float *)adjA, ldaa, strideAA, accumulate, st);
}

chol_status chol_hbm_stream(int mode, const void *src, void *dst, size_t bytes, void *stream)
{
    if (mode < 0 || mode > 2 || bytes % 16 != 0)
        return CHOL_ERR_INVALID_VALUE;
    if (bytes == 0)
        return CHOL_OK;
    if ((mode != 1 && (!src || (uintptr_t)src % 16)) || !dst || (uintptr_t)dst % 16)
        return CHOL_ERR_INVALID_VALUE;
    const size_t dst_bytes = mode == 0 ? (size_t)CHOL_HBM_READ_SINK_FLOATS * 4 : bytes;
    if (mode != 1) {
        const Extent a{(uintptr_t)src, (uintptr_t)src + bytes}, b{(uintptr_t)dst, (uintptr_t)dst + dst_bytes};
        if (overlap(a, b))
            return CHOL_ERR_INVALID_VALUE;
    }
    clear_stale_status();
    return chol::hbm_stream(mode, src, dst, bytes, (hipStream_t)stream);
}

chol_status chol_wave_dot_fwd_adj(chol_dtype dt, int64_t n, const void *a, const void *b, void *y,
                                  const void *ybar, void *abar, void *bbar, int staging, void *stream)
{
    if (!valid_dtype(dt) || n < 0 || n > 64 || (staging != 0 && staging != 1))
        return CHOL_ERR_INVALID_VALUE;
    if (!y || !ybar || (n > 0 && (!a || !b || !abar || !bbar)))
        return CHOL_ERR_INVALID_VALUE;
    hipStream_t st = (hipStream_t)stream;
    clear_stale_status();
    if (dt == CHOL_F64)
        return chol::wave_dot<double>((int)n, (const double *)a, (const double *)b, (double *)y,
                                      (const double *)ybar, (double *)abar, (double *)bbar, staging, st);
    return chol::wave_dot<float>((int)n, (const float *)a, (const float *)b, (float *)y, (const float *)ybar,
                                 (float *)abar, (float *)bbar, staging, st);
}

chol_status chol_wave_sum_fwd_adj(chol_dtype dt, int64_t n, const void *a, void *y, const void *ybar, void *abar,
                                  int staging, void *stream)
{
    if (!valid_dtype(dt) || n < 0 || n > 64 || (staging != 0 && staging != 1))
        return CHOL_ERR_INVALID_VALUE;
    if (!y || !ybar || (n > 0 && (!a || !abar)))
        return CHOL_ERR_INVALID_VALUE;
    hipStream_t st = (hipStream_t)stream;
    clear_stale_status();
    if (dt == CHOL_F64)
        return chol::wave_sum<double>((int)n, (const double *)a, (double *)y, (const double *)ybar, (double *)abar,
                                      staging, st);
    return chol::wave_sum<float>((int)n, (const float *)a, (float *)y, (const float *)ybar, (float *)abar, staging,
                                 st);
}

} // extern "C"
