// Per-kernel-family timing: an event pair around each launch of a family on
// the stream it runs on; chol_profile_stop() waits for the last event and sums
// the elapsed times per family.
#include "profile.hpp"

#include <mutex>
#include <vector>

namespace chol {
namespace prof {

std::atomic<uint32_t> g_mask{0};

namespace {
struct Rec {
    int id;
    hipEvent_t a, b;
    double work;
};
std::mutex g_mu;
std::vector<Rec> g_recs;
std::vector<hipEvent_t> g_pool;

hipEvent_t take()
{
    if (!g_pool.empty()) {
        hipEvent_t e = g_pool.back();
        g_pool.pop_back();
        return e;
    }
    hipEvent_t e = nullptr;
    if (hipEventCreate(&e) != hipSuccess)
        return nullptr;
    return e;
}
} // namespace

Scope::Scope(int id_, hipStream_t st_, double work_) : id(id_), st(st_), work(work_)
{
    if (id < 0 || id >= 32 || !((g_mask.load(std::memory_order_relaxed) >> id) & 1u))
        return;
    std::lock_guard<std::mutex> lk(g_mu);
    a = take();
    b = take();
    if (!a || !b) {
        if (a)
            g_pool.push_back(a);
        if (b)
            g_pool.push_back(b);
        a = b = nullptr;
        return;
    }
    (void)hipEventRecord(a, st);
}

Scope::~Scope()
{
    if (!a || !b)
        return;
    (void)hipEventRecord(b, st);
    std::lock_guard<std::mutex> lk(g_mu);
    g_recs.push_back(Rec{id, a, b, work});
}

LaunchEvents::LaunchEvents(int id_, double work_) : id(id_), work(work_)
{
    if (id < 0 || id >= 32 || !((g_mask.load(std::memory_order_relaxed) >> id) & 1u))
        return;
    std::lock_guard<std::mutex> lk(g_mu);
    a = take();
    b = take();
    if (!a || !b) {
        if (a)
            g_pool.push_back(a);
        if (b)
            g_pool.push_back(b);
        a = b = nullptr;
    }
}

LaunchEvents::~LaunchEvents()
{
    if (!a || !b)
        return;
    std::lock_guard<std::mutex> lk(g_mu);
    g_recs.push_back(Rec{id, a, b, work});
}

} // namespace prof
} // namespace chol

using namespace chol::prof;

extern "C" {

chol_status chol_profile_start(uint32_t mask)
{
    std::lock_guard<std::mutex> lk(g_mu);
    for (auto &r : g_recs) {
        g_pool.push_back(r.a);
        g_pool.push_back(r.b);
    }
    g_recs.clear();
    g_mask.store(mask);
    return CHOL_OK;
}

chol_status chol_profile_stop(int32_t max_ids, int64_t *count, double *ms, double *work)
{
    g_mask.store(0);
    std::lock_guard<std::mutex> lk(g_mu);
    if (max_ids < 0 || (max_ids > 0 && (!count || !ms || !work)))
        return CHOL_ERR_INVALID_VALUE;
    for (int i = 0; i < max_ids; ++i) {
        count[i] = 0;
        ms[i] = 0.0;
        work[i] = 0.0;
    }
    chol_status s = CHOL_OK;
    for (auto &r : g_recs) {
        float t = 0.f;
        if (hipEventSynchronize(r.b) != hipSuccess || hipEventElapsedTime(&t, r.a, r.b) != hipSuccess)
            s = CHOL_ERR_HIP;
        if (r.id >= 0 && r.id < max_ids) {
            count[r.id] += 1;
            ms[r.id] += t;
            work[r.id] += r.work;
        }
        g_pool.push_back(r.a);
        g_pool.push_back(r.b);
    }
    g_recs.clear();
    return s;
}

} // extern "C"
