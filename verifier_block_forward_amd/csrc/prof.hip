// prof.hip -- per-kernel timing for measurement (dbf_profile_start / dbf_profile_stop).
//
// While profiling is on, each launch the library makes takes a pair of HIP events
// from a pool and is dispatched with hipExtLaunchKernel, which binds the events to
// the dispatch itself: the elapsed time between them is the kernel's execution.
// Events are created on first use and kept for the next profile. The state is
// process-wide and guarded by a mutex; launches beyond the requested number run
// untimed.
#include <mutex>
#include <vector>

#include "../../include/dbf.h"
#include "kernels.hpp"

namespace dbf {

namespace {

struct ProfRec {
    int cls;
    const char *name;
    hipEvent_t e0, e1;
};

std::mutex g_mu;
bool g_on = false;
int g_cap = 0;
std::vector<ProfRec> g_recs;
std::vector<hipEvent_t> g_pool;  // every event created so far, reused in order
size_t g_pool_next = 0;

hipEvent_t pool_event() {
    if (g_pool_next < g_pool.size()) return g_pool[g_pool_next++];
    hipEvent_t e = nullptr;
    if (hipEventCreate(&e) != hipSuccess) return nullptr;
    g_pool.push_back(e);
    g_pool_next++;
    return e;
}

}  // namespace

bool prof_take(int cls, const char *name, hipEvent_t *e0, hipEvent_t *e1) {
    std::lock_guard<std::mutex> lk(g_mu);
    if (!g_on || (int)g_recs.size() >= g_cap) return false;
    ProfRec r{cls, name, pool_event(), pool_event()};
    if (!r.e0 || !r.e1) return false;
    g_recs.push_back(r);
    *e0 = r.e0;
    *e1 = r.e1;
    return true;
}

}  // namespace dbf

extern "C" {

int dbf_profile_start(int32_t max_records) {
    if (max_records < 1 || max_records > DBF_PROF_MAX_RECORDS) return DBF_EINVAL;
    std::lock_guard<std::mutex> lk(dbf::g_mu);
    dbf::g_recs.clear();
    dbf::g_recs.reserve((size_t)max_records);
    dbf::g_pool_next = 0;
    dbf::g_cap = max_records;
    dbf::g_on = true;
    return DBF_OK;
}

int dbf_profile_stop(dbf_prof_record *out, int32_t max_out, int32_t *n_out) {
    std::lock_guard<std::mutex> lk(dbf::g_mu);
    dbf::g_on = false;
    int rc = DBF_OK;
    const int n = (int)dbf::g_recs.size();
    for (int i = 0; i < n; i++) {
        const dbf::ProfRec &r = dbf::g_recs[i];
        float ms = 0.f;
        if (hipEventSynchronize(r.e1) != hipSuccess || hipEventElapsedTime(&ms, r.e0, r.e1) != hipSuccess)
            rc = DBF_EHIP;
        if (out && i < max_out) {
            out[i].cls = r.cls;
            out[i].reserved_ = 0;
            out[i].kernel = r.name;
            out[i].us = 1e3 * (double)ms;
        }
    }
    if (n_out) *n_out = n;
    dbf::g_recs.clear();
    dbf::g_pool_next = 0;
    return rc;
}

}  // extern "C"
