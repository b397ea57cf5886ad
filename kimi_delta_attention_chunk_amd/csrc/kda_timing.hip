// kda_timing.hip -- opt-in per-kernel timing for benchmarks and profiling.
//
// When enabled, every kernel the library launches is bracketed by a pair of
// hipEvents recorded on the caller's stream.  Nothing synchronises until the
// caller asks for the numbers (kda_timing_collect), so the enqueue path stays
// asynchronous.  Disabled (the default), the hooks cost one relaxed atomic load.
#include <atomic>
#include <mutex>
#include <string>
#include <vector>

#include "../../include/kda.h"
#include "kda_internal.h"

namespace kda {
namespace {

struct Pending {
    const char* name;
    hipEvent_t start, stop;
};
struct Total {
    std::string name;
    int64_t launches;
    double ms;
};

std::atomic<int> g_on{0};
std::mutex g_mu;
std::vector<Pending> g_pending;
std::vector<Total> g_totals;
std::vector<hipEvent_t> g_free;
thread_local hipEvent_t t_start = nullptr;

hipEvent_t take_event() {
    if (!g_free.empty()) {
        hipEvent_t e = g_free.back();
        g_free.pop_back();
        return e;
    }
    hipEvent_t e = nullptr;
    if (hipEventCreate(&e) != hipSuccess) return nullptr;
    return e;
}

}  // namespace

void prof_begin(hipStream_t s) {
    if (!g_on.load(std::memory_order_relaxed)) return;
    std::lock_guard<std::mutex> lk(g_mu);
    t_start = take_event();
    if (t_start) (void)hipEventRecord(t_start, s);
}

void prof_end(hipStream_t s, const char* name) {
    if (!g_on.load(std::memory_order_relaxed) || t_start == nullptr) return;
    std::lock_guard<std::mutex> lk(g_mu);
    hipEvent_t e = take_event();
    if (e == nullptr) return;
    (void)hipEventRecord(e, s);
    g_pending.push_back({name, t_start, e});
    t_start = nullptr;
}

}  // namespace kda

extern "C" {

int kda_timing_enable(int on) {
    std::lock_guard<std::mutex> lk(kda::g_mu);
    for (auto& p : kda::g_pending) {
        kda::g_free.push_back(p.start);
        kda::g_free.push_back(p.stop);
    }
    kda::g_pending.clear();
    kda::g_totals.clear();
    kda::g_on.store(on ? 1 : 0);
    return KDA_OK;
}

int kda_timing_collect(void) {
    std::lock_guard<std::mutex> lk(kda::g_mu);
    int rc = KDA_OK;
    for (auto& p : kda::g_pending) {
        float ms = 0.f;
        if (hipEventSynchronize(p.stop) != hipSuccess || hipEventElapsedTime(&ms, p.start, p.stop) != hipSuccess) {
            rc = KDA_ERR_HIP;
        } else {
            bool found = false;
            for (auto& t : kda::g_totals)
                if (t.name == p.name) { t.launches += 1; t.ms += ms; found = true; break; }
            if (!found) kda::g_totals.push_back({p.name, 1, (double)ms});
        }
        kda::g_free.push_back(p.start);
        kda::g_free.push_back(p.stop);
    }
    kda::g_pending.clear();
    return rc;
}

int kda_timing_count(void) {
    std::lock_guard<std::mutex> lk(kda::g_mu);
    return (int)kda::g_totals.size();
}

int kda_timing_get(int i, const char** name, int64_t* launches, double* total_ms) {
    std::lock_guard<std::mutex> lk(kda::g_mu);
    if (i < 0 || i >= (int)kda::g_totals.size() || !name || !launches || !total_ms) return KDA_ERR_INVALID;
    *name = kda::g_totals[i].name.c_str();
    *launches = kda::g_totals[i].launches;
    *total_ms = kda::g_totals[i].ms;
    return KDA_OK;
}

}  // extern "C"
