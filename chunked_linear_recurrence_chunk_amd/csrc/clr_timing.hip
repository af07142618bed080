// clr_timing.hip -- per-kernel timing state behind clr_timing_enable /
// clr_timing_report (a profiling aid; not used unless enabled).
#include <hip/hip_runtime.h>
#include <string.h>

#include <mutex>
#include <string>
#include <vector>

#include "clr.h"
#include "clr_launch.h"

namespace clr {
namespace {
struct Rec {
    const char* name;
    hipEvent_t a, b;
};
std::mutex g_mu;
bool g_on = false;
std::vector<Rec> g_recs;
std::vector<hipEvent_t> g_free;

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

bool timing_on() {
    std::lock_guard<std::mutex> lk(g_mu);
    return g_on;
}

bool timing_events(hipEvent_t* a, hipEvent_t* b) {
    std::lock_guard<std::mutex> lk(g_mu);
    *a = take_event();
    *b = take_event();
    if (*a && *b) return true;
    if (*a) g_free.push_back(*a);
    if (*b) g_free.push_back(*b);
    return false;
}

void timing_record(const char* name, hipEvent_t a, hipEvent_t b) {
    std::lock_guard<std::mutex> lk(g_mu);
    g_recs.push_back({name, a, b});
}

}  // namespace clr

extern "C" {

int clr_timing_enable(int on) {
    std::lock_guard<std::mutex> lk(clr::g_mu);
    clr::g_on = on != 0;
    return CLR_OK;
}

int clr_timing_report(clr_kernel_time_t* out, int max_entries) {
    std::vector<clr::Rec> recs;
    {
        std::lock_guard<std::mutex> lk(clr::g_mu);
        recs.swap(clr::g_recs);
    }
    int n = 0, rc = CLR_OK;
    for (const auto& r : recs) {
        if (hipEventSynchronize(r.b) != hipSuccess) { rc = CLR_EHIP; continue; }
        float ms = 0.f;
        if (hipEventElapsedTime(&ms, r.a, r.b) != hipSuccess) { rc = CLR_EHIP; continue; }
        int i = 0;
        for (; i < n; ++i)
            if (strncmp(out[i].name, r.name, sizeof(out[i].name)) == 0) break;
        if (i == n) {
            if (n >= max_entries) continue;
            memset(&out[n], 0, sizeof(out[n]));
            strncpy(out[n].name, r.name, sizeof(out[n].name) - 1);
            ++n;
        }
        out[i].launches += 1;
        out[i].total_ms += ms;
    }
    {
        std::lock_guard<std::mutex> lk(clr::g_mu);
        for (const auto& r : recs) {
            clr::g_free.push_back(r.a);
            clr::g_free.push_back(r.b);
        }
    }
    return rc == CLR_OK ? n : -rc;
}

}  // extern "C"
