// clr_aux.hip -- the auxiliary stream of the split-and-overlap forward and
// its process-global split setting.
//
// Per device, one non-blocking stream (default priority) and a few events are
// created on first use and kept until the process ends.  A call that uses them
// holds a per-process lock while it enqueues, so the event record / wait
// pairs of two host threads never interleave.
#include <hip/hip_runtime.h>

#include <atomic>
#include <mutex>

#include "clr.h"
#include "clr_launch.h"

namespace clr {
namespace {
constexpr int MAX_DEV = 64;
struct AuxDev {
    hipStream_t s = nullptr;
    hipEvent_t ev[AUX_EVENTS] = {};
    bool tried = false;
};
std::mutex g_aux_mu;
AuxDev g_aux[MAX_DEV];
// Share of the blocks (per mille) that go into the first part; 0 = no split.
std::atomic<int> g_split{FWD_SPLIT_DEFAULT};
// Value columns per forward-scan work-group (16 or 32).
std::atomic<int> g_scan_bv{16};

void aux_release(AuxDev& a) {
    for (auto& e : a.ev)
        if (e) hipEventDestroy(e), e = nullptr;
    if (a.s) hipStreamDestroy(a.s), a.s = nullptr;
}
}  // namespace

int fwd_split_permille() { return g_split.load(std::memory_order_relaxed); }
int scan_bv() { return g_scan_bv.load(std::memory_order_relaxed); }

AuxGuard::AuxGuard(hipStream_t main) : lk_(g_aux_mu) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= MAX_DEV) return;
    if (main) {
        hipDevice_t sd = -1;
        if (hipStreamGetDevice(main, &sd) != hipSuccess || sd != dev) return;
    }
    AuxDev& a = g_aux[dev];
    if (!a.tried) {
        a.tried = true;
        bool ok = hipStreamCreateWithFlags(&a.s, hipStreamNonBlocking) == hipSuccess;
        for (auto& e : a.ev) ok = ok && hipEventCreateWithFlags(&e, hipEventDisableTiming) == hipSuccess;
        if (!ok) aux_release(a);
    }
    if (a.s) {
        stream = a.s;
        ev = a.ev;
    }
}

}  // namespace clr

extern "C" int clr_set_fwd_split(int permille) {
    if (permille < 0 || permille >= 1000) return CLR_EINVAL;
    clr::g_split.store(permille, std::memory_order_relaxed);
    return CLR_OK;
}

extern "C" int clr_get_fwd_split(void) { return clr::fwd_split_permille(); }

extern "C" int clr_set_scan_bv(int bv) {
    if (bv != 16 && bv != 32) return CLR_EINVAL;
    clr::g_scan_bv.store(bv, std::memory_order_relaxed);
    return CLR_OK;
}

extern "C" int clr_get_scan_bv(void) { return clr::scan_bv(); }
