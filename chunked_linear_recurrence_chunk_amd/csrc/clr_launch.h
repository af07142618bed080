// clr_launch.h -- kernel launch helper with optional per-kernel timing.
//
// When timing is enabled (clr_timing_enable), each launch goes through
// hipExtLaunchKernelGGL with a start/stop event pair, so the duration of every
// kernel is measured on the stream it runs on; clr_timing_report aggregates
// them by kernel name.  Otherwise it is a plain hipLaunchKernelGGL.
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>

#include <mutex>

namespace clr {

// Split-and-overlap forward: share of a call's blocks (per mille) in the first
// part, 0 = no split.  Set through clr_set_fwd_split.  Off by default: each
// dependency between the two streams' hardware queues costs 10-20 us on
// MI355X (measured), more than the overlap can hide.
constexpr int FWD_SPLIT_DEFAULT = 0;
int fwd_split_permille();
// Value columns per work-group of the Gated DeltaNet forward scan (16 or 32);
// set through clr_set_scan_bv.
int scan_bv();

// The auxiliary stream of the current device and its events, held under a
// process-wide lock for the lifetime of the guard.  `stream` stays null when
// no auxiliary stream is available (creation failed, or `main` belongs to
// another device); the caller then runs the unsplit schedule.
constexpr int AUX_EVENTS = 4;
struct AuxGuard {
    explicit AuxGuard(hipStream_t main);
    hipStream_t stream = nullptr;
    hipEvent_t* ev = nullptr;

  private:
    std::lock_guard<std::mutex> lk_;
};

bool timing_on();
// Returns false if events could not be obtained (then the launch is untimed).
bool timing_events(hipEvent_t* start, hipEvent_t* stop);
void timing_record(const char* name, hipEvent_t start, hipEvent_t stop);

template <typename K, typename... Args>
inline void launch(const char* name, K kernel, dim3 grid, dim3 block, hipStream_t st, Args... args) {
    hipEvent_t a, b;
    if (timing_on() && timing_events(&a, &b)) {
        hipExtLaunchKernelGGL(kernel, grid, block, 0, st, a, b, 0, args...);
        timing_record(name, a, b);
    } else {
        hipLaunchKernelGGL(kernel, grid, block, 0, st, args...);
    }
}

}  // namespace clr
