// clr_launch.h -- kernel launch helper with optional per-kernel timing.
//
// When timing is enabled (clr_timing_enable), each launch goes through
// hipExtLaunchKernelGGL with a start/stop event pair, so the duration of every
// kernel is measured on the stream it runs on; clr_timing_report aggregates
// them by kernel name.  Otherwise it is a plain hipLaunchKernelGGL.
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>

namespace clr {

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
