// gla.hip -- GLA chunk forward/backward on gfx950 (in progress).
#include "clr_kernels.h"

namespace clr {
hipError_t launch_gla_fwd(const GlaLaunch&, hipStream_t) { return hipErrorNotSupported; }
hipError_t launch_gla_bwd(const GlaLaunch&, hipStream_t) { return hipErrorNotSupported; }
}  // namespace clr
