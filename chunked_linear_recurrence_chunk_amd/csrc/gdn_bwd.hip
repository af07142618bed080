// gdn_bwd.hip -- Gated DeltaNet chunk backward on gfx950 (in progress).
#include "clr_kernels.h"

namespace clr {
hipError_t launch_gdn_bwd(const GdnLaunch&, hipStream_t) { return hipErrorNotSupported; }
}  // namespace clr
