// gdn_fwd.hip -- Gated DeltaNet chunk forward: launch sequence prep -> scan -> out
// (the Pre / ST / Out split of the StateFlow paper, Sec. 2.2, Eq. 2).
#include "gdn_kernels.h"

namespace clr {

// ---------------------------------------------------------------------------
// Host-side launchers
// ---------------------------------------------------------------------------
template <typename E, int DK, int DV>
hipError_t launch_gdn_fwd_t(const GdnLaunch& L, hipStream_t st) {
    const dim3 gblk(L.NC, L.H, L.B);
    GdnPrepArgs<E> pa{(const E*)L.k, (const E*)L.v, (const E*)L.g, (const E*)L.beta, L.T, L.H, L.NC,
                      L.ws.gam, (E*)L.ws.W, (E*)L.ws.KhT, (E*)L.ws.UtT};
    launch("gdn_prep", gdn_prep_kernel<E, DK, DV>, gblk, dim3(256), st, pa);
    GdnScanArgs<E> sa{L.ws.gam, (const E*)L.ws.W, (const E*)L.ws.KhT, (const E*)L.ws.UtT, L.S_in, L.S_out,
                      (E*)L.ws.hT, (E*)L.ws.UT, L.H, L.NC, L.B * L.H};
    launch("gdn_scan_fwd", gdn_scan_fwd_kernel<E, DK, DV, false>, dim3(scan_grid(DV / 16, L.B * L.H)), dim3(256), st, sa);
    if (L.o) {
        GdnOutArgs<E> oa{(const E*)L.q, (const E*)L.k, L.ws.gam, (const E*)L.ws.hT, (const E*)L.ws.UT, (E*)L.o,
                         L.T, L.H, L.NC};
        launch("gdn_out", gdn_out_kernel<E, DK, DV>, gblk, dim3(256), st, oa);
    }
    return hipGetLastError();
}

hipError_t launch_gdn_fwd(const GdnLaunch& L, hipStream_t st) {
#define CLR_CASE(E, DK, DV) \
    if (L.dk == DK && L.dv == DV) return launch_gdn_fwd_t<E, DK, DV>(L, st);
    if (L.bf16) {
        CLR_FOR_GDN_SHAPES(bf16)
    } else {
        CLR_FOR_GDN_SHAPES(float)
    }
#undef CLR_CASE
    return hipErrorInvalidValue;
}

}  // namespace clr
