// gdn_bwd.hip -- Gated DeltaNet chunk backward on gfx950.
// Kernels: gdn_bwd_kernels.h.  This file holds the launch sequence.
#include "gdn_bwd_kernels.h"

namespace clr {

template <typename E, int DK, int DV>
hipError_t launch_gdn_bwd_t(const GdnLaunch& L, hipStream_t st) {
    const dim3 gblk(L.NC, L.H, L.B);
    const GdnWs& ws = L.ws;
    GdnPrepArgs<E> pa{(const E*)L.k, (const E*)L.v, (const E*)L.g, (const E*)L.beta, L.T, L.H, L.NC,
                      ws.gam, (E*)ws.W, (E*)ws.KhT, (float*)ws.UtT, ws.eg};
    pa.TT = (E*)ws.TT;
    pa.q = (const E*)L.q;
    pa.dO = (const E*)L.dO;
    pa.WT = (E*)ws.WT;
    pa.Kh = (E*)ws.Kh;
    pa.dvlT = (E*)ws.dvlT;
    pa.Rt = (E*)ws.Rt;
    const bool saved = L.saved_h != nullptr;
    if (saved) {  // no forward recompute: its operands are not needed
        pa.W = nullptr;
        pa.KhT = nullptr;
        pa.UtT = nullptr;
    }
    launch("gdn_prep_bwd", gdn_prep_kernel<E, DK, DV, true>, gblk, dim3(512), st, pa);
    GdnScanArgs<E> sa{ws.eg, (const E*)ws.W, (const E*)ws.KhT, (const E*)ws.UtT, L.S_in, nullptr,
                      (E*)ws.hT, (E*)ws.UT, L.H, L.NC, L.B * L.H};
    GdnScanBwdArgs<E> sb{ws.eg, (const E*)ws.Kh, (const E*)ws.WT, (const E*)ws.dvlT, ws.Rt,
                         L.dS_out, L.dS_in, (E*)ws.dhT, ws.dUT, L.H, L.NC, L.B * L.H};
    sb.dh_lo = (E*)ws.dhT_lo;
    const int G = (int)scan_grid(DV / 16, L.B * L.H);
    constexpr int NCW = scan_can_split<E, DK>() ? 2 : 1, NP = scan_np_fast<NCW>;
    if (saved)  // the forward's states and U are read below: the reverse scan alone
        launch("gdn_scan_rev", gdn_scan_rev_kernel<E, DK, DV, false, NP, NCW>, dim3(G),
               dim3(scan_threads<NP, NCW>), st, sb);
    else
        launch("gdn_scan_pair", gdn_scan_pair_kernel<E, DK, DV, false, NP, NCW>, dim3(2 * G),
               dim3(scan_threads<NP, NCW>), st, sa, sb, G);
    GdnIntraArgs<E> ia{(const E*)L.q, (const E*)L.k, (const E*)L.v, (const E*)L.beta, (const E*)L.dO,
                       ws.gam, (const E*)(saved ? L.saved_h : ws.hT), (const E*)ws.dhT,
                       (const E*)(saved ? L.saved_U : ws.UT), (const float*)ws.dUT,
                       (const E*)ws.TT,
                       (E*)L.dq, (E*)L.dk_, (E*)L.dv_, (E*)L.dg, (E*)L.dbeta, L.T, L.H, L.NC};
    ia.dh_lo = (const E*)ws.dhT_lo;
    launch("gdn_bwd_intra", gdn_bwd_intra_kernel<E, DK, DV>, gblk, dim3(512), st, ia);
    return hipGetLastError();
}

hipError_t launch_gdn_bwd(const GdnLaunch& L, hipStream_t st) {
#define CLR_CASE(E, DK, DV) \
    if (L.dk == DK && L.dv == DV) return launch_gdn_bwd_t<E, DK, DV>(L, st);
    if (L.bf16) {
        CLR_FOR_GDN_SHAPES(bf16)
    } else {
        CLR_FOR_GDN_BWD_SHAPES_F32(float)
    }
#undef CLR_CASE
    return hipErrorInvalidValue;
}

}  // namespace clr
