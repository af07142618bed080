// gla.hip -- Gated Linear Attention (per-key-channel decay, no delta term)
// Kernels: gla_kernels.h.  This file holds the launch sequences.
#include "gla_kernels.h"

namespace clr {

// ---------------------------------------------------------------------------
// Host-side launchers
// ---------------------------------------------------------------------------
template <typename E, int DK, int DV, bool SG>
hipError_t launch_gla_fwd_t(const GlaLaunch& L, hipStream_t st) {
    const dim3 gblk(L.NC, L.H, L.B);
    const GlaWs& ws = L.ws;
    using SL = GlaSlices<E, DK, DV>;
    GlaPrepArgs<E> pa{(const E*)L.q, (const E*)L.k, (const E*)L.g, L.T, L.H, L.NC, ws.eC, (E*)ws.KhT, nullptr, nullptr};
    pa.range = ws.range;
    launch(SG ? "m2_prep" : "gla_prep", gla_prep_kernel<E, DK, false, SG>, gblk, dim3(256), st, pa);
    GlaScanArgs<E> sa{ws.eC, (const E*)ws.KhT, (const E*)L.v, L.S_in, L.S_out, (E*)ws.hT, L.T, L.H, L.NC, L.B * L.H};
    const dim3 sgrid(scan_grid(SL::NG, L.B * L.H));
    // saved activations: the out kernel stores the states once more, in the
    // block adjoints' layout; without an output the scan does
    if (L.saved_h && !L.o) {
        sa.hN = (E*)L.saved_h;
        launch(SG ? "m2_scan_fwd_save" : "gla_scan_fwd_save", gla_scan_fwd_kernel<E, DK, DV, false, true>, sgrid, dim3(SL::THREADS), st, sa);
    } else {
        launch(SG ? "m2_scan_fwd" : "gla_scan_fwd", gla_scan_fwd_kernel<E, DK, DV, false>, sgrid, dim3(SL::THREADS), st, sa);
    }
    if (L.o) {
        GlaOutArgs<E> oa{(const E*)L.q, (const E*)L.k, (const E*)L.v, (const E*)L.g, (const E*)ws.hT, (E*)L.o, L.T, L.H, L.NC};
        if (L.saved_h) {
            oa.hN = (E*)L.saved_h;
            launch(SG ? "m2_out_save" : "gla_out_save", gla_out_kernel<E, DK, DV, SG, true>, gblk, dim3(512), st, oa);
        } else {
            launch(SG ? "m2_out" : "gla_out", gla_out_kernel<E, DK, DV, SG>, gblk, dim3(512), st, oa);
        }
    }
    return hipGetLastError();
}

template <typename E, int DK, int DV, bool SG>
hipError_t launch_gla_bwd_t(const GlaLaunch& L, hipStream_t st) {
    const dim3 gblk(L.NC, L.H, L.B);
    const GlaWs& ws = L.ws;
    using SL = GlaSlices<E, DK, DV>;
    // with saved states the forward recompute (and the decayed keys it reads) drops out
    const bool saved = L.saved_h != nullptr;
    GlaPrepArgs<E> pa{(const E*)L.q, (const E*)L.k, (const E*)L.g, L.T, L.H, L.NC,
                      ws.eC, saved ? nullptr : (E*)ws.KhT, (E*)ws.QgT, (E*)ws.Kh};
    pa.range = ws.range;
    launch(SG ? "m2_prep_bwd" : "gla_prep_bwd", gla_prep_kernel<E, DK, true, SG>, gblk, dim3(256), st, pa);
    if (!saved) {
        GlaScanArgs<E> sa{ws.eC, (const E*)ws.KhT, (const E*)L.v, L.S_in, nullptr, (E*)ws.hT, L.T, L.H, L.NC, L.B * L.H};
        launch(SG ? "m2_scan_fwd_rec" : "gla_scan_fwd_rec", gla_scan_fwd_kernel<E, DK, DV, true>, dim3(scan_grid(SL::NG, L.B * L.H)), dim3(SL::THREADS), st, sa);
    }
    GlaScanBwdArgs<E> sb{ws.eC, (const E*)ws.Kh, (const E*)ws.QgT, (const E*)L.dO, L.dS_out, L.dS_in,
                         (E*)ws.dh, (E*)ws.dVs, L.T, L.H, L.NC, L.B * L.H};
    launch(SG ? "m2_scan_bwd" : "gla_scan_bwd", gla_scan_bwd_kernel<E, DK, DV>, dim3(scan_grid(SL::NG, L.B * L.H)), dim3(SL::THREADS), st, sb);
    GlaIntraArgs<E> ia{(const E*)L.q, (const E*)L.k, (const E*)L.v, (const E*)L.dO, (const E*)L.g, (const E*)(saved ? L.saved_h : ws.hT),
                       (const E*)ws.dh, (const E*)ws.dVs, (E*)L.dq, (E*)L.dk_, (E*)L.dv_, (E*)L.dg, L.T, L.H, L.NC};
    launch(SG ? "m2_bwd_intra" : "gla_bwd_intra", gla_bwd_intra_kernel<E, DK, DV, SG>, gblk, dim3(512), st, ia);
    return hipGetLastError();
}

hipError_t launch_gla_fwd(const GlaLaunch& L, hipStream_t st) {
#define CLR_CASE(E, DK, DV) \
    if (L.dk == DK && L.dv == DV) \
        return L.scalar_gate ? launch_gla_fwd_t<E, DK, DV, true>(L, st) : launch_gla_fwd_t<E, DK, DV, false>(L, st);
    if (L.bf16) {
        CLR_FOR_GLA_SHAPES(bf16)
    } else {
        CLR_FOR_GLA_SHAPES(float)
    }
#undef CLR_CASE
    return hipErrorInvalidValue;
}

hipError_t launch_gla_bwd(const GlaLaunch& L, hipStream_t st) {
#define CLR_CASE(E, DK, DV) \
    if (L.dk == DK && L.dv == DV) \
        return L.scalar_gate ? launch_gla_bwd_t<E, DK, DV, true>(L, st) : launch_gla_bwd_t<E, DK, DV, false>(L, st);
    if (L.bf16) {
        CLR_FOR_GLA_SHAPES(bf16)
    } else {
        CLR_FOR_GDN_BWD_SHAPES_F32(float)
    }
#undef CLR_CASE
    return hipErrorInvalidValue;
}

}  // namespace clr
