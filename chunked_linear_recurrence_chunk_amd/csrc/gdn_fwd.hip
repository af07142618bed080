// gdn_fwd.hip -- Gated DeltaNet chunk forward: launch sequence prep -> scan -> out
// (the Pre / ST / Out split of the StateFlow paper, Sec. 2.2, Eq. 2).
#include "gdn_kernels.h"

namespace clr {

// ---------------------------------------------------------------------------
// Host-side launchers
// ---------------------------------------------------------------------------
// The three stages over blocks [n0, n1) of every head.
template <typename E, int DK, int DV>
struct GdnFwdStages {
    const GdnLaunch& L;
    void prep(int n0, int n1, hipStream_t st) const {
        GdnPrepArgs<E> pa{(const E*)L.k, (const E*)L.v, (const E*)L.g, (const E*)L.beta, L.T, L.H, L.NC,
                          L.ws.gam, (E*)L.ws.W, (E*)L.ws.KhT, (float*)L.ws.UtT, L.ws.eg};
        pa.n0 = n0;
        launch("gdn_prep", gdn_prep_kernel<E, DK, DV>, dim3(n1 - n0, L.H, L.B), dim3(512), st, pa);
    }
    void scan(int n0, int n1, const float* S_in, float* S_out, hipStream_t st) const {
        GdnScanArgs<E> sa{L.ws.eg, (const E*)L.ws.W, (const E*)L.ws.KhT, (const E*)L.ws.UtT, S_in, S_out,
                          (E*)L.ws.hT, L.saved_U ? L.saved_U : L.ws.UT, L.H, L.NC, L.B * L.H};
        sa.hN = (E*)L.saved_h;
        sa.n0 = n0;
        sa.n1 = n1;
        if (scan_bv() == 32 && DV % 32 == 0) {
            // two value slices per work-group, sharing their W and K^T stream
            constexpr int NP = scan_np_fast<2>;
            launch("gdn_scan_fwd", gdn_scan_fwd_kernel<E, DK, DV, false, false, NP, 2>,
                   dim3(scan_grid(DV / 32, L.B * L.H)), dim3(scan_threads<NP, 2>), st, sa);
        } else {
            constexpr int NP = scan_np_fast<1>;
            launch("gdn_scan_fwd", gdn_scan_fwd_kernel<E, DK, DV, false, false, NP>,
                   dim3(scan_grid(DV / 16, L.B * L.H)), dim3(scan_threads<NP, 1>), st, sa);
        }
    }
    void out(int n0, int n1, hipStream_t st) const {
        GdnOutArgs<E> oa{(const E*)L.q, (const E*)L.k, L.ws.gam, (const E*)L.ws.hT,
                         (const E*)(L.saved_U ? L.saved_U : L.ws.UT), (E*)L.o, L.T, L.H, L.NC};
        oa.n0 = n0;
        launch("gdn_out", gdn_out_kernel<E, DK, DV>, dim3(n1 - n0, L.H, L.B), dim3(256), st, oa);
    }
};

// First block of the second part of a split forward, or 0 for no split.  The
// state scan runs on B*H*dv/16 work-groups, fewer than the CUs at small
// batch, so the block-parallel stages of one part can run beside the scan of
// the other (StateFlow, Sec. 3.4.2 "Split and Overlap", forward wavefront
// Pre(1) -> (ST(1) || Pre(2)) -> (ST(2) || Out(1)) -> Out(2)).  Each part
// keeps at least 8 blocks.
inline int fwd_split_block(const GdnLaunch& L) {
    const int pm = fwd_split_permille();
    if (pm <= 0 || L.no_split || !L.o || L.NC < 16) return 0;
    int n1 = (int)(((long long)L.NC * pm + 500) / 1000);
    if (n1 < 8) n1 = 8;
    if (n1 > L.NC - 8) n1 = L.NC - 8;
    return n1;
}

template <typename E, int DK, int DV>
hipError_t launch_gdn_fwd_t(const GdnLaunch& L, hipStream_t st) {
    const GdnFwdStages<E, DK, DV> f{L};
    const int n1 = fwd_split_block(L);
    if (n1 > 0) {
        AuxGuard aux(st);
        if (aux.stream) {
            // main stream: Pre(1), ST(1), [Pre(2) done] ST(2), Out(2), [Out(1) done]
            // aux stream:  [Pre(1) done] Pre(2), [ST(1) done] Out(1)
            hipStream_t s2 = aux.stream;
            hipEvent_t* ev = aux.ev;
            const int NC = L.NC;
            f.prep(0, n1, st);
            hipEventRecord(ev[0], st);
            f.scan(0, n1, L.S_in, L.ws.Smid, st);
            hipEventRecord(ev[1], st);
            hipStreamWaitEvent(s2, ev[0], 0);
            f.prep(n1, NC, s2);
            hipEventRecord(ev[2], s2);
            hipStreamWaitEvent(st, ev[2], 0);
            f.scan(n1, NC, L.ws.Smid, L.S_out, st);
            hipStreamWaitEvent(s2, ev[1], 0);
            f.out(0, n1, s2);
            hipEventRecord(ev[3], s2);
            f.out(n1, NC, st);
            hipStreamWaitEvent(st, ev[3], 0);
            return hipGetLastError();
        }
    }
    f.prep(0, L.NC, st);
    f.scan(0, L.NC, L.S_in, L.S_out, st);
    if (L.o) f.out(0, L.NC, st);
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
