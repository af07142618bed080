// clr_conv.h -- short-convolution kernel arguments and launchers (internal).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>

namespace clr {

template <typename E> struct ConvArgs {
    int B, T, C, W, act;
    const E* x;
    const float *w, *bias;
    const E* state_in;
    E *y, *state_out;
    // backward (the state gradients are partial sums: kept in fp32 so that
    // chunked runs continue the unchunked fold exactly)
    const E* dy;
    const float* dstate_out;
    E* dx;
    float* dstate_in;
    float *dw, *dbias;
    float* part;  // [B * tile groups][W + 1][C] partial weight / bias gradients
    int tpg;      // backward: tiles per group (each thread walks one run of tiles)
};

// Backward geometry: 4 channels per thread, 4-token tiles, work-groups of
// CONV_BWD_TG token groups x 128 threads.
constexpr int CONV_BWD_NV = 4, CONV_BWD_TT = 4, CONV_BWD_TG = 4;

// Work-groups per batch along the tokens (grid y) of the backward, and the
// tiles each thread walks (*tpg).  Aims at about 8 waves per CU in total
// (256 CUs); every thread's run of tiles is non-empty except at the very end.
inline int conv_bwd_tile_groups(int B, int T, int C, int tt, int* tpg = nullptr) {
    const int ntiles = (T + tt - 1) / tt;
    const long threads_per_group = (long)B * (C / CONV_BWD_NV);  // one token group across every channel
    long want = (256L * 8 * 64) / (threads_per_group > 0 ? threads_per_group : 1);  // token groups wanted
    if (want < 1) want = 1;
    if (want > ntiles) want = ntiles > 0 ? ntiles : 1;
    const int per = ntiles > 0 ? (int)((ntiles + want - 1) / want) : 1;
    if (tpg) *tpg = per;
    const int groups = ntiles > 0 ? (ntiles + per - 1) / per : 1;  // token groups in total
    return (groups + CONV_BWD_TG - 1) / CONV_BWD_TG;
}

template <typename E> hipError_t launch_shortconv_fwd(const ConvArgs<E>& a, hipStream_t st);
template <typename E> hipError_t launch_shortconv_bwd(const ConvArgs<E>& a, int accumulate, hipStream_t st);

}  // namespace clr
