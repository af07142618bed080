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
};

// Channels per thread and tokens per tile of the backward (the tile's rows
// stay in registers).
constexpr int CONV_BWD_NV = 4, CONV_BWD_TT = 8;

// Tile groups per batch of the backward grid: about 512 work-groups of 128
// threads in total, at most one per tile.
inline int conv_bwd_tile_groups(int B, int T, int C, int tt) {
    const int ntiles = (T + tt - 1) / tt;
    const int gx = (C / CONV_BWD_NV + 127) / 128;
    int g = 512 / (gx * B);
    if (g < 1) g = 1;
    if (g > ntiles) g = ntiles;
    return g;
}

template <typename E> hipError_t launch_shortconv_fwd(const ConvArgs<E>& a, hipStream_t st);
template <typename E> hipError_t launch_shortconv_bwd(const ConvArgs<E>& a, int accumulate, hipStream_t st);

}  // namespace clr
