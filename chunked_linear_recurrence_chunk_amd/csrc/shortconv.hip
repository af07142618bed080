// shortconv.hip -- causal depthwise short convolution with a boundary state,
// forward and backward (the local-convolution boundary state that the
// StateFlow paper, Sec. 1 and Sec. 3.3, hands from one sequence chunk to the
// next next to the recurrent state).
//
// Per batch b, channel c and token t of a chunk:
//     xe = [state_in ; x]                      (W - 1 carried rows first)
//     z_t = bias_c + sum_j w[c][j] xe[t + j],  y_t = act(z_t)
//     state_out = the last W - 1 rows of xe.
// The work is element-wise and HBM-bound: each thread owns a few channels
// (8 in the forward, 4 in the backward, which keeps more rows per thread) over
// a tile of TT tokens and issues every row load of its tile (plus the W - 1
// halo rows) before computing; a wave reads or writes 256 - 1024 contiguous
// bytes of a token row per instruction.
#include <hip/hip_runtime.h>

#include "clr_device.h"
#include "clr_launch.h"
#include "clr_conv.h"

namespace clr {
namespace {

// NV consecutive elements of one token row, as loaded (NV * sizeof(E) bytes).
template <typename E, int NV> struct RowV {
    static constexpr int NW = NV * (int)sizeof(E) / 4;  // 32-bit words
    unsigned u[NW];
};
template <typename E, int NV>
__device__ __forceinline__ RowV<E, NV> ld_row(const E* p) {
    RowV<E, NV> r;
    if constexpr (RowV<E, NV>::NW == 2) {
        const uint2 v = *(const uint2*)p;
        r.u[0] = v.x, r.u[1] = v.y;
    } else {
#pragma unroll
        for (int k = 0; k < RowV<E, NV>::NW / 4; ++k) {
            const uint4 v = ((const uint4*)p)[k];
            r.u[4 * k] = v.x, r.u[4 * k + 1] = v.y, r.u[4 * k + 2] = v.z, r.u[4 * k + 3] = v.w;
        }
    }
    return r;
}
template <typename E, int NV>
__device__ __forceinline__ RowV<E, NV> zero_row() {
    RowV<E, NV> r;
#pragma unroll
    for (int k = 0; k < RowV<E, NV>::NW; ++k) r.u[k] = 0u;
    return r;
}
template <typename E, int NV>
__device__ __forceinline__ void st_row(E* p, const RowV<E, NV>& r) {
    if constexpr (RowV<E, NV>::NW == 2) {
        *(uint2*)p = uint2{r.u[0], r.u[1]};
    } else {
#pragma unroll
        for (int k = 0; k < RowV<E, NV>::NW / 4; ++k)
            ((uint4*)p)[k] = uint4{r.u[4 * k], r.u[4 * k + 1], r.u[4 * k + 2], r.u[4 * k + 3]};
    }
}
template <int NV>
__device__ __forceinline__ float elem(const RowV<bf16, NV>& r, int i) {
    const unsigned w = r.u[i >> 1];
    return __uint_as_float((i & 1) ? (w & 0xffff0000u) : (w << 16));
}
template <int NV>
__device__ __forceinline__ float elem(const RowV<float, NV>& r, int i) {
    return __uint_as_float(r.u[i]);
}
// store NV floats as E (bf16: round to nearest even)
template <typename E, int NV>
__device__ __forceinline__ void st_vals(E* p, const float* v) {
    RowV<E, NV> r;
    if constexpr (sizeof(E) == 2) {
#pragma unroll
        for (int k = 0; k < NV / 2; ++k) {
            const bf16 lo = (bf16)v[2 * k], hi = (bf16)v[2 * k + 1];
            r.u[k] = (unsigned)__builtin_bit_cast(unsigned short, lo) |
                     ((unsigned)__builtin_bit_cast(unsigned short, hi) << 16);
        }
    } else {
#pragma unroll
        for (int k = 0; k < NV; ++k) r.u[k] = __float_as_uint(v[k]);
    }
    st_row<E, NV>(p, r);
}

// SiLU and its derivative with the hardware reciprocal (about 1 ulp) instead
// of an IEEE division: the division sequence alone would make these
// element-wise kernels VALU-bound.  exp(-z) = inf for very negative z gives
// s = 0, the correct limit.
template <int ACT> __device__ __forceinline__ float act_f(float z) {
    if constexpr (ACT == 0) return z;
    else return z * __builtin_amdgcn_rcpf(1.f + __expf(-z));
}
template <int ACT> __device__ __forceinline__ float act_d(float z) {
    if constexpr (ACT == 0) return 1.f;
    else {
        const float s = __builtin_amdgcn_rcpf(1.f + __expf(-z));
        return s * (1.f + z * (1.f - s));
    }
}

// Row of token t (channels c0 .. c0 + NV - 1) of xe: x for 0 <= t < T, the carried
// state for -(W-1) <= t < 0 (zero when absent), zero past the chunk.
// The load is unconditional (from a selected, always valid address) so that
// a tile's row loads issue back to back without branches between them.
template <typename E, int W, int NV>
__device__ __forceinline__ RowV<E, NV> xe_row(const ConvArgs<E>& a, int b, int t, int c0) {
    const bool in_x = t >= 0 && t < a.T, in_s = t < 0 && a.state_in != nullptr;
    const E* px = a.x + ((size_t)b * a.T + (in_x ? t : 0)) * a.C + c0;
    const E* ps = in_s ? a.state_in + ((size_t)b * (W - 1) + (W - 1 + t)) * a.C + c0 : px;
    RowV<E, NV> r = ld_row<E, NV>(in_x ? px : ps);
    if (!in_x && !in_s) r = zero_row<E, NV>();
    return r;
}

// The taps and bias of this work-group's channels [cb0, cb0 + 128 NV), staged
// through LDS with coalesced loads (w is [C][W] row-major, so the block's taps
// are one contiguous run), then read per thread into registers.
// Work-groups of more than 128 threads stage with the first 128; thread
// threadIdx.x % 128 owns channels NV * (threadIdx.x % 128) of the block.
template <int W, int NV>
__device__ __forceinline__ void load_taps(const float* __restrict__ wg, const float* __restrict__ bg, int C,
                                          float (&w)[W][NV], float (&bias)[NV]) {
    __shared__ __align__(16) float sw[128 * NV * W], sb[128 * NV];
    const int cb0 = blockIdx.x * 128 * NV, nch = min(128 * NV, C - cb0);  // nch: a multiple of 8
    const int tx = threadIdx.x & 127;
    if (threadIdx.x < 128) {
    // float4 loads with compile-time trip counts, all issued before the first
    // wait (a runtime-bounded loop would wait for each load in turn)
    constexpr int NW4 = NV * W / 4, NB4 = NV / 4;
    float4 tw[NW4], tb[NB4];
    const float4* w4 = (const float4*)(wg + (size_t)cb0 * W);
#pragma unroll
    for (int k = 0; k < NW4; ++k) {
        const int e = threadIdx.x + 128 * k;
        tw[k] = e < nch * W / 4 ? w4[e] : float4{0.f, 0.f, 0.f, 0.f};
    }
#pragma unroll
    for (int k = 0; k < NB4; ++k) {
        const int e = threadIdx.x + 128 * k;
        tb[k] = (bg && e < nch / 4) ? ((const float4*)(bg + cb0))[e] : float4{0.f, 0.f, 0.f, 0.f};
    }
#pragma unroll
    for (int k = 0; k < NW4; ++k) ((float4*)sw)[threadIdx.x + 128 * k] = tw[k];
#pragma unroll
    for (int k = 0; k < NB4; ++k) ((float4*)sb)[threadIdx.x + 128 * k] = tb[k];
    }
    __syncthreads();
    const int l0 = tx * NV;
#pragma unroll
    for (int i = 0; i < NV; ++i) {
        bias[i] = l0 + i < nch ? sb[l0 + i] : 0.f;
#pragma unroll
        for (int j = 0; j < W; ++j) w[j][i] = l0 + i < nch ? sw[(l0 + i) * W + j] : 0.f;
    }
}

template <typename E, int W, int TT, int ACT>
__global__ __launch_bounds__(128) void shortconv_fwd_kernel(ConvArgs<E> a) {
    constexpr int NV = 4;  // channels per thread
    const int cg = blockIdx.x * 128 + threadIdx.x;
    const bool active = cg * NV < a.C;
    const int c0 = active ? cg * NV : 0, b = blockIdx.z, t0 = blockIdx.y * TT, T = a.T, C = a.C;
    constexpr int NR = TT + W - 1;  // rows: tokens t0 - W + 1 .. t0 + TT - 1
    // the tile's row loads go out first; the taps are staged meanwhile
    RowV<E, NV> raw[NR];
    if (t0 >= W - 1 && t0 + TT <= T) {  // interior tile: every row is in x
        const E* xb = a.x + ((size_t)b * T + (t0 - W + 1)) * C + c0;
#pragma unroll
        for (int r = 0; r < NR; ++r) raw[r] = ld_row<E, NV>(xb + (size_t)r * C);
    } else {
#pragma unroll
        for (int r = 0; r < NR; ++r) raw[r] = xe_row<E, W, NV>(a, b, t0 - W + 1 + r, c0);
    }
    float w[W][NV], bias[NV];
    load_taps<W, NV>(a.w, a.bias, a.C, w, bias);
    if (!active) return;
#pragma unroll
    for (int k = 0; k < TT; ++k) {
        const int t = t0 + k;
        if (t < T) {
            float z[NV];
#pragma unroll
            for (int i = 0; i < NV; ++i) {
                float acc = bias[i];
#pragma unroll
                for (int j = 0; j < W; ++j) acc += w[j][i] * elem(raw[k + j], i);
                z[i] = act_f<ACT>(acc);
            }
            st_vals<E, NV>(a.y + ((size_t)b * T + t) * C + c0, z);
        }
    }
    // state_out = xe rows of tokens T - W + 1 .. T - 1, written by the tile
    // that holds the last token (row r of raw is token t0 - W + 1 + r)
    if (W > 1 && a.state_out && t0 <= T - 1 && T - 1 < t0 + TT) {
#pragma unroll
        for (int r = 0; r < NR; ++r) {
            const int k = r - (T - t0);  // state row of raw row r
            if (k >= 0 && k < W - 1) st_row<E, NV>(a.state_out + ((size_t)b * (W - 1) + k) * C + c0, raw[r]);
        }
    }
}

// Backward.  A work-group is CONV_BWD_TG token groups x 128 threads; thread
// (tg, x) owns NV channels and the contiguous run of tiles
// [(CONV_BWD_TG blockIdx.y + tg) tpg, +tpg) of its batch, walked from the
// top down:
//   dz_t   = dy_t * act'(z_t)
//   dx_s   = [dstate_out row s + W - 1 - T] + sum_j w[j] dz_{s + W - 1 - j}
//            (j ascending, i.e. the latest token first, terms with
//             0 <= token < T only), so that a chunk's dstate_in continues the
//            same left fold in the previous chunk: chunked runs give the
//            unchunked bits
//   dstate_in rows r < W - 1 likewise with dz_{r - j}
//   dw[j] += dz_t xe[t + j],  dbias += dz_t.
// Going down, the W - 1 lowest x rows of a tile's window are the top rows of
// the next window and the dz of its W - 1 lowest tokens are the next tile's
// look-ahead, so both are carried in registers; only the run's first tile
// computes a look-ahead from halo rows.  The token groups' weight / bias sums
// are added in LDS in group order and written as one row of the partial
// table (reduced in a fixed order afterwards).
template <typename E, int W, int TT, int ACT>
__global__ __launch_bounds__(128 * CONV_BWD_TG) void shortconv_bwd_kernel(ConvArgs<E> a) {
    constexpr int NV = CONV_BWD_NV, TG = CONV_BWD_TG;  // channels per thread, token groups
    static_assert(NV == 4, "partial rows are stored as one float4 per tap");
    __shared__ __align__(16) float red[TG][W + 1][128 * NV];
    float w[W][NV], bias[NV];
    load_taps<W, NV>(a.w, a.bias, a.C, w, bias);
    const int tx = threadIdx.x & 127, tg = threadIdx.x >> 7;
    const int cg = blockIdx.x * 128 + tx;
    const bool active = cg * NV < a.C;
    const int c0 = active ? cg * NV : 0, b = blockIdx.z, T = a.T, C = a.C;
    const int ntiles = (T + TT - 1) / TT;
    const int k_lo = (TG * blockIdx.y + tg) * a.tpg, k_hi = min(k_lo + a.tpg, ntiles);
    float dwp[W][NV], dbp[NV];
#pragma unroll
    for (int i = 0; i < NV; ++i) {
        dbp[i] = 0.f;
#pragma unroll
        for (int j = 0; j < W; ++j) dwp[j][i] = 0.f;
    }
    // xw[r]: xe row of token t0 - W + 1 + r (window r < TT + W - 1; the last
    // W - 1 slots are used only for the first tile's look-ahead)
    constexpr int NXW = TT + W - 1, NX = NXW + W - 1;
    RowV<E, NV> xw[NX], dyc[TT];
    float dz[TT + W - 1][NV];  // dz of tokens t0 + m (m >= TT: look-ahead)
    auto dy_row = [&](int t) {
        RowV<E, NV> r = ld_row<E, NV>(a.dy + ((size_t)b * T + (t < T ? t : T - 1)) * C + c0);
        if (t >= T) r = zero_row<E, NV>();
        return r;
    };
    auto dz_of = [&](int t, int r0, float* out, const RowV<E, NV>& dyr) {
        // z of token t from window rows r0 .. r0 + W - 1
#pragma unroll
        for (int i = 0; i < NV; ++i) {
            float z = bias[i];
#pragma unroll
            for (int j = 0; j < W; ++j) z += w[j][i] * elem(xw[r0 + j], i);
            out[i] = t < T ? elem(dyr, i) * act_d<ACT>(z) : 0.f;
        }
    };
    if (active && k_lo < k_hi) {
        // first (top) tile of the run: its window, dy rows and the look-ahead
        int t0 = (k_hi - 1) * TT;
#pragma unroll
        for (int r = 0; r < NX; ++r) xw[r] = xe_row<E, W, NV>(a, b, t0 - W + 1 + r, c0);
#pragma unroll
        for (int m = 0; m < TT; ++m) dyc[m] = dy_row(t0 + m);
        {
            RowV<E, NV> dya[W > 1 ? W - 1 : 1];
#pragma unroll
            for (int m = 0; m < W - 1; ++m) dya[m] = dy_row(t0 + TT + m);
#pragma unroll
            for (int m = 0; m < W - 1; ++m) dz_of(t0 + TT + m, TT + m, dz[TT + m], dya[m]);
        }
        for (int k = k_hi - 1; k >= k_lo; --k) {
            t0 = k * TT;
#pragma unroll
            for (int m = 0; m < TT; ++m) dz_of(t0 + m, m, dz[m], dyc[m]);
            // weight and bias gradients over this tile's tokens
#pragma unroll
            for (int m = 0; m < TT; ++m)
                if (t0 + m < T) {
#pragma unroll
                    for (int i = 0; i < NV; ++i) {
                        dbp[i] += dz[m][i];
#pragma unroll
                        for (int j = 0; j < W; ++j) dwp[j][i] += dz[m][i] * elem(xw[m + j], i);
                    }
                }
            // dx of the tile's tokens
#pragma unroll
            for (int kk = 0; kk < TT; ++kk) {
                const int s = t0 + kk;
                if (s < T) {
                    float acc[NV];
                    const int so = s + W - 1 - T;  // state_out row fed by token s
                    if (so >= 0 && a.dstate_out) {
                        const RowV<float, NV> d = ld_row<float, NV>(a.dstate_out + ((size_t)b * (W - 1) + so) * C + c0);
#pragma unroll
                        for (int i = 0; i < NV; ++i) acc[i] = elem(d, i);
                    } else {
#pragma unroll
                        for (int i = 0; i < NV; ++i) acc[i] = 0.f;
                    }
#pragma unroll
                    for (int j = 0; j < W; ++j) {
                        const int m = kk + W - 1 - j;  // token s + W - 1 - j
                        if (t0 + m < T) {
#pragma unroll
                            for (int i = 0; i < NV; ++i) acc[i] += w[j][i] * dz[m][i];
                        }
                    }
                    st_vals<E, NV>(a.dx + ((size_t)b * T + s) * C + c0, acc);
                }
            }
            // gradient of the carried state (xe rows 0 .. W - 2), from tile 0
            if (W > 1 && k == 0) {
#pragma unroll
                for (int r = 0; r < W - 1; ++r) {
                    float acc[NV];
                    if (r >= T && a.dstate_out) {
                        const RowV<float, NV> d = ld_row<float, NV>(a.dstate_out + ((size_t)b * (W - 1) + (r - T)) * C + c0);
#pragma unroll
                        for (int i = 0; i < NV; ++i) acc[i] = elem(d, i);
                    } else {
#pragma unroll
                        for (int i = 0; i < NV; ++i) acc[i] = 0.f;
                    }
#pragma unroll
                    for (int j = 0; j < W; ++j) {
                        const int m = r - j;  // token r - j
                        if (m >= 0 && m < T) {
#pragma unroll
                            for (int i = 0; i < NV; ++i) acc[i] += w[j][i] * dz[m][i];
                        }
                    }
                    st_vals<float, NV>(a.dstate_in + ((size_t)b * (W - 1) + r) * C + c0, acc);
                }
            }
            if (k > k_lo) {  // slide down one tile: carry, then the next tile's new rows
#pragma unroll
                for (int r = 0; r < W - 1; ++r) xw[TT + r] = xw[r];
#pragma unroll
                for (int m = 0; m < W - 1; ++m)
#pragma unroll
                    for (int i = 0; i < NV; ++i) dz[TT + m][i] = dz[m][i];
#pragma unroll
                for (int r = 0; r < TT; ++r) xw[r] = xe_row<E, W, NV>(a, b, t0 - TT - W + 1 + r, c0);
#pragma unroll
                for (int m = 0; m < TT; ++m) dyc[m] = dy_row(t0 - TT + m);
            }
        }
    }
    // the token groups' sums, added in group order; partial row
    // p = b * gridDim.y + blockIdx.y: [W + 1][C] (taps, then bias)
#pragma unroll
    for (int j = 0; j < W; ++j) *(float4*)&red[tg][j][tx * NV] = float4{dwp[j][0], dwp[j][1], dwp[j][2], dwp[j][3]};
    *(float4*)&red[tg][W][tx * NV] = float4{dbp[0], dbp[1], dbp[2], dbp[3]};
    __syncthreads();
    if (tg != 0 || !active) return;
    float* part = a.part + ((size_t)b * gridDim.y + blockIdx.y) * C * (W + 1) + c0;
#pragma unroll
    for (int j = 0; j <= W; ++j) {
        float4 v = *(const float4*)&red[0][j][tx * NV];
#pragma unroll
        for (int q = 1; q < TG; ++q) {
            const float4 u = *(const float4*)&red[q][j][tx * NV];
            v = float4{v.x + u.x, v.y + u.y, v.z + u.z, v.w + u.w};
        }
        *(float4*)(part + (size_t)j * C) = v;
    }
}

// dw[c][j] (= or +=) the sum over the P partial rows, likewise dbias.  Four
// lanes share one output: lane q sums rows q, q + 4, ... in order, then the
// four sums are added in the order q = 0..3 (deterministic).
__global__ __launch_bounds__(256) void shortconv_reduce_kernel(const float* part, int P, int C, int W, float* dw,
                                                               float* dbias, int accumulate) {
    __shared__ float red[4][64];
    const int n = C * (W + 1);
    const int el = threadIdx.x & 63, q = threadIdx.x >> 6, e = blockIdx.x * 64 + el;
    float s = 0.f;
    if (e < n)
        for (int p = q; p < P; p += 4) s += part[(size_t)p * n + e];
    red[q][el] = s;
    __syncthreads();
    if (q != 0 || e >= n) return;
    s = ((red[0][el] + red[1][el]) + red[2][el]) + red[3][el];
    const int j = e / C, c = e % C;  // tap-major partial layout [W + 1][C]
    if (j < W) {
        float* o = dw + (size_t)c * W + j;
        *o = accumulate ? *o + s : s;
    } else if (dbias) {
        dbias[c] = accumulate ? dbias[c] + s : s;
    }
}

template <typename E, int W>
hipError_t fwd_t(const ConvArgs<E>& a, hipStream_t st) {
    constexpr int TT = sizeof(E) == 2 ? 16 : 8;
    const dim3 grid((a.C / 4 + 127) / 128, (a.T + TT - 1) / TT, a.B);
    if (a.act)
        launch("shortconv_fwd", shortconv_fwd_kernel<E, W, TT, 1>, grid, dim3(128), st, a);
    else
        launch("shortconv_fwd", shortconv_fwd_kernel<E, W, TT, 0>, grid, dim3(128), st, a);
    return hipGetLastError();
}

template <typename E, int W>
hipError_t bwd_t(const ConvArgs<E>& a, int accumulate, hipStream_t st) {
    constexpr int TT = CONV_BWD_TT;
    int tpg;
    const int groups = conv_bwd_tile_groups(a.B, a.T, a.C, TT, &tpg);
    ConvArgs<E> ag = a;
    ag.tpg = tpg;
    const dim3 grid((a.C / CONV_BWD_NV + 127) / 128, groups, a.B);
    if (a.act)
        launch("shortconv_bwd", shortconv_bwd_kernel<E, W, TT, 1>, grid, dim3(128 * CONV_BWD_TG), st, ag);
    else
        launch("shortconv_bwd", shortconv_bwd_kernel<E, W, TT, 0>, grid, dim3(128 * CONV_BWD_TG), st, ag);
    const int P = a.B * (int)grid.y, n = a.C * (W + 1);
    launch("shortconv_reduce", shortconv_reduce_kernel, dim3((n + 63) / 64), dim3(256), st, (const float*)a.part, P,
           a.C, W, a.dw, a.dbias, accumulate);
    return hipGetLastError();
}

}  // namespace

template <typename E>
hipError_t launch_shortconv_fwd(const ConvArgs<E>& a, hipStream_t st) {
    switch (a.W) {
        case 1: return fwd_t<E, 1>(a, st);
        case 2: return fwd_t<E, 2>(a, st);
        case 3: return fwd_t<E, 3>(a, st);
        case 4: return fwd_t<E, 4>(a, st);
    }
    return hipErrorInvalidValue;
}
template <typename E>
hipError_t launch_shortconv_bwd(const ConvArgs<E>& a, int accumulate, hipStream_t st) {
    switch (a.W) {
        case 1: return bwd_t<E, 1>(a, accumulate, st);
        case 2: return bwd_t<E, 2>(a, accumulate, st);
        case 3: return bwd_t<E, 3>(a, accumulate, st);
        case 4: return bwd_t<E, 4>(a, accumulate, st);
    }
    return hipErrorInvalidValue;
}
template hipError_t launch_shortconv_fwd<bf16>(const ConvArgs<bf16>&, hipStream_t);
template hipError_t launch_shortconv_fwd<float>(const ConvArgs<float>&, hipStream_t);
template hipError_t launch_shortconv_bwd<bf16>(const ConvArgs<bf16>&, int, hipStream_t);
template hipError_t launch_shortconv_bwd<float>(const ConvArgs<float>&, int, hipStream_t);

}  // namespace clr
