// gla_kernels.h -- GLA (and Mamba-2 member, KDA forward prep) kernels
// (internal; the launch sequences are in gla.hip).
//
// chunk forward and backward on gfx950.
//
// The layer (key-major state S in R^{dk x dv}, gate g_t in R^{dk}, g <= 0):
//   S_t = Diag(exp(g_t)) S_{t-1} + k_t v_t^T,   o_t = S_t^T q_t,
// the "rank-1" (element-wise) gated transition of the StateFlow paper
// ("StateFlow: Sequence Pipeline Parallelism for Long-Context Modeling with
// Linear Recurrence", Sec. 2.1).  Per 64-token block, b = cumsum(g) per
// channel, S0 the state entering the block:
//   O  = (Q * exp(b)) S0 + P V,   P[t][s] = sum_i q_t[i] k_s[i] exp(b_t[i] - b_s[i])  (s <= t)
//   S1 = Diag(exp(b_C)) S0 + (K * exp(b_C - b))^T V
// Following the numerics notes on the GLA paper's page (relative decay in log
// space, 16-token secondary tiles, reciprocal rescaling bounded by e^80 so the
// diagonal tiles can also use dense matrix products), P is formed per pair of
// 16-token tiles (R, S): off-diagonal pairs use the boundary before tile R as
// reference, so both rescaling factors are <= 1 and the product is exact for
// any gates; diagonal pairs use the tile's middle token as reference, exact
// while the decay within half a tile stays within 80 nats per channel (factors
// are clamped at e^80 beyond that, which keeps everything finite).
//
// Kernels:  prep (b, Kh^T; backward also (Q*exp(b))^T and Kh),
//           scan (sequential over blocks: S <- exp(b_C) * S + Kh^T V, saving h_n),
//           out  (parallel over blocks),
//           dscan (reverse: dS <- exp(b_C) * dS + (Q*exp(b))^T dO, saving dh_n and Kh dh_n),
//           intra (parallel over blocks: dq, dk, dv, dg by the block adjoints; dg by the
//                  per-channel gate scaling identity
//                  dg_r[i] = sum_{tau >= r}(q dq - k dk)[i] + rowsum(S1 * dh)[i]).
#pragma once

#include "gdn_kernels.h"

namespace clr {

// exp clamped at e^80 (the rescaling bound of the diagonal tiles)
constexpr float DIAG_RANGE = 80.f;
__device__ __forceinline__ float expu(float x) { return __expf(fminf(x, DIAG_RANGE)); }

// Whether the block's gates leave the diagonal tiles' bound: some channel d
// decays by more than DIAG_RANGE nats between a 16-token tile's first token
// and its middle (token 7), or between the middle and its last token, so that
// a rescaling factor of the diagonal pair terms would be clamped.  All
// threads call it (a block-wide OR); bs is the cumulative gate b[t][d] in LDS
// (row pitch PB).
template <int DK, int PB>
__device__ __forceinline__ bool diag_out_of_range(const float* bs) {
    bool out = false;
    for (int i = threadIdx.x; i < 4 * DK; i += blockDim.x) {
        const int R = i / DK, d = i % DK;
        const float b0 = bs[(16 * R) * PB + d], bm = bs[(16 * R + 7) * PB + d], b1 = bs[(16 * R + 15) * PB + d];
        out |= (b0 - bm > DIAG_RANGE) || (bm - b1 > DIAG_RANGE);
    }
    return __syncthreads_or(out);
}

template <typename E> struct GlaPrepArgs {
    const E *q, *k, *g;
    int T, H, NC;
    float* eC;
    E *KhT, *QgT, *Kh;
    int* range = nullptr;  // per block: 1 if the gates leave the diagonal tiles' bound
};
template <typename E> struct GlaScanArgs {
    const float* eC;
    const E *KhT, *v;
    const float* S_in;
    float* S_out;
    E* hT;
    int T, H, NC, BH;
    // saved activations: the state entering each block, also in the tiled
    // [d][v] layout the block adjoints read (forward scan with HN only)
    E* hN = nullptr;
};
template <typename E> struct GlaOutArgs {
    const E *q, *k, *v, *g;
    const E* hT;
    E* o;
    int T, H, NC;
    // saved activations: the states once more, in the block adjoints' tiled
    // [d][v] layout (out kernel with HN only)
    E* hN = nullptr;
};
template <typename E> struct GlaScanBwdArgs {
    const float* eC;
    const E *Kh, *QgT, *dO;
    const float* dS_out;
    float* dS_in;
    E *dh, *dVs;
    int T, H, NC, BH;
};
template <typename E> struct GlaIntraArgs {
    const E *q, *k, *v, *dO, *g;
    const E *h, *dh, *dVs;
    E *dq, *dk, *dv, *dg;
    int T, H, NC;
    // KDA (v is U): dM [.., 64, 64] and dX [.., 64, dk] fp32 per block, beta
    const float *dM = nullptr, *dX = nullptr;
    const E* beta = nullptr;
};

__device__ __forceinline__ f32x4 ld4f(const float* p) { return *(const f32x4*)p; }

// B fragment of a token-major tensor with k = token (t = 32 j + kmap(g, i)),
// n = column c: eight element loads (rows past the sequence end are zero).
template <typename E>
__device__ __forceinline__ Frag<E> ldfrag_tokcol(const E* base, size_t ld, int j, int g, int c, int nvalid) {
    float x[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const int t = 32 * j + (i < 4 ? 4 * g + i : 16 + 4 * g + i - 4);
        x[i] = t < nvalid ? to_f(base[(size_t)t * ld + c]) : 0.f;
    }
    return frag_from_acc<E>(f32x4{x[0], x[1], x[2], x[3]}, f32x4{x[4], x[5], x[6], x[7]});
}

// ---------------------------------------------------------------------------
// Block gate cumsum b[t][d] = sum_{s <= t} g[s][d] (tokens past the end of
// the sequence contribute 0: every caller stages those rows of g as zeros,
// so the reads need no test and go out together), from a row-major g tile in
// LDS (pitch PG) into fp32 LDS (pitch PB).  256 threads take 256 / DK token segments per channel:
// each sums its segment in token order, then adds the totals of the earlier
// segments in order.  The split does not depend on the work-group size, so
// every kernel that forms b gets bit-identical values.  `seg` is 256 floats
// of LDS scratch; all threads of the work-group must call this.
// ---------------------------------------------------------------------------
template <typename E, int DK, int PG, int PB>
__device__ __forceinline__ void gate_cumsum(const E* gs, float* bs, float* seg, int nvalid) {
    constexpr int S = 256 / DK, L = BLK / S;  // segments per channel, tokens per segment
    const int tid = threadIdx.x, d = tid % DK, sg = tid / DK;
    (void)nvalid;  // rows at or past nvalid are zero in gs
    if (tid < 256) {
        float gv[L];
#pragma unroll
        for (int i = 0; i < L; ++i) gv[i] = to_f(gs[(sg * L + i) * PG + d]);
        float run = 0.f;
#pragma unroll
        for (int i = 0; i < L; ++i) {
            const int t = sg * L + i;
            run += gv[i];
            bs[t * PB + d] = run;
        }
        seg[tid] = run;
    }
    __syncthreads();
    if (tid < 256 && sg > 0) {
        float off = 0.f;
        for (int k = 0; k < sg; ++k) off += seg[k * DK + d];
#pragma unroll
        for (int i = 0; i < L; ++i) bs[(sg * L + i) * PB + d] += off;
    }
}

// The gate rows of one block as a [64][DK] tile in registers (staged into LDS
// with store_rows): the per-channel gate g[t][d], or with SG the per-token
// scalar gate of the Mamba-2 member broadcast over the DK channels (the
// scalar-identity transition of the StateFlow paper, Sec. 2.1, Eq. 1).
// Tokens at or past nvalid read as 0 (an identity step).
template <bool SG, typename E, int DK, int NT = 256>
__device__ __forceinline__ RowsRegs<E, BLK, DK, NT> load_gate(const E* g, size_t tok0, int h, int H, int nvalid) {
    if constexpr (!SG) {
        const size_t ldk = (size_t)H * DK;
        return load_rows<E, BLK, DK, NT>(g + tok0 * ldk + (size_t)h * DK, ldk, nvalid);
    } else {
        using X = RowsRegs<E, BLK, DK, NT>;
        X x;
#pragma unroll
        for (int j = 0; j < X::N; ++j) {
            const int idx = threadIdx.x + NT * j, t = idx / X::PER_ROW;
            const E gv = (idx < X::UNITS && t < nvalid) ? g[(tok0 + t) * H + h] : from_f<E>(0.f);
            union {
                uint4 u;
                E e[X::VEC];
            } c;
#pragma unroll
            for (int v = 0; v < X::VEC; ++v) c.e[v] = gv;
            x.u[j] = c.u;
        }
        return x;
    }
}

// A fragment of row `row` of a row-major LDS tile X (k = column c = col +
// kmap(g, i)), element c scaled by exp(sgn * (brow[c] - ref[c])).
template <typename E>
__device__ __forceinline__ Frag<E> frag_row_decay(const E* X, int PX, int row, int col, const float* brow,
                                                  const float* ref, float sgn) {
    const int g = (threadIdx.x & 63) >> 4;
    const int c0 = col + 4 * g, c1 = col + 16 + 4 * g;
    const f32x4 d0 = ld4f(brow + c0) - ld4f(ref + c0), d1 = ld4f(brow + c1) - ld4f(ref + c1);
    f32x4 s0, s1;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        s0[i] = expu(sgn * d0[i]);
        s1[i] = expu(sgn * d1[i]);
    }
    return ldfrag_scaled(X + row * PX + col + 4 * g, s0, s1);
}
// The same fragment as a split pair (the decayed keys of the KDA scans, whose
// rounding would add components to a state that decays slowly).
template <typename E>
__device__ __forceinline__ Frag2<E> frag_row_decay2(const E* X, int PX, int row, int col, const float* brow,
                                                    const float* ref, float sgn) {
    const int g = (threadIdx.x & 63) >> 4;
    const int c0 = col + 4 * g, c1 = col + 16 + 4 * g;
    const f32x4 d0 = ld4f(brow + c0) - ld4f(ref + c0), d1 = ld4f(brow + c1) - ld4f(ref + c1);
    f32x4 s0, s1;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        s0[i] = expu(sgn * d0[i]);
        s1[i] = expu(sgn * d1[i]);
    }
    const E* p = X + row * PX + col + 4 * g;
    return split8<E>(ld4(p) * s0, ld4(p + 16) * s1);
}

// A fragment of X^T (m = feature m0 + r, k = token s = k0 + kmap(g, i)) from
// a row-major LDS tile X[s][feature], element scaled by
// exp(sgn * (b[s][m] - ref[m])) and zero for tokens outside [klo, khi).
// The b values are read four at a time (k is always inside the 64-token
// tile, so every read is in bounds); the empty asm keeps the compiler from
// moving each read under its range test, which serialises them, and outside
// [klo, khi) the exponent is -inf, so the factor is exactly 0.  klo and khi
// must be the same for every lane of the wave.
template <typename E>
__device__ __forceinline__ void col_decay_scales(const float* bs, int PB, int m, int k0, const float* ref, float sgn,
                                                 int klo, int khi, float (&sc)[8]) {
    const int g = (threadIdx.x & 63) >> 4;
    const float rm = ref[m];
#pragma unroll
    for (int hbl = 0; hbl < 2; ++hbl) {
        // a 16-token half wholly outside [klo, khi) has every factor 0 (the same
        // values the exponentials of -inf give); the range is the wave's, so the
        // test is a scalar branch
        const int kb = k0 + 16 * hbl;
        if (__builtin_amdgcn_readfirstlane((kb + 16 <= klo || kb >= khi) ? 1 : 0)) {
#pragma unroll
            for (int i = 0; i < 4; ++i) sc[4 * hbl + i] = 0.f;
            continue;
        }
        float bv[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) bv[i] = bs[(k0 + 16 * hbl + 4 * g + i) * PB + m];
        asm volatile("" : "+v"(bv[0]), "+v"(bv[1]), "+v"(bv[2]), "+v"(bv[3]));
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int k = k0 + 16 * hbl + 4 * g + i;
            const float y = sgn * (bv[i] - rm);
            sc[4 * hbl + i] = expu((k >= klo && k < khi) ? y : -__builtin_inff());
        }
    }
}
template <typename E>
__device__ __forceinline__ Frag<E> frag_col_decay(const E* X, int PX, const float* bs, int PB, int m0, int k0,
                                                  const float* ref, float sgn, int klo, int khi) {
    const int l = threadIdx.x & 63, r = l & 15;
    Frag<E> x = ldfrag_tr(X, PX, k0, m0, l);
    float sc[8];
    col_decay_scales<E>(bs, PB, m0 + r, k0, ref, sgn, klo, khi, sc);
    if constexpr (sizeof(E) == 2) {
#pragma unroll
        for (int i = 0; i < 8; ++i) x.v[i] = (bf16)((float)x.v[i] * sc[i]);
    } else {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            x.lo[i] *= sc[i];
            x.hi[i] *= sc[4 + i];
        }
    }
    return x;
}
// The same fragment as a split pair.
template <typename E>
__device__ __forceinline__ Frag2<E> frag_col_decay2(const E* X, int PX, const float* bs, int PB, int m0, int k0,
                                                    const float* ref, float sgn, int klo, int khi) {
    const int l = threadIdx.x & 63, r = l & 15;
    const Frag<E> x = ldfrag_tr(X, PX, k0, m0, l);
    float sc[8];
    col_decay_scales<E>(bs, PB, m0 + r, k0, ref, sgn, klo, khi, sc);
    f32x4 a, b;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        if constexpr (sizeof(E) == 2) {
            a[i] = (float)x.v[i] * sc[i];
            b[i] = (float)x.v[4 + i] * sc[4 + i];
        } else {
            a[i] = x.lo[i] * sc[i];
            b[i] = x.hi[i] * sc[4 + i];
        }
    }
    return split8<E>(a, b);
}

// ---------------------------------------------------------------------------
// prep: one work-group per (block, head, batch).  Writes exp(b_C) and the
// tiled Kh^T (backward also the tiled (Q*exp(b))^T and Kh), all from
// row-major LDS tiles staged with every load in flight at once.
// ---------------------------------------------------------------------------
template <typename E, int DK, bool BWD, bool SG>
__global__ __launch_bounds__(256) void gla_prep_kernel(GlaPrepArgs<E> a) {
    const int n = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
    const int tid = threadIdx.x, w = tid >> 6, l = tid & 63;
    const int T = a.T, H = a.H, NC = a.NC;
    const size_t tok0 = (size_t)b * T + (size_t)n * BLK;
    const size_t chunk = ((size_t)b * H + h) * NC + n;
    const int nvalid = min(BLK, T - n * BLK);
    const size_t ldk = (size_t)H * DK;
    constexpr int PK = RP<E, DK>, PB = DK + 4, ND = DK / 16, KK = DK / 32;

    // g is staged in the Q tile's space (Q is stored there once the cumsum is done)
    __shared__ __align__(16) E Ks[BLK * PK], Qs[BLK * PK];
    __shared__ __align__(16) float Bs[BLK * PB];
    __shared__ __align__(16) float zrow[DK];
    __shared__ float seg[256];

    {
        const auto kx = load_rows<E, BLK, DK>(a.k + tok0 * ldk + (size_t)h * DK, ldk, nvalid);
        const auto gx = load_gate<SG, E, DK>(a.g, tok0, h, H, nvalid);
        RowsRegs<E, BLK, DK> qx;
        if constexpr (BWD) qx = load_rows<E, BLK, DK>(a.q + tok0 * ldk + (size_t)h * DK, ldk, nvalid);
        store_rows<E, BLK, DK, PK>(kx, Ks);
        store_rows<E, BLK, DK, PK>(gx, Qs);
        if (tid < DK) zrow[tid] = 0.f;
        __syncthreads();
        gate_cumsum<E, DK, PK, PB>(Qs, Bs, seg, nvalid);
        __syncthreads();
        const bool over = diag_out_of_range<DK, PB>(Bs);
        if (a.range && tid == 0) a.range[chunk] = over ? 1 : 0;
        if constexpr (BWD) {
            store_rows<E, BLK, DK, PK>(qx, Qs);
            __syncthreads();
        }
    }
    const float* bC = Bs + (BLK - 1) * PB;
    if (tid < DK) a.eC[chunk * DK + tid] = __expf(bC[tid]);
    // Kh^T (A: m = d, k = t) fragment (db, j) = B fragment of K * exp(b_C - b)
    // (the backward that reads saved states has no scan to feed: KhT null)
    E* KhT = a.KhT ? a.KhT + chunk * BLK * DK : nullptr;
    E* QgT = BWD ? a.QgT + chunk * BLK * DK : nullptr;
#pragma unroll
    for (int f = w; f < 2 * ND; f += 4) {
        const int db = f >> 1, j = f & 1;
        if (KhT) st_fragT(KhT, f, l, frag_col_decay(Ks, PK, Bs, PB, 16 * db, 32 * j, bC, -1.f, 0, BLK));
        if constexpr (BWD) st_fragT(QgT, f, l, frag_col_decay(Qs, PK, Bs, PB, 16 * db, 32 * j, zrow, 1.f, 0, BLK));
    }
    if constexpr (BWD) {
        // Kh (A: m = t, k = d) fragment (tb, kk)
        E* Kh = a.Kh + chunk * BLK * DK;
#pragma unroll
        for (int f = w; f < 4 * KK; f += 4) {
            const int tb = f / KK, kk = f % KK, t = 16 * tb + (l & 15);
            st_fragT(Kh, f, l, frag_row_decay(Ks, PK, t, 32 * kk, Bs + t * PB, bC, -1.f));
        }
    }
}

// ---------------------------------------------------------------------------
// Scans.  One work-group per (NS value slices of 16, head, batch): NS
// consumer waves each run the recurrence of one slice with its fp32 state
// in accumulator tiles, NPW producer waves stream the block operands into
// an LDS ring (clr_ring.h).  The per-channel decay makes each step
// element-wise plus one product that does not depend on the state.
// A slot holds the tiled block operands shared by the slices, then each
// slice's 64 x 16 rows of V (or dO) row-major (read transposed), then exp(b_C).
// ---------------------------------------------------------------------------
template <typename E, int DK, int DV> struct GlaSlices {
    static constexpr int NS = DV / 16 < 4 ? DV / 16 : 4, NG = DV / 16 / NS, NPW = 4;
    static constexpr int UPF = sizeof(E) == 2 ? 1 : 2, NVU = (int)sizeof(E);  // units per 64 x 16 slice
    static constexpr int LPR = (int)sizeof(E), VEC = 16 / (int)sizeof(E);      // lanes per 16-value row
    static constexpr int THREADS = 64 * (NS + NPW);
};

// Source of unit q (0 .. NVU-1) of the token-major 64 x 16 slice starting at
// `rows` (row stride ld); rows past the sequence end repeat the last valid one
// (its operands there are zero, so the values only have to be finite).
template <typename E, int DV>
__device__ __forceinline__ const void* slice_src(const E* rows, size_t ld, int q, int l, int nvalid) {
    using SL = GlaSlices<E, 16, DV>;
    const int t = q * (64 / SL::LPR) + l / SL::LPR, part = l % SL::LPR;
    const int ts = t < nvalid ? t : nvalid - 1;
    return rows + (size_t)ts * ld + part * SL::VEC;
}

template <typename E, int DK, int DV, bool HNAT, bool HN = false> struct GlaScanGeom : GlaSlices<E, DK, DV> {
    using SL = GlaSlices<E, DK, DV>;
    static constexpr int ND = DK / 16, NKU = 2 * ND * SL::UPF;
    static constexpr int NU = NKU + SL::NS * SL::NVU + 1;  // Kh^T | V slices | exp(b_C)
    static constexpr int SLOT = RingGeom<NU, SL::NPW>::SLOT;
    static constexpr int TILE = HNAT || HN ? state_tile_bytes(DK, sizeof(E)) : 16;  // per consumer wave
    static constexpr int PF = (144 * 1024 - SL::NS * TILE) / SLOT;
    static constexpr int P = PF > 4 ? 4 : (PF < 2 ? 2 : PF);
};

// HNAT: the saved states hT in the tiled [d][v] layout of the block adjoints
// (backward recompute), else in the fragment tiles of the out kernel; HN: the
// latter, and each state once more in the former at hN (saved activations).
template <typename E, int DK, int DV, bool HNAT, bool HN = false>
__global__ __launch_bounds__((GlaSlices<E, DK, DV>::THREADS)) void gla_scan_fwd_kernel(GlaScanArgs<E> a) {
    static_assert(!(HNAT && HN), "one tiled [d][v] store per block");
    using SG = GlaScanGeom<E, DK, DV, HNAT, HN>;
    constexpr int ND = SG::ND, KK = DK / 32, NS = SG::NS, NU = SG::NU, P = SG::P, NKU = SG::NKU, NVU = SG::NVU;
    constexpr int NPW = SG::NPW, UE = UNIT_ELEMS<E>, LE = LANE_ELEMS<E>;
    using G = RingGeom<NU, NPW>;
    __shared__ __align__(16) char ring[P * G::SLOT];
    __shared__ __align__(16) E tiles[NS * SG::TILE / sizeof(E)];
    const int H = a.H, NC = a.NC;
    int b, h, vg;
    if (!scan_coords(SG::NG, a.BH, H, b, h, vg)) return;
    const int w = threadIdx.x >> 6, l = threadIdx.x & 63, r = l & 15, g = l >> 4;
    const size_t bh = (size_t)b * H + h, ldv = (size_t)H * DV;

    if (w >= NS) {  // producers
        const int pid = w - NS;
        auto issue = [&](int n) {
            const size_t c = bh * NC + n;
            const int nvalid = min(BLK, a.T - n * BLK);
            const E* KhT = a.KhT + c * BLK * DK + l * LE;
            const E* vrows = a.v + ((size_t)b * a.T + (size_t)n * BLK) * ldv + (size_t)h * DV + 16 * NS * vg;
            const float* eC = a.eC + c * DK + 4 * min(l, DK / 4 - 1);
            auto src = [&](int u) -> const void* {
                if (u < NKU) return KhT + u * UE;
                if (u < NKU + NS * NVU) {
                    const int q = u - NKU;
                    return slice_src<E, DV>(vrows + 16 * (q / NVU), ldv, q % NVU, l, nvalid);
                }
                return eC;
            };
            ring_issue_units<NU, NPW>(ring + (n % P) * G::SLOT, pid, src);
        };
        const int pre = NC < P - 1 ? NC : P - 1;
        for (int n = 0; n < pre; ++n) issue(n);
        ring_wait<G::NU_MIN>(pre - 1);  // block 0 has landed
        ring_barrier();
        for (int n = 0; n < NC; ++n) {
            if (n + P - 1 < NC) issue(n + P - 1);
            const int last = (n + P - 1 < NC ? n + P - 1 : NC - 1);
            ring_wait<G::NU_MIN>(last - (n + 1));  // block n + 1 has landed
            ring_barrier();
        }
        return;
    }

    // consumer wave w: value slice vb
    const int vb = NS * vg + w, v0 = 16 * vb;
    E* tile = tiles + w * (SG::TILE / (int)sizeof(E));
    f32x4 S[ND];
    const float* Sin = a.S_in ? a.S_in + bh * DK * DV : nullptr;
#pragma unroll
    for (int db = 0; db < ND; ++db)
#pragma unroll
        for (int i = 0; i < 4; ++i) S[db][i] = Sin ? Sin[(size_t)(16 * db + 4 * g + i) * DV + v0 + r] : 0.f;
    ring_barrier();
    for (int n = 0; n < NC; ++n) {
        const char* slot = ring + (n % P) * G::SLOT;
        if (a.hT) {
            E* hT = a.hT + (bh * NC + n) * DK * DV;
            if constexpr (HNAT) {
                Frag<E> fs[KK];
#pragma unroll
                for (int kk = 0; kk < KK; ++kk) fs[kk] = frag_from_acc<E>(S[2 * kk], S[2 * kk + 1]);
                store_state_tr<E, DK, DV>(hT, fs, tile, v0, l);
            } else {
#pragma unroll
                for (int kk = 0; kk < KK; ++kk) st8T(hT, vb * KK + kk, l, S[2 * kk], S[2 * kk + 1]);
            }
        }
        if constexpr (HN) {
            Frag<E> fs[KK];
#pragma unroll
            for (int kk = 0; kk < KK; ++kk) fs[kk] = frag_from_acc<E>(S[2 * kk], S[2 * kk + 1]);
            store_state_tr<E, DK, DV>(a.hN + (bh * NC + n) * DK * DV, fs, tile, v0, l);
        }
        const E* Vs = (const E*)(slot + (NKU + w * NVU) * RING_UNIT);
        const float* eCs = (const float*)(slot + (NU - 1) * RING_UNIT);
        Frag<E> vf[2];
#pragma unroll
        for (int j = 0; j < 2; ++j) vf[j] = ldfrag_tr(Vs, 16, 32 * j, 0, l);
#pragma unroll
        for (int db = 0; db < ND; ++db) {
            f32x4 acc = S[db] * ld4f(eCs + 16 * db + 4 * g);
#pragma unroll
            for (int j = 0; j < 2; ++j) mma(acc, ring_frag(slot, 2 * db + j, l, (E*)nullptr), vf[j]);
            S[db] = acc;
        }
        ring_barrier();
    }
    if (a.S_out) {
        float* So = a.S_out + bh * DK * DV;
#pragma unroll
        for (int db = 0; db < ND; ++db)
#pragma unroll
            for (int i = 0; i < 4; ++i) So[(size_t)(16 * db + 4 * g + i) * DV + v0 + r] = S[db][i];
    }
}

// ---------------------------------------------------------------------------
// out: one work-group (8 waves) per (block, head, batch); waves R and R + 4
// own tokens 16R..16R+15 and split the value slices.  O^T tiles: inter part (h^T (Q*exp(b))^T) plus P V.  Q, K,
// V and the gate are staged row-major in LDS (V read transposed; when V does
// not fit, its fragments are gathered from global memory).
// ---------------------------------------------------------------------------
template <typename E, int DK, int DV> struct GlaOutLds {
    static constexpr int PK = RP<E, DK>, PV = RP<E, DV>, PB = DK + 4;
    static constexpr size_t o_Q = 0, o_K = o_Q + sizeof(E) * BLK * PK, o_B = o_K + sizeof(E) * BLK * PK;
    static constexpr size_t o_V = o_B + 4 * BLK * PB;  // V rows; g is staged here first
    static constexpr size_t vbytes = sizeof(E) * BLK * (PV > PK ? PV : PK);
    static constexpr bool VLDS = o_V + vbytes <= 150 * 1024;
    static constexpr size_t total = o_V + (VLDS ? vbytes : sizeof(E) * BLK * PK);
};

// HN: each h^T slice the kernel loads is also stored at hN in the block
// adjoints' tiled [d][v] layout, through a per-wave LDS tile (the slices of
// a half are spread over its four waves): the saved states of gla_fwd_save,
// written here, off the scan's sequential chain.
template <typename E, int DK, int DV, bool SG, bool HN = false>
__global__ __launch_bounds__(512) void gla_out_kernel(GlaOutArgs<E> a) {
    using Lay = GlaOutLds<E, DK, DV>;
    constexpr int NT = 512;
    constexpr int PK = Lay::PK, PV = Lay::PV, PB = Lay::PB, KK = DK / 32, NVH = DV / 32;  // value slices per half
    constexpr int HTB = HN && sizeof(E) == 2 ? state_tile_bytes(DK, sizeof(E)) : 16;  // per wave
    __shared__ __align__(16) char lds[Lay::total];
    __shared__ __align__(16) E htile[8 * HTB / sizeof(E)];
    __shared__ __align__(16) float zrow[DK];
    __shared__ float seg[256];
    // the P^T tiles (sb, R) in accumulator layout, one writer each
    __shared__ __align__(16) Raw4<E> Px[4][4][64];
    E* Qs = (E*)(lds + Lay::o_Q);
    E* Ks = (E*)(lds + Lay::o_K);
    float* Bs = (float*)(lds + Lay::o_B);
    E* Vs = (E*)(lds + Lay::o_V);

    const int n = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
    // wave w8: token tile R = w8 & 3, half hf = w8 >> 2 (halves split the value slices)
    const int tid = threadIdx.x, w8 = tid >> 6, R = w8 & 3, hf = w8 >> 2, l = tid & 63, r = l & 15, g = l >> 4;
    const int T = a.T, H = a.H, NC = a.NC;
    const size_t tok0 = (size_t)b * T + (size_t)n * BLK;
    const size_t chunk = ((size_t)b * H + h) * NC + n;
    const int nvalid = min(BLK, T - n * BLK);
    const size_t ldk = (size_t)H * DK, ldv = (size_t)H * DV;
    const E* vbase = a.v + tok0 * ldv + (size_t)h * DV;
    const E* hT = a.hT + chunk * DK * DV;

    // h^T slices of this half, loaded AHEAD slices before their use
    constexpr int AHEAD = NVH > 2 ? 2 : 1, NB = AHEAD + 1;
    Frag<E> fh[NB][KK];
    auto load_slice = [&](int buf, int vb) {
#pragma unroll
        for (int kk = 0; kk < KK; ++kk) fh[buf][kk] = ldfragT(hT, vb * KK + kk, l);
    };
    {
        const auto qx = load_rows<E, BLK, DK, NT>(a.q + tok0 * ldk + (size_t)h * DK, ldk, nvalid);
        const auto kx = load_rows<E, BLK, DK, NT>(a.k + tok0 * ldk + (size_t)h * DK, ldk, nvalid);
        const auto gx = load_gate<SG, E, DK, NT>(a.g, tok0, h, H, nvalid);
#pragma unroll
        for (int j = 0; j < AHEAD; ++j) load_slice(j, hf * NVH + j);
        store_rows<E, BLK, DK, PK, NT>(qx, Qs);
        store_rows<E, BLK, DK, PK, NT>(kx, Ks);
        store_rows<E, BLK, DK, PK, NT>(gx, Vs);
        if (tid < DK) zrow[tid] = 0.f;
    }
    __syncthreads();
    if constexpr (Lay::VLDS) {
        const auto vx = load_rows<E, BLK, DV, NT>(vbase, ldv, nvalid);
        gate_cumsum<E, DK, PK, PB>(Vs, Bs, seg, nvalid);
        __syncthreads();
        store_rows<E, BLK, DV, PV, NT>(vx, Vs);
    } else {
        gate_cumsum<E, DK, PK, PB>(Vs, Bs, seg, nvalid);
    }
    __syncthreads();

    const int tl = 16 * R + r;
    const float* bt = Bs + tl * PB;
    const float* refO = R > 0 ? Bs + (16 * R - 1) * PB : zrow;  // boundary before tile R
    const float* refD = Bs + (16 * R + 7) * PB;                 // middle of tile R
    // The wave forms the P^T tiles sb = hf, hf + 2 that are <= R (below): the
    // off-diagonal ones (sb < R) take qo, the diagonal one (sb = R) qd, so a
    // wave builds only the decayed Q fragments it uses (a scalar test: R and
    // hf are the wave's).
    const bool need_qo = __builtin_amdgcn_readfirstlane(hf < R ? 1 : 0);
    const bool need_qd = __builtin_amdgcn_readfirstlane((R & 1) == hf ? 1 : 0);
    Frag<E> qi[KK], qo[KK], qd[KK];
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) {
        qi[kk] = frag_row_decay(Qs, PK, tl, 32 * kk, bt, zrow, 1.f);
        qo[kk] = need_qo ? frag_row_decay(Qs, PK, tl, 32 * kk, bt, refO, 1.f) : Frag<E>{};
        qd[kk] = need_qd ? frag_row_decay(Qs, PK, tl, 32 * kk, bt, refD, 1.f) : Frag<E>{};
    }
    // P^T[sb][R]: rows s, column t = tl.  Both waves of token tile R need
    // all of its tiles; wave (R, hf) forms the tiles sb = hf, hf + 2 (when
    // sb <= R), rounded to E as the product below takes them, and the two
    // exchange them through LDS.
#pragma unroll
    for (int u = 0; u < 2; ++u) {
        const int sb = hf + 2 * u;
        if (sb <= R) {
            f32x4 acc = zero4();
            const int s = 16 * sb + r;
            const float* ref = sb < R ? refO : refD;
#pragma unroll
            for (int kk = 0; kk < KK; ++kk)
                mma(acc, frag_row_decay(Ks, PK, s, 32 * kk, Bs + s * PB, ref, -1.f), sb < R ? qo[kk] : qd[kk]);
#pragma unroll
            for (int i = 0; i < 4; ++i)
                if (16 * sb + 4 * g + i > tl) acc[i] = 0.f;
            Px[sb][R][l] = to_raw4<E>(acc);
        }
    }
    __syncthreads();
    f32x4 P[4];
#pragma unroll
    for (int sb = 0; sb < 4; ++sb) P[sb] = sb <= R ? cvt4(Px[sb][R][l]) : zero4();
    Frag<E> fp[2];
    fp[0] = frag_from_acc<E>(P[0], P[1]);
    fp[1] = frag_from_acc<E>(P[2], P[3]);
    E* ob = a.o + tok0 * ldv + (size_t)h * DV;
    auto compute_slice = [&](int buf, int vb) {
        f32x4 acc = zero4();
#pragma unroll
        for (int kk = 0; kk < KK; ++kk) mma(acc, fh[buf][kk], qi[kk]);
#pragma unroll
        for (int j = 0; j < 2; ++j)
            if (2 * j <= R) {
                if constexpr (Lay::VLDS) mma(acc, ldfrag_tr(Vs, PV, 32 * j, 16 * vb, l), fp[j]);
                else mma(acc, ldfrag_tokcol(vbase, ldv, j, g, 16 * vb + r, nvalid), fp[j]);
            }
        if (tl < nvalid) st4(ob + (size_t)tl * ldv + 16 * vb + 4 * g, acc);
        if constexpr (HN) {
            if ((vb & 3) == R)  // R is the wave's: a scalar test
                store_state_tr<E, DK, DV>(a.hN + chunk * DK * DV, fh[buf], htile + w8 * (HTB / (int)sizeof(E)),
                                          16 * vb, l);
        }
    };
#pragma unroll
    for (int jv = 0; jv < NVH; ++jv) {
        if (jv + AHEAD < NVH) load_slice((jv + AHEAD) % NB, hf * NVH + jv + AHEAD);
        compute_slice(jv % NB, hf * NVH + jv);
    }
}

// ---------------------------------------------------------------------------
// dscan: reverse over the blocks, same work-group shape as the forward scan.
// Saves dh_n (tiled, key-major) and dVs_n = Kh_n dh_n (the state part of dV,
// token-major).  Slot: Kh | (Q*exp(b))^T | dO slices | exp(b_C).
// ---------------------------------------------------------------------------
template <typename E, int DK, int DV> struct GlaDscanGeom : GlaSlices<E, DK, DV> {
    using SL = GlaSlices<E, DK, DV>;
    static constexpr int ND = DK / 16, KK = DK / 32;
    static constexpr int NHU = 4 * KK * SL::UPF, NQU = 2 * ND * SL::UPF;
    static constexpr int NU = NHU + NQU + SL::NS * SL::NVU + 1;
    static constexpr int SLOT = RingGeom<NU, SL::NPW>::SLOT;
    // per consumer wave: the state store's tile, or the dV rows' staging
    static constexpr int TILE = state_tile_bytes(DK, sizeof(E)) > BLK * 16 * (int)sizeof(E)
                                    ? state_tile_bytes(DK, sizeof(E)) : BLK * 16 * (int)sizeof(E);
    static constexpr int PF = (144 * 1024 - SL::NS * TILE) / SLOT;
    static constexpr int P = PF > 4 ? 4 : (PF < 2 ? 2 : PF);
};

template <typename E, int DK, int DV>
__global__ __launch_bounds__((GlaSlices<E, DK, DV>::THREADS)) void gla_scan_bwd_kernel(GlaScanBwdArgs<E> a) {
    using SG = GlaDscanGeom<E, DK, DV>;
    constexpr int ND = SG::ND, KK = SG::KK, NS = SG::NS, NU = SG::NU, P = SG::P, NHU = SG::NHU, NQU = SG::NQU;
    constexpr int NVU = SG::NVU, UPF = SG::UPF, NPW = SG::NPW, UE = UNIT_ELEMS<E>, LE = LANE_ELEMS<E>;
    using G = RingGeom<NU, NPW>;
    __shared__ __align__(16) char ring[P * G::SLOT];
    __shared__ __align__(16) E tiles[NS * SG::TILE / sizeof(E)];
    const int H = a.H, NC = a.NC;
    int b, h, vg;
    if (!scan_coords(SG::NG, a.BH, H, b, h, vg)) return;
    const int w = threadIdx.x >> 6, l = threadIdx.x & 63, r = l & 15, g = l >> 4;
    const size_t bh = (size_t)b * H + h, ldv = (size_t)H * DV;

    // round m handles block NC - 1 - m
    if (w >= NS) {  // producers
        const int pid = w - NS;
        auto issue = [&](int m) {
            const int n = NC - 1 - m;
            const size_t c = bh * NC + n;
            const int nvalid = min(BLK, a.T - n * BLK);
            const E* Kh = a.Kh + c * BLK * DK + l * LE;
            const E* QgT = a.QgT + c * BLK * DK + l * LE;
            const E* drows = a.dO + ((size_t)b * a.T + (size_t)n * BLK) * ldv + (size_t)h * DV + 16 * NS * vg;
            const float* eC = a.eC + c * DK + 4 * min(l, DK / 4 - 1);
            auto src = [&](int u) -> const void* {
                if (u < NHU) return Kh + u * UE;
                if (u < NHU + NQU) return QgT + (u - NHU) * UE;
                if (u < NHU + NQU + NS * NVU) {
                    const int q = u - NHU - NQU;
                    return slice_src<E, DV>(drows + 16 * (q / NVU), ldv, q % NVU, l, nvalid);
                }
                return eC;
            };
            ring_issue_units<NU, NPW>(ring + (m % P) * G::SLOT, pid, src);
        };
        const int pre = NC < P - 1 ? NC : P - 1;
        for (int m = 0; m < pre; ++m) issue(m);
        ring_wait<G::NU_MIN>(pre - 1);  // round 0 has landed
        ring_barrier();
        for (int m = 0; m < NC; ++m) {
            if (m + P - 1 < NC) issue(m + P - 1);
            const int last = (m + P - 1 < NC ? m + P - 1 : NC - 1);
            ring_wait<G::NU_MIN>(last - (m + 1));  // round m + 1 has landed
            ring_barrier();
        }
        return;
    }

    const int vb = NS * vg + w, v0 = 16 * vb;
    E* tile = tiles + w * (SG::TILE / (int)sizeof(E));
    f32x4 dS[ND];
    const float* dSo = a.dS_out ? a.dS_out + bh * DK * DV : nullptr;
#pragma unroll
    for (int db = 0; db < ND; ++db)
#pragma unroll
        for (int i = 0; i < 4; ++i) dS[db][i] = dSo ? dSo[(size_t)(16 * db + 4 * g + i) * DV + v0 + r] : 0.f;
    ring_barrier();
    for (int m = 0; m < NC; ++m) {
        const size_t c = bh * NC + (NC - 1 - m);
        const char* slot = ring + (m % P) * G::SLOT;
        Frag<E> fs[KK];
#pragma unroll
        for (int kk = 0; kk < KK; ++kk) fs[kk] = frag_from_acc<E>(dS[2 * kk], dS[2 * kk + 1]);
        store_state_tr<E, DK, DV>(a.dh + c * DK * DV, fs, tile, v0, l);
        f32x4 dVs[4];
#pragma unroll
        for (int tb = 0; tb < 4; ++tb) {
            f32x4 acc = zero4();
#pragma unroll
            for (int kk = 0; kk < KK; ++kk) mma(acc, ring_frag(slot, tb * KK + kk, l, (E*)nullptr), fs[kk]);
            dVs[tb] = acc;
        }
        store_rows16<E, BLK>(a.dVs + c * BLK * DV, DV, dVs, tile, v0, r, g);
        const E* dOs = (const E*)(slot + (NHU + NQU + w * NVU) * RING_UNIT);
        const float* eCs = (const float*)(slot + (NU - 1) * RING_UNIT);
        Frag<E> df[2];
#pragma unroll
        for (int j = 0; j < 2; ++j) df[j] = ldfrag_tr(dOs, 16, 32 * j, 0, l);
#pragma unroll
        for (int db = 0; db < ND; ++db) {
            f32x4 acc = dS[db] * ld4f(eCs + 16 * db + 4 * g);
#pragma unroll
            for (int j = 0; j < 2; ++j) mma(acc, ring_frag(slot, NHU / UPF + 2 * db + j, l, (E*)nullptr), df[j]);
            dS[db] = acc;
        }
        ring_barrier();
    }
    float* dSi = a.dS_in + bh * DK * DV;
#pragma unroll
    for (int db = 0; db < ND; ++db)
#pragma unroll
        for (int i = 0; i < 4; ++i) dSi[(size_t)(16 * db + 4 * g + i) * DV + v0 + r] = dS[db][i];
}

// ---------------------------------------------------------------------------
// intra: one work-group (8 waves) per (block, head, batch); waves R and R + 4
// own tokens 16R..16R+15 (as t for dq, as s for dk and dv) and split each
// phase's loops.  All output tiles are
// transposed ([feature][token]) so each lane stores four contiguous values.
// K, Q, V, dO and the gate tile are staged row-major in LDS with every load
// of a stage in flight at once; the block gate cumsum is formed in LDS.
// ---------------------------------------------------------------------------
template <typename E, int DK, int DV> struct GlaIntraLds {
    static constexpr int PK = RP<E, DK>, PV = RP<E, DV>, PB = DK + 4, PD = DK + 1;
    static constexpr size_t o_K = 0;                                   // E[64][PK]
    static constexpr size_t o_Q = o_K + sizeof(E) * BLK * PK;          // E[64][PK]
    static constexpr size_t o_B = o_Q + sizeof(E) * BLK * PK;          // f32[64][PB]  b = cumsum(g)
    static constexpr size_t o_U = o_B + 4 * BLK * PB;                  // union:
    static constexpr size_t u_G = o_U;                                 //   g staging E[64][PK]
    static constexpr size_t u_dO = o_U, u_V = u_dO + sizeof(E) * BLK * PV;  //   dO, V  E[64][PV]
    static constexpr size_t u_dg = o_U;                                //   dgb f32[64][PD]
    static constexpr size_t end1 = u_V + sizeof(E) * BLK * PV, end2 = u_dg + 4 * BLK * PD;
    // dgb fits in the dO rows: V stays readable while dgb is written
    static constexpr bool VKEEP = 4 * BLK * PD <= sizeof(E) * BLK * PV;
    static constexpr size_t total = end1 > end2 ? end1 : end2;
};

// With KDA the same kernel runs the pair and state parts of the KDA block
// adjoints: v is U (token-major), P and dV are skipped (dv comes from the WY
// adjoint kernel), and the strictly lower dM of the decayed Gram product adds
// its row side (M[t][s], t as row) and column side to dK, with the X part
// beta e^b dX; the gate term becomes q dq - k dk + 2 k (M row side + X part).
template <typename E, int DK, int DV, bool SG, bool KDA = false>
__global__ __launch_bounds__(512) void gla_bwd_intra_kernel(GlaIntraArgs<E> a) {
    using Lay = GlaIntraLds<E, DK, DV>;
    constexpr int NT = 512;
    constexpr int PK = Lay::PK, PV = Lay::PV, PB = Lay::PB, PD = Lay::PD, KV = DV / 32, KK = DK / 32;
    static_assert(Lay::total <= 150 * 1024, "LDS budget");
    __shared__ __align__(16) char lds[Lay::total];
    __shared__ float rsum[4][DK], rowhd[4][DK], seg[256], segt[SG ? 1 : NT];
    __shared__ __align__(16) float zrow[DK];
    E* Ks = (E*)(lds + Lay::o_K);
    E* Qs = (E*)(lds + Lay::o_Q);
    float* Bs = (float*)(lds + Lay::o_B);

    const int n = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
    // wave w8: token tile R = w8 & 3, half hf = w8 >> 2 (halves split the value
    // and feature loops)
    const int tid = threadIdx.x, w8 = tid >> 6, R = w8 & 3, hf = w8 >> 2, l = tid & 63, r = l & 15, g = l >> 4;
    const int T = a.T, H = a.H, NC = a.NC;
    const size_t tok0 = (size_t)b * T + (size_t)n * BLK;
    const size_t chunk = ((size_t)b * H + h) * NC + n;
    const int nvalid = min(BLK, T - n * BLK);
    const size_t ldk = (size_t)H * DK, ldv = (size_t)H * DV;
    const E* qb = a.q + tok0 * ldk + (size_t)h * DK;
    const E* kb = a.k + tok0 * ldk + (size_t)h * DK;
    const E* vbase = a.v + tok0 * ldv + (size_t)h * DV;
    const E* dob = a.dO + tok0 * ldv + (size_t)h * DV;
    const E* S0 = a.h + chunk * DK * DV;    // tiled [d][v]
    const E* dS1 = a.dh + chunk * DK * DV;  // tiled [d][v]

    // ---- staging: K, Q, g; then dO, V while the gate cumsum runs ----
    {
        const auto kx = load_rows<E, BLK, DK, NT>(kb, ldk, nvalid);
        const auto qx = load_rows<E, BLK, DK, NT>(qb, ldk, nvalid);
        const auto gx = load_gate<SG, E, DK, NT>(a.g, tok0, h, H, nvalid);
        store_rows<E, BLK, DK, PK, NT>(kx, Ks);
        store_rows<E, BLK, DK, PK, NT>(qx, Qs);
        store_rows<E, BLK, DK, PK, NT>(gx, (E*)(lds + Lay::u_G));
        if (tid < DK) zrow[tid] = 0.f;
    }
    __syncthreads();
    {
        const auto ox = load_rows<E, BLK, DV, NT>(dob, ldv, nvalid);
        const auto vx = load_rows<E, BLK, DV, NT>(vbase, ldv, nvalid);
        gate_cumsum<E, DK, PK, PB>((const E*)(lds + Lay::u_G), Bs, seg, nvalid);
        __syncthreads();
        store_rows<E, BLK, DV, PV, NT>(ox, (E*)(lds + Lay::u_dO));
        store_rows<E, BLK, DV, PV, NT>(vx, (E*)(lds + Lay::u_V));
    }
    __syncthreads();
    const E* dOs = (const E*)(lds + Lay::u_dO);
    const E* Vs = (const E*)(lds + Lay::u_V);

    const int tl = 16 * R + r;  // this lane's token (column of every transposed tile)
    const float* bt = Bs + tl * PB;
    const float* refO = R > 0 ? Bs + (16 * R - 1) * PB : zrow;  // boundary before tile R
    const float* refD = Bs + (16 * R + 7) * PB;                 // middle of tile R
    const float* refE = Bs + (16 * R + 15) * PB;                // end of tile R
    const float* bC = Bs + (BLK - 1) * PB;

    Frag<E> fdo[KV], fv[KV];
#pragma unroll
    for (int kk = 0; kk < KV; ++kk) {
        fdo[kk] = ldfrag(dOs + tl * PV + 32 * kk + 4 * g);  // Bt = dO, rows of tile R
        fv[kk] = ldfrag(Vs + tl * PV + 32 * kk + 4 * g);    // Bt = V, rows of tile R
    }
    // K row tl scaled for the two references of (3)
    Frag<E> fkD[KK], fkE[KK];
    if constexpr (!KDA) {
#pragma unroll
        for (int kk = 0; kk < KK; ++kk) {
            fkD[kk] = frag_row_decay(Ks, PK, tl, 32 * kk, bt, refD, -1.f);
            fkE[kk] = frag_row_decay(Ks, PK, tl, 32 * kk, bt, refE, -1.f);
        }
    }
    // (1) dP^T[sb][R] (rows s, col t = tl), (2) dP[tb][R] (rows t, col s = tl),
    // (3) P[tb][R] (rows t, col s = tl); all masked to s <= t.
    f32x4 dPT[4], dP[4], P[4];
#pragma unroll
    for (int x = 0; x < 4; ++x) {
        f32x4 acc = zero4();
        if (x <= R) {
#pragma unroll
            for (int kk = 0; kk < KV; ++kk) mma(acc, ldfrag(Vs + (16 * x + r) * PV + 32 * kk + 4 * g), fdo[kk]);
#pragma unroll
            for (int i = 0; i < 4; ++i)
                if (16 * x + 4 * g + i > tl) acc[i] = 0.f;
        }
        dPT[x] = acc;
        f32x4 acc2 = zero4(), acc3 = zero4();
        if (x >= R) {
#pragma unroll
            for (int kk = 0; kk < KV; ++kk) mma(acc2, ldfrag(dOs + (16 * x + r) * PV + 32 * kk + 4 * g), fv[kk]);
            if constexpr (!KDA) {
                const float* ref = x > R ? refE : refD;
                const int t = 16 * x + r;
#pragma unroll
                for (int kk = 0; kk < KK; ++kk) {
                    Frag<E> fq = frag_row_decay(Qs, PK, t, 32 * kk, Bs + t * PB, ref, 1.f);
                    mma(acc3, fq, x > R ? fkE[kk] : fkD[kk]);
                }
            }
#pragma unroll
            for (int i = 0; i < 4; ++i)
                if (16 * x + 4 * g + i < tl) {
                    acc2[i] = 0.f;
                    acc3[i] = 0.f;
                }
        }
        dP[x] = acc2;
        P[x] = acc3;
    }
    // split dP^T into off-diagonal (s < 16R) and diagonal (s in tile R) parts,
    // dP into later (t >= 16R + 16) and diagonal parts
    Frag<E> fptO[2], fptD[2], fpL[2], fpD[2], fP[2];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
        f32x4 o0 = (2 * j < R) ? dPT[2 * j] : zero4(), o1 = (2 * j + 1 < R) ? dPT[2 * j + 1] : zero4();
        f32x4 d0 = (2 * j == R) ? dPT[2 * j] : zero4(), d1 = (2 * j + 1 == R) ? dPT[2 * j + 1] : zero4();
        fptO[j] = frag_from_acc<E>(o0, o1);
        fptD[j] = frag_from_acc<E>(d0, d1);
        f32x4 l0 = (2 * j > R) ? dP[2 * j] : zero4(), l1 = (2 * j + 1 > R) ? dP[2 * j + 1] : zero4();
        f32x4 e0 = (2 * j == R) ? dP[2 * j] : zero4(), e1 = (2 * j + 1 == R) ? dP[2 * j + 1] : zero4();
        fpL[j] = frag_from_acc<E>(l0, l1);
        fpD[j] = frag_from_acc<E>(e0, e1);
        fP[j] = frag_from_acc<E>(P[2 * j], P[2 * j + 1]);
    }
    // KDA: dM^T[x][R] (rows s, col t = tl) and dM[x][R] (rows t, col s = tl),
    // split like dP^T and dP
    Frag<E> fmtO[2], fmtD[2], fmL[2], fmD[2];
    if constexpr (KDA) {
        const float* dMb = a.dM + chunk * BLK * BLK;
        f32x4 mT[4], mR[4];
#pragma unroll
        for (int x = 0; x < 4; ++x) {
            mT[x] = x <= R ? ld4f(dMb + tl * BLK + 16 * x + 4 * g) : zero4();
            f32x4 v4 = zero4();
            if (x >= R) {
#pragma unroll
                for (int i = 0; i < 4; ++i) v4[i] = dMb[(16 * x + 4 * g + i) * BLK + tl];
            }
            mR[x] = v4;
        }
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            f32x4 o0 = (2 * j < R) ? mT[2 * j] : zero4(), o1 = (2 * j + 1 < R) ? mT[2 * j + 1] : zero4();
            f32x4 d0 = (2 * j == R) ? mT[2 * j] : zero4(), d1 = (2 * j + 1 == R) ? mT[2 * j + 1] : zero4();
            fmtO[j] = frag_from_acc<E>(o0, o1);
            fmtD[j] = frag_from_acc<E>(d0, d1);
            f32x4 l0 = (2 * j > R) ? mR[2 * j] : zero4(), l1 = (2 * j + 1 > R) ? mR[2 * j + 1] : zero4();
            f32x4 e0 = (2 * j == R) ? mR[2 * j] : zero4(), e1 = (2 * j + 1 == R) ? mR[2 * j + 1] : zero4();
            fmL[j] = frag_from_acc<E>(l0, l1);
            fmD[j] = frag_from_acc<E>(e0, e1);
        }
    }
    const float bet_tl = KDA && tl < nvalid ? to_f(a.beta[(tok0 + tl) * H + h]) : 0.f;
    // (6) dV^T[vb][R] = dO^T P + (Kh dh)^T   (rows v, col s = tl)
    if constexpr (!KDA) {
        // the state part of dV, all loads issued before use (rows past the
        // sequence end read the last valid row and are dropped)
        constexpr int NVH = DV / 32;  // value blocks per half
        Raw4<E> dsr[NVH];
        const E* dVrow = a.dVs + chunk * BLK * DV + (size_t)min(tl, nvalid - 1) * DV;
#pragma unroll
        for (int jv = 0; jv < NVH; ++jv) dsr[jv] = ldraw4(dVrow + 16 * (hf * NVH + jv) + 4 * g);
#pragma unroll
        for (int jv = 0; jv < NVH; ++jv) {
            const int vb = hf * NVH + jv;
            f32x4 acc = tl < nvalid ? cvt4(dsr[jv]) : zero4();
#pragma unroll
            for (int j = 0; j < 2; ++j)
                if (32 * j + 32 > 16 * R) mma(acc, ldfrag_tr(dOs, PV, 32 * j, 16 * vb, l), fP[j]);
            if (tl < nvalid) st4(a.dv + (tok0 + tl) * ldv + (size_t)h * DV + 16 * vb + 4 * g, acc);
        }
    }
    __syncthreads();  // dO, V no longer read from LDS: the union becomes dgb
    float* dgb = (float*)(lds + Lay::u_dg);
    constexpr int NDH = DK / 32;  // feature blocks per half
    // (4) dQ^T and (5) dK^T, per 16-row block of features d (this half's
    // blocks).  The state fragments of the next block are loaded while the
    // current block's decay terms run.
    Frag<E> fh[KV], fd[KV];
#pragma unroll
    for (int kk = 0; kk < KV; ++kk) {
        fh[kk] = ldfragT(S0, (hf * NDH) * KV + kk, l);
        fd[kk] = ldfragT(dS1, (hf * NDH) * KV + kk, l);
    }
#pragma unroll
    for (int jd = 0; jd < NDH; ++jd) {
        const int db = hf * NDH + jd;
        // dQ inter exp(b_t) (S0 dO^T), the state part of dK, and the row sums
        // of S0 * dh for rows 16 db + r (wave R sums the value blocks kk = R mod 4)
        f32x4 qi = zero4(), ks = zero4();
        float hd = 0.f;
#pragma unroll
        for (int kk = 0; kk < KV; ++kk) {
            mma(qi, fh[kk], fdo[kk]);
            if constexpr (Lay::VKEEP) mma(ks, fd[kk], ldfrag(Vs + tl * PV + 32 * kk + 4 * g));
            else mma(ks, fd[kk], fv[kk]);
            if ((kk & 3) == R) {
                if constexpr (sizeof(E) == 2) {
#pragma unroll
                    for (int i = 0; i < 8; ++i) hd += (float)fh[kk].v[i] * (float)fd[kk].v[i];
                } else {
#pragma unroll
                    for (int i = 0; i < 4; ++i) hd += fh[kk].lo[i] * fd[kk].lo[i] + fh[kk].hi[i] * fd[kk].hi[i];
                }
            }
        }
        hd += __shfl_xor(hd, 16, 64);
        hd += __shfl_xor(hd, 32, 64);
        if (g == 0) rowhd[R][16 * db + r] = hd;
        if (jd + 1 < NDH) {
#pragma unroll
            for (int kk = 0; kk < KV; ++kk) {
                fh[kk] = ldfragT(S0, (db + 1) * KV + kk, l);
                fd[kk] = ldfragT(dS1, (db + 1) * KV + kk, l);
            }
        }
        // dQ: intra, off-diagonal (reference b_{16R-1}) and diagonal (reference b_{16R+7});
        // KDA: the same decayed K fragments give the M row side (eo, ed)
        f32x4 qo = zero4(), qd = zero4(), eo = zero4(), ed = zero4();
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            if (32 * j < 16 * R) {
                const Frag<E> x = frag_col_decay(Ks, PK, Bs, PB, 16 * db, 32 * j, refO, -1.f, 0, 16 * R);
                mma(qo, x, fptO[j]);
                if constexpr (KDA) mma(eo, x, fmtO[j]);
            }
            if (32 * j <= 16 * R && 16 * R < 32 * j + 32) {
                const Frag<E> x = frag_col_decay(Ks, PK, Bs, PB, 16 * db, 32 * j, refD, -1.f, 16 * R, 16 * R + 16);
                mma(qd, x, fptD[j]);
                if constexpr (KDA) mma(ed, x, fmtD[j]);
            }
        }
        // dK: intra, later tiles (reference b_{16R+15}) and diagonal;
        // KDA: the M column side with K in place of Q (fo, fd2)
        f32x4 kl = zero4(), kd = zero4(), fo = zero4(), fd2 = zero4();
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            if (32 * j + 32 > 16 * R + 16) {
                mma(kl, frag_col_decay(Qs, PK, Bs, PB, 16 * db, 32 * j, refE, 1.f, 16 * R + 16, BLK), fpL[j]);
                if constexpr (KDA) mma(fo, frag_col_decay(Ks, PK, Bs, PB, 16 * db, 32 * j, refE, 1.f, 16 * R + 16, BLK), fmL[j]);
            }
            if (32 * j <= 16 * R && 16 * R < 32 * j + 32) {
                mma(kd, frag_col_decay(Qs, PK, Bs, PB, 16 * db, 32 * j, refD, 1.f, 16 * R, 16 * R + 16), fpD[j]);
                if constexpr (KDA) mma(fd2, frag_col_decay(Ks, PK, Bs, PB, 16 * db, 32 * j, refD, 1.f, 16 * R, 16 * R + 16), fmD[j]);
            }
        }
        // element-wise factors: rows d = 16 db + 4 g + i, column token tl
        const int d0 = 16 * db + 4 * g;
        const f32x4 btv = ld4f(bt + d0), rOv = ld4f(refO + d0), rDv = ld4f(refD + d0), rEv = ld4f(refE + d0);
        const f32x4 bCv = ld4f(bC + d0);
        f32x4 dq, dk;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            dq[i] = qi[i] * __expf(btv[i]) + qo[i] * __expf(btv[i] - rOv[i]) + qd[i] * expu(btv[i] - rDv[i]);
            const float es = __expf(bCv[i] - btv[i]);
            dk[i] = kl[i] * __expf(rEv[i] - btv[i]) + kd[i] * expu(rDv[i] - btv[i]) + ks[i] * es;
        }
        float qk[4] = {0.f, 0.f, 0.f, 0.f};
        const f32x4 qv = ld4(Qs + tl * PK + d0), kv = ld4(Ks + tl * PK + d0);
        f32x4 ex = zero4();  // KDA: M row side + X part of dK (enter the gate term with + k)
        if constexpr (KDA) {
            const f32x4 dxv = tl < nvalid ? ld4f(a.dX + chunk * BLK * DK + (size_t)tl * DK + d0) : zero4();
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float e = eo[i] * __expf(btv[i] - rOv[i]) + ed[i] * expu(btv[i] - rDv[i]);
                const float f = fo[i] * __expf(rEv[i] - btv[i]) + fd2[i] * expu(rDv[i] - btv[i]);
                ex[i] = e + bet_tl * dxv[i] * __expf(btv[i]);
                dk[i] += ex[i] + f;
            }
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            qk[i] = qv[i] * dq[i] - kv[i] * dk[i] + 2.f * kv[i] * ex[i];
        }
        // sum_s Kh[s][d] X[d][s] over this wave's 16 tokens (rows d0 + i)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const float x = row16_sum(kv[i] * __expf(bCv[i] - btv[i]) * ks[i]);
            if (r == 0) rsum[R][d0 + i] = x;
        }
        if (tl < nvalid) {
            st4(a.dq + (tok0 + tl) * ldk + (size_t)h * DK + d0, dq);
            st4(a.dk + (tok0 + tl) * ldk + (size_t)h * DK + d0, dk);
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) dgb[tl * PD + d0 + i] = qk[i];
    }
    __syncthreads();
    if constexpr (!SG) {
        // (7) dg[t][d] = sum_{tau >= t} dgb[tau][d] + rowsum(S1 * dh)[d]: thread
        // (sg, d) takes the L-token segment sg of channel d; segment totals
        // first, then each thread adds the later segments' totals (in order)
        // and runs its own segment backwards.
        constexpr int NSEG = NT / DK, L = BLK / NSEG;
        static_assert(NT % DK == 0 && BLK % NSEG == 0, "token segments");
        const int d = tid % DK, sg = tid / DK;
        {
            float x = 0.f;
#pragma unroll 4
            for (int i = L - 1; i >= 0; --i) x += dgb[(sg * L + i) * PD + d];
            segt[sg * DK + d] = x;
        }
        __syncthreads();
        {
            const float hdd = (rowhd[0][d] + rowhd[1][d]) + (rowhd[2][d] + rowhd[3][d]);
            float acc = __expf(bC[d]) * hdd + rsum[0][d] + rsum[1][d] + rsum[2][d] + rsum[3][d];
            for (int s2 = NSEG - 1; s2 > sg; --s2) acc += segt[s2 * DK + d];
            E* dgp = a.dg + (tok0 + (size_t)sg * L) * ldk + (size_t)h * DK + d;
#pragma unroll 4
            for (int i = L - 1; i >= 0; --i) {
                acc += dgb[(sg * L + i) * PD + d];
                if (sg * L + i < nvalid) dgp[(size_t)i * ldk] = from_f<E>(acc);
            }
        }
    } else {
        // (7) scalar gate: the channel sum of the per-channel dg above,
        //   dg[t] = sum_{tau >= t} sum_d dgb[tau][d] + sum_d c_d,
        //   c_d = exp(b_C[d]) rowsum(S0 * dh)[d] + sum_s Kh[s][d] X[d][s].
        // Row sums by eight lanes per token; c by wave 1; the reverse scan over
        // the 64 tokens by wave 0 (fixed order throughout).
        {
            const int t = tid >> 3, p = tid & 7;
            float x = 0.f;
            for (int d = p; d < DK; d += 8) x += dgb[t * PD + d];
            x += __shfl_xor(x, 1, 64);
            x += __shfl_xor(x, 2, 64);
            x += __shfl_xor(x, 4, 64);
            if (p == 0) seg[t] = x;
        }
        if (w8 == 1) {
            float c = 0.f;
            for (int d = l; d < DK; d += 64)
                c += __expf(bC[d]) * ((rowhd[0][d] + rowhd[1][d]) + (rowhd[2][d] + rowhd[3][d])) + rsum[0][d] + rsum[1][d] +
                     rsum[2][d] + rsum[3][d];
#pragma unroll
            for (int m = 32; m >= 1; m >>= 1) c += __shfl_xor(c, m, 64);
            if (l == 0) seg[BLK] = c;
        }
        __syncthreads();
        if (w8 == 0) {
            float x = seg[l];
#pragma unroll
            for (int off = 1; off < 64; off <<= 1) {
                const float y = __shfl_down(x, off, 64);
                if (l + off < 64) x += y;
            }
            if (l < nvalid) a.dg[(tok0 + l) * H + h] = from_f<E>(x + seg[BLK]);
        }
    }
}

// ---------------------------------------------------------------------------
// KDA forward prep: per-key-channel decay with the delta rule's erase and
// write (the diagonal-plus-low-rank transition of the StateFlow paper,
// Sec. 2.1, Eq. 1).  With b = cumsum(g) per channel in the block,
//   M[t][s] = sum_d k_t[d] k_s[d] e^{b_t[d] - b_s[d]}   (s < t)
//   T = (I + Diag(beta) M)^-1,  W = T Diag(beta) (K * e^b),  Ut = T Diag(beta) V
// and the scan forms U = Ut - W S, S <- Diag(e^{b_C}) S + (K * e^{b_C - b})^T U:
// the delta-rule WY form with the channel-wise decay absorbed into the
// factors.  M is formed per pair of 16-token tiles with the same references
// as the GLA products (boundary before the row tile off the diagonal, the
// tile's middle token on it).  Outputs use the Gated DeltaNet workspace
// layouts (W, -Ut^T, Kh^T tiled), plus exp(b_C) padded to 256 floats.
// ---------------------------------------------------------------------------
// Precision as for the Gated DeltaNet prep (gdn_kernels.h, "Precision"): T is
// kept in fp32 and W, Ut are formed from its hi/lo split; Ut is stored fp32;
// the decayed keys Kh^T = (K e^{b_C - b})^T are stored as a bf16 hi/lo pair
// (KhT, KhT_lo): with a per-channel decay the scan cannot multiply the exact
// keys, and a rounded decayed key adds components that a slowly decaying
// state keeps.
template <typename E> struct KdaPrepArgs {
    const E *k, *v, *g, *beta;
    int T, H, NC;
    float* eC;
    E *W, *KhT;
    float* UtT;
    E* KhT_lo;
    int* range = nullptr;  // per block: 1 if the gates leave the diagonal tiles' bound
    // backward only (nullable): T^T (tiled [s][t]), the decayed Gram product M
    // (strictly lower, fp32, 16 accumulator tiles) and K e^b (row-major [64][dk])
    E* TT = nullptr;
    float* M = nullptr;
    E* Kd = nullptr;
};

// dst[t][d] = src[t][d] e^{b_t[d]} over a 64 x DK tile (row pitch PX; dst row
// pitch PD, PX when not given; b row pitch PB), 16-byte vectors, all NT threads.
template <typename E, int DK, int PX, int PB, int NT>
__device__ __forceinline__ void scale_exp_rows(const E* src, const float* Bs, E* dst, int PD = PX) {
    constexpr int VEC = 16 / (int)sizeof(E), PER_ROW = DK / VEC, UNITS = BLK * PER_ROW;
#pragma unroll
    for (int j = 0; j < (UNITS + NT - 1) / NT; ++j) {
        const int u = (int)threadIdx.x + NT * j;
        if (UNITS % NT == 0 || u < UNITS) {
            const int t = u / PER_ROW, c = (u % PER_ROW) * VEC;
            union {
                uint4 u;
                E e[VEC];
            } x;
            x.u = *(const uint4*)(src + t * PX + c);
#pragma unroll
            for (int i = 0; i < VEC; ++i) x.e[i] = from_f<E>(to_f(x.e[i]) * __expf(Bs[t * PB + c + i]));
            *(uint4*)(dst + t * PD + c) = x.u;
        }
    }
}

// Block row w of the per-channel decayed Gram product of K,
//   M[t][s] = sum_d k_t[d] k_s[d] e^{b_t[d] - b_s[d]}   (s < t),
// column blocks j <= w with (j & 1) == half when halves split them (all j
// when half < 0).  Each 16 x 16 tile is one dense product of rescaled rows
// against a reference row of b between the tiles: the boundary before tile w
// off the diagonal (both factors <= 1), the middle of tile w on it.
// emit(row, col, value) receives every element of the visited tiles (0 on
// and above the diagonal).
template <typename E, int DK, int PK, int PB, typename F>
__device__ __forceinline__ void kda_gram_row(const E* Ks, const float* Bs, const float* zrow, int w, int half,
                                             F&& emit) {
    constexpr int KK = DK / 32;
    const int l = threadIdx.x & 63, r = l & 15, g = l >> 4;
    const int tl = 16 * w + r;
    const float* refO = w > 0 ? Bs + (16 * w - 1) * PB : zrow;
    const float* refD = Bs + (16 * w + 7) * PB;
    Frag<E> fo[KK], fd[KK];
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) {
        fo[kk] = frag_row_decay(Ks, PK, tl, 32 * kk, Bs + tl * PB, refO, 1.f);
        fd[kk] = frag_row_decay(Ks, PK, tl, 32 * kk, Bs + tl * PB, refD, 1.f);
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        if (half >= 0 && (j & 1) != half) continue;
        f32x4 acc = zero4();
        if (j <= w) {
            const int s = 16 * j + r;
            const float* ref = j < w ? refO : refD;
#pragma unroll
            for (int kk = 0; kk < KK; ++kk)
                mma(acc, j < w ? fo[kk] : fd[kk], frag_row_decay(Ks, PK, s, 32 * kk, Bs + s * PB, ref, -1.f));
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int row = 16 * w + 4 * g + i, col = 16 * j + r;
            emit(row, col, col < row ? acc[i] : 0.f);
        }
    }
}

// KDA prep: one work-group (8 waves) per (block, head, batch).  Wave w8: row
// block w = w8 & 3, half hf = w8 >> 2 (the halves split the Gram's column
// blocks and the output tiles).
template <typename E, int DK, int DV>
__global__ __launch_bounds__(512) void kda_prep_kernel(KdaPrepArgs<E> a) {
    constexpr int NT = 512;
    const int n = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
    const int tid = threadIdx.x, w8 = tid >> 6, w = w8 & 3, hf = w8 >> 2, l = tid & 63, r = l & 15, g = l >> 4;
    const int T = a.T, H = a.H, NC = a.NC;
    const size_t tok0 = (size_t)b * T + (size_t)n * BLK;
    const size_t chunk = ((size_t)b * H + h) * NC + n;
    const int nvalid = min(BLK, T - n * BLK);
    const size_t ldk = (size_t)H * DK, ldv = (size_t)H * DV;
    constexpr int PK = RP<E, DK>, PV = RP<E, DV>, PB = DK + 4, ND = DK / 16;

    // LDS: K, the cumulative gate b (fp32) and one fp32 64 x 64 region that
    // holds g (for the cumsum), then A, then T, then V; K * e^b is formed
    // where it is read.  About 73 KB with dk = dv = 128: two work-groups per CU.
    __shared__ __align__(16) E Ks[BLK * PK];
    __shared__ __align__(16) float Bs[BLK * PB];
    __shared__ __align__(16) float Am[BLK * AP], Td[4 * 256];  // g, A, T (fp32), V
    __shared__ __align__(16) float zrow[DK];
    __shared__ float seg[256];
    __shared__ __align__(16) float s_bet[BLK];
    static_assert(sizeof(E) * BLK * PK <= sizeof(float) * BLK * AP && sizeof(E) * BLK * PV <= sizeof(float) * BLK * AP,
                  "g and V fit the A region");
    E* Gs = (E*)Am;  // g, staged for the cumsum
    E* Vs = (E*)Am;  // V, once T has been read into registers

    // V waits in registers until its rows are staged (after T)
    const auto vx = load_rows<E, BLK, DV, NT>(a.v + tok0 * ldv + (size_t)h * DV, ldv, nvalid);
    {
        const auto kx = load_rows<E, BLK, DK, NT>(a.k + tok0 * ldk + (size_t)h * DK, ldk, nvalid);
        const auto gx = load_gate<false, E, DK, NT>(a.g, tok0, h, H, nvalid);
        if (tid < BLK) s_bet[tid] = tid < nvalid ? to_f(a.beta[(tok0 + tid) * H + h]) : 0.f;
        if (tid < DK) zrow[tid] = 0.f;
        store_rows<E, BLK, DK, PK, NT>(kx, Ks);
        store_rows<E, BLK, DK, PK, NT>(gx, Gs);
        __syncthreads();
        gate_cumsum<E, DK, PK, PB>(Gs, Bs, seg, nvalid);
        __syncthreads();
        const bool over = diag_out_of_range<DK, PB>(Bs);
        if (a.range && tid == 0) a.range[chunk] = over ? 1 : 0;
    }
    // exp(b_C) per channel
    const float* bC = Bs + (BLK - 1) * PB;
    if (tid < 256) a.eC[chunk * 256 + tid] = tid < DK ? __expf(bC[tid]) : 0.f;
    // Am[t][s] = beta_t M[t][s] (s < t); M as accumulator tiles for the backward
    float* Mg = a.M ? a.M + chunk * BLK * BLK : nullptr;
    kda_gram_row<E, DK, PK, PB>(Ks, Bs, zrow, w, hf, [&](int row, int col, float m) {
        Am[row * AP + col] = s_bet[row] * m;
        if (Mg) Mg[(4 * (row >> 4) + (col >> 4)) * 256 + l * 4 + (row & 3)] = m;
    });
    __syncthreads();
    if (a.Kd)  // K e^b (factors <= 1), row-major, for the backward
        scale_exp_rows<E, DK, PK, PB, NT>(Ks, Bs, a.Kd + chunk * BLK * DK, DK);
    f32x4 tc[4];
    if (hf == 0) {
        // T = (I + A)^-1, wave w holds column block w
        tri_inverse_cols(Am, Td, tc);  // one barrier inside
        const int s = 16 * w + r;
        if (a.TT) {
#pragma unroll
            for (int i = 0; i < 4; ++i) st4(a.TT + chunk * BLK * BLK + toff<E>(s, 16 * i + 4 * g, BLK), tc[i]);
        }
    } else {
        __syncthreads();  // matches the barrier inside tri_inverse_cols
    }
    __syncthreads();  // A no longer read: T (fp32) takes its place
    if (hf == 0) {
        const int s = 16 * w + r;
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int ii = 0; ii < 4; ++ii) Am[(16 * i + 4 * g + ii) * AP + s] = tc[i][ii];
    }
    __syncthreads();
    // Row fragment (m = t, k = s) of T1 = T Diag(beta): fp32, scaled, split
    auto tfrag = [&](int t, int k0) {
        const float* p = Am + t * AP + k0 + 4 * g;
        return split8<E>(ld4(p) * ld4f(s_bet + k0 + 4 * g), ld4(p + 16) * ld4f(s_bet + k0 + 16 + 4 * g));
    };
    // W^T[d][t] = sum_s (K * e^b)^T[d][s] T1[t][s]  -> stored as W[t][d] (tiled)
    E* Wout = a.W + chunk * BLK * DK;
    // a wave's tiles below all lie in token block w8 & 3, so its split T1 rows
    // are formed once
    const int tbw = w8 & 3;
    const Frag2<E> t1[2] = {tfrag(16 * tbw + r, 0), tfrag(16 * tbw + r, 32)};
#pragma unroll
    for (int tile = w8; tile < ND * 4; tile += 8) {
        const int db = tile >> 2, tb = tbw;
        f32x4 acc = zero4();
#pragma unroll
        for (int j = 0; j < 2; ++j)  // (K e^b)^T fragment, scaled as it is read
            mma2(acc, frag_col_decay(Ks, PK, Bs, PB, 16 * db, 32 * j, zrow, 1.f, 0, BLK), t1[j]);
        st4(Wout + toff<E>(16 * tb + r, 16 * db + 4 * g, DK), acc);
    }
    // Ut and Kh^T feed only the forward scan: a backward that reads the
    // forward's saved states passes them null (a kernel argument: uniform)
    if (a.UtT) {
        __syncthreads();  // every wave has its T1 rows: V takes T's place
        store_rows<E, BLK, DV, PV, NT>(vx, Vs);
        __syncthreads();
        // Ut = T1 V, stored negated as fp32 -Ut^T (tiled)
        float* Uout = a.UtT + chunk * BLK * DV;
#pragma unroll
        for (int tile = w8; tile < 4 * (DV / 16); tile += 8) {
            const int tb = tbw, vb = tile / 4;
            f32x4 acc = zero4();
#pragma unroll
            for (int j = 0; j < 2; ++j) mma2(acc, t1[j], ldfrag_tr(Vs, PV, 32 * j, 16 * vb, l));
            *(f32x4*)(Uout + toff<float>(16 * vb + r, 16 * tb + 4 * g, BLK)) = -acc;
        }
    }
    if (a.KhT) {
        // Kh^T[d][t] = K[t][d] e^{b_C[d] - b_t[d]} (tiled, hi/lo pair), fragment (db, j)
        E* KhT = a.KhT + chunk * BLK * DK;
        E* KhTl = a.KhT_lo + chunk * BLK * DK;
#pragma unroll
        for (int f = w8; f < 2 * ND; f += 8) {
            const int db = f >> 1, j = f & 1;
            const Frag2<E> x = frag_col_decay2(Ks, PK, Bs, PB, 16 * db, 32 * j, bC, -1.f, 0, BLK);
            st_fragT(KhT, f, l, x.hi);
            if constexpr (sizeof(E) == 2) st_fragT(KhTl, f, l, x.lo);
        }
    }
}

}  // namespace clr
