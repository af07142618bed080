// gdn_kernels.h -- Gated DeltaNet chunk-forward kernels on gfx950 (shared by
// the forward and by the backward, which recomputes the forward).
//
// The layer (key-major state S in R^{dk x dv}):
//   S_t = alpha_t (I - beta_t k_t k_t^T) S_{t-1} + beta_t k_t v_t^T,  o_t = S_t^T q_t,
// i.e. the scalar-plus-low-rank transition of the StateFlow paper ("StateFlow:
// Sequence Pipeline Parallelism for Long-Context Modeling with Linear
// Recurrence", Sec. 2.1, Eq. 1), run in the chunkwise Pre / ST / Out split of
// its Sec. 2.2 (Eq. 2) over 64-token blocks:
//
//   prep  (Pre, parallel over blocks):  gamma = cumsum(g), the UT transform
//         T = (I + Diag(beta) strict_lower(K K^T * G))^-1 and the WY pair
//         W = T Diag(beta Gam) K, Ut = T Diag(beta) V   (Gam = exp(gamma),
//         G[r,s] = exp(gamma_r - gamma_s)); also K^T.
//   scan  (ST, sequential over blocks, parallel over heads x 16-wide value
//         slices): h_n = S;  U_n = Ut_n - W_n S;  S <- Gam_C S + K_n^T (e * U_n),
//         e_t = exp(gamma_C - gamma_t)  (so S_C gains Kh^T U, Kh = Diag(e) K).
//   out   (Out, parallel over blocks):  O = Diag(Gam) Q h_n + (Q K^T * G * tril) U_n.
//
// U_n is the delta rule's "new value" V^new of Eq. 2.  Every per-block matrix
// in the workspace (W, K^T, Ut^T, the saved states, U^T) is kept in the tiled
// fragment-major layout of clr_device.h, so that each wave moves whole 1-KB
// runs straight into (or out of) matrix-core fragments.
//
// Precision.  Inputs, W, K^T and the saved states h_n are in the input type;
// T, Ut and U are fp32, and enter bf16 products as hi/lo pairs (split
// operands, clr_device.h).  With repeated keys and beta near 1 the writes of
// one key within a block nearly cancel (U telescopes), so one bf16 rounding of
// T, Ut or U per token grows in the sums over tokens; and a rounded decayed key
// Diag(e) K would add components outside the span of the keys, which a state
// that hardly decays keeps.  The scan therefore multiplies the exact keys by
// the fp32 e * U, and rounds nothing that T multiplies to a single bf16.  The
// U that the output kernel and the block adjoints read (products that do not
// feed the state) is stored in the input type, and so are the backward's
// dS-independent terms R and dvloc, each added once per block.
#pragma once

#include <type_traits>

#include "clr_kernels.h"
#include "clr_ring.h"

namespace clr {

// LDS row pitch (elements) of a 64-token-wide transposed tile.
constexpr int PT = BLK + 8;

// ---------------------------------------------------------------------------
// Unit-lower-triangular inverse T = (I + A)^-1 of a 64 x 64 fp32 matrix A
// (strictly lower) held in LDS with row pitch AP, on the fp32 matrix cores.
//
// 16 x 16 products: mma16(acc, a, b) with a = A[r][4g + j] and b = B[4g + j][r]
// (j = 0..3), i.e. `a` is the accumulator tile of A^T and `b` that of B.
//
//  1. Wave w inverts its diagonal block N = A_ww (nilpotent, N^16 = 0) by
//     doubling: (I + N)^-1 = (I - N)(I + N^2)(I + N^4)(I + N^8), exactly.
//  2. Wave w then forms its column block: T_iw = -T_ii sum_{k=w}^{i-1} A_ik T_kw
//     for i = w+1..3, keeping T_kw in registers.
// Requires 256 threads.  Td is LDS scratch of 4 x 16 x 16 floats.  Returns
// in tiles[i] the accumulator tile T[16 i + 4 g + .][16 w + r].
// ---------------------------------------------------------------------------
constexpr int AP = BLK + 4;  // row pitch of the fp32 64 x 64 LDS matrices

__device__ __forceinline__ void mma16f(f32x4& acc, f32x4 a, f32x4 b) {
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a[0], b[0], acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a[1], b[1], acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a[2], b[2], acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a[3], b[3], acc, 0, 0, 0);
}

__device__ inline void tri_inverse_cols(const float* Am, float* Td, f32x4 (&tiles)[4]) {
    const int tid = threadIdx.x, w = tid >> 6, l = tid & 63, r = l & 15, g = l >> 4;
    const int o = 16 * w;
    // N = A_ww as tiles of N (rows 4g+i, col r) and of N^T
    f32x4 N, NT;
#pragma unroll
    for (int i = 0; i < 4; ++i) N[i] = Am[(o + 4 * g + i) * AP + o + r];
    NT = *(const f32x4*)(Am + (o + r) * AP + o + 4 * g);
    f32x4 N2 = zero4(), N2T = zero4(), N4 = zero4(), N4T = zero4(), N8 = zero4();
    mma16f(N2, NT, N);
    mma16f(N2T, N, NT);
    mma16f(N4, N2T, N2);
    mma16f(N4T, N2, N2T);
    mma16f(N8, N4T, N4);
    f32x4 Y = N8;
#pragma unroll
    for (int i = 0; i < 4; ++i)
        if (4 * g + i == r) Y[i] += 1.f;
    mma16f(Y, N4T, Y);   // (I + N^4)(I + N^8)
    mma16f(Y, N2T, Y);   // (I + N^2)(...)
    mma16f(Y, -NT, Y);   // (I - N)(...)
    // diagonal block to LDS (row-major 16 x 16) for the other waves
#pragma unroll
    for (int i = 0; i < 4; ++i) Td[w * 256 + (4 * g + i) * 16 + r] = Y[i];
    // (loops fully unrolled so the tiles stay in registers; w is wave-uniform)
#pragma unroll
    for (int i = 0; i < 4; ++i) tiles[i] = (i == w) ? Y : zero4();
    __syncthreads();
#pragma unroll
    for (int i = 1; i < 4; ++i) {
        if (i > w) {
            f32x4 X = zero4();
#pragma unroll
            for (int k = 0; k < 3; ++k) {
                if (k >= w && k < i) {
                    const f32x4 a = *(const f32x4*)(Am + (16 * i + r) * AP + 16 * k + 4 * g);  // A_ik^T tile
                    mma16f(X, a, tiles[k]);
                }
            }
            const f32x4 tii = *(const f32x4*)(Td + i * 256 + r * 16 + 4 * g);  // T_ii^T tile
            f32x4 Tiw = zero4();
            mma16f(Tiw, -tii, X);
            tiles[i] = Tiw;
        }
    }
}

// Transposed staging of an R x CC tile (row stride ld elements in global
// memory) into LDS dst[CC][DP]:  dst[c][r] = src[r][c].  Rows r >= nvalid
// (tokens past the end of the sequence) are staged as zeros.
// With PERM the source columns are in fragment-packed order and are restored
// to natural order in dst.
template <typename E, int R, int CC, int DP, bool PERM = false>
__device__ void stage_T(const E* __restrict__ src, size_t ld, E* dst, int nvalid) {
    constexpr int VEC = 16 / sizeof(E);  // elements per 16-byte load
    constexpr int PER_ROW = CC / VEC;
    for (int idx = threadIdx.x; idx < R * PER_ROW; idx += blockDim.x) {
        const int t = idx / PER_ROW, cb = idx % PER_ROW;
        E tmp[VEC];
        if (t < nvalid) *(uint4*)tmp = *(const uint4*)(src + (size_t)t * ld + cb * VEC);
        else *(uint4*)tmp = uint4{0u, 0u, 0u, 0u};
#pragma unroll
        for (int ii = 0; ii < VEC; ++ii) {
            const int i = (ii + cb) % VEC;  // rotate to spread LDS banks
            const int c = PERM ? kunperm(cb * VEC + i) : cb * VEC + i;
            dst[c * DP + t] = tmp[i];
        }
    }
}
// 64-token x D token-major tile -> dst[D][PT] (token index contiguous).
template <typename E, int D>
__device__ void stage_transposed(const E* __restrict__ src, size_t ld, E* dst, int nvalid) {
    stage_T<E, BLK, D, PT>(src, ld, dst, nvalid);
}

// Row pitch (elements) of a row-major LDS tile with D columns: keeps rows
// 16-byte aligned and spreads consecutive rows over the LDS banks.
template <typename E, int D> constexpr int RP = D + 16 / (int)sizeof(E);

// Scale element i of a fragment whose k index runs over k0 + kmap(g, i) by s[k].
__device__ __forceinline__ void frag_scale_k(Frag<bf16>& x, const float* s, int k0, int g) {
#pragma unroll
    for (int i = 0; i < 8; ++i) x.v[i] = (bf16)((float)x.v[i] * s[k0 + (i < 4 ? 4 * g + i : 16 + 4 * g + i - 4)]);
}
__device__ __forceinline__ void frag_scale_k(Frag<float>& x, const float* s, int k0, int g) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        x.lo[i] *= s[k0 + 4 * g + i];
        x.hi[i] *= s[k0 + 16 + 4 * g + i];
    }
}
__device__ __forceinline__ void st_fragT(bf16* base, int f, int l, const Frag<bf16>& x) {
    *(bf16x8*)(base + ((size_t)f * 64 + l) * 8) = x.v;
}
__device__ __forceinline__ void st_fragT(float* base, int f, int l, const Frag<float>& x) {
    *(f32x4*)(base + ((size_t)(2 * f) * 64 + l) * 4) = x.lo;
    *(f32x4*)(base + ((size_t)(2 * f + 1) * 64 + l) * 4) = x.hi;
}

// ---------------------------------------------------------------------------
// prep: one work-group (8 waves) per (block n, head h, batch b).  K and V are
// staged row-major in LDS with all loads in flight at once; products that
// contract over the token index read them transposed (ldfrag_tr).
//
// With BWD it also does the dS-independent part of the backward for the
// block (the reverse scan's operands) from the same staged tiles:
//   W^T and K (tiled),
//   dvloc = P^T dO,  P[t][s] = (q_t . k_s) exp(gamma_t - gamma_s)  (s <= t),
//   R = (Diag(Gam) Q)^T dO - W^T dvloc = Z^T dO,  Z = Diag(Gam) Q - P W,
// and writes T^T for the block adjoints.  The LDS regions of
// the first part are reused by the second:
//   [Ks | Vs -> Qs | Am -> Ws | Td | T (fp32) -> dOs],  P^T over Ks (or after
//   the last region when it does not fit there).
// ---------------------------------------------------------------------------
template <typename E, int DK, int DV> struct PrepLds {
    static constexpr int PK = RP<E, DK>, PV = RP<E, DV>;
    static constexpr size_t o_K = 0, o_V = o_K + sizeof(E) * BLK * PK;
    static constexpr size_t o_A = o_V + sizeof(E) * BLK * PV, o_Td = o_A + 4 * BLK * AP;
    static constexpr size_t o_T1 = o_Td + 4 * 1024, o_T2 = o_T1 + sizeof(E) * BLK * PT;
    static constexpr size_t end1 = o_T2 + sizeof(E) * BLK * PT;
    static constexpr bool P_OVER_K = sizeof(E) * BLK * PT <= sizeof(E) * BLK * PK;
    static constexpr size_t o_P = P_OVER_K ? o_K : end1;
    static constexpr size_t total = P_OVER_K ? end1 : end1 + sizeof(E) * BLK * PT;
    // T (fp32, row pitch AP) is kept where T1 and T2 were
    static_assert((size_t)4 * BLK * AP <= end1 - o_T1, "fp32 T fits the T1, T2 regions");
    // the backward's second part fits the regions of the first
    static constexpr bool BWD_FITS = DK == DV && sizeof(E) * BLK * PK <= 4 * BLK * AP &&
                                     sizeof(E) * BLK * PV <= 2 * sizeof(E) * BLK * PT;
};

template <typename E, int DK, int DV, bool BWD = false>
__global__ __launch_bounds__(512) void gdn_prep_kernel(GdnPrepArgs<E> a) {
    constexpr int NT = 512;
    const int n = a.n0 + blockIdx.x, h = blockIdx.y, b = blockIdx.z;
    // wave w8: row block w = w8 & 3, half hf = w8 >> 2 (the halves split the
    // Gram's column blocks and the output tiles)
    const int tid = threadIdx.x, w8 = tid >> 6, w = w8 & 3, hf = w8 >> 2, l = tid & 63, r = l & 15, g = l >> 4;
    const int T = a.T, H = a.H, NC = a.NC;
    const size_t tok0 = (size_t)b * T + (size_t)n * BLK;  // first token (b, n*64)
    const size_t chunk = ((size_t)b * H + h) * NC + n;    // workspace block index
    const int nvalid = min(BLK, T - n * BLK);             // tokens of this block inside the sequence
    using Lay = PrepLds<E, DK, DV>;
    constexpr int PK = Lay::PK, PV = Lay::PV, ND = DK / 16, KK = DK / 32;

    __shared__ __align__(16) float s_gam[BLK], s_bet[BLK], s_Gam[BLK], s_bG[BLK];
    __shared__ __align__(16) char lds[Lay::total];
    E* Ks = (E*)(lds + Lay::o_K);
    E* Vs = (E*)(lds + Lay::o_V);
    float* Am = (float*)(lds + Lay::o_A);
    float* Td = (float*)(lds + Lay::o_Td);

    const size_t ldk = (size_t)H * DK, ldv = (size_t)H * DV;
    // wave 0's gate and beta loads go out first, so that the cumsum waits for
    // them alone (rows past the end read the last valid token; selected below)
    E graw = from_f<E>(0.f), braw = from_f<E>(0.f);
    if (w8 == 0) {
        const size_t ig = (tok0 + min(l, nvalid - 1)) * H + h;
        graw = a.g[ig];
        braw = a.beta[ig];
    }
    const auto kx = load_rows<E, BLK, DK, NT>(a.k + tok0 * ldk + (size_t)h * DK, ldk, nvalid);
    const auto vx = load_rows<E, BLK, DV, NT>(a.v + tok0 * ldv + (size_t)h * DV, ldv, nvalid);
    // backward: Q and dO in flight through the Gram and inverse phases
    RowsRegs<E, BLK, DK, NT> qx;
    RowsRegs<E, BLK, DV, NT> ox;
    if constexpr (BWD) {
        qx = load_rows<E, BLK, DK, NT>(a.q + tok0 * ldk + (size_t)h * DK, ldk, nvalid);
        ox = load_rows<E, BLK, DV, NT>(a.dO + tok0 * ldv + (size_t)h * DV, ldv, nvalid);
    }
    if (w8 == 0) {
        // tokens past the end are identity steps: g = 0, beta = 0
        const float gv = l < nvalid ? to_f(graw) : 0.f;
        const float bv = l < nvalid ? to_f(braw) : 0.f;
        const float gam = wave_prefix_sum(gv);
        const float gC = __shfl(gam, BLK - 1, 64);
        s_gam[l] = gam;
        s_Gam[l] = __expf(gam);
        s_bet[l] = bv;
        a.gam[chunk * BLK + l] = gam;
        // the scans' per-token decay to the block end, and Gam_C in the last slot
        a.eg[chunk * BLK + l] = l < BLK - 1 ? __expf(gC - gam) : __expf(gC);
    }
    store_rows<E, BLK, DK, PK, NT>(kx, Ks);
    store_rows<E, BLK, DV, PV, NT>(vx, Vs);
    __syncthreads();

    // Gram block row w: A[r][s] = beta_r exp(gamma_r - gamma_s) (k_r . k_s), s < r
    // (column blocks j of this wave's half: j & 1 == hf)
    {
        Frag<E> fa[KK];
#pragma unroll
        for (int kk = 0; kk < KK; ++kk) fa[kk] = ldfrag(Ks + (16 * w + r) * PK + 32 * kk + 4 * g);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            if ((j & 1) != hf) continue;
            f32x4 acc = zero4();
            if (j <= w) {
#pragma unroll
                for (int kk = 0; kk < KK; ++kk) mma(acc, fa[kk], ldfrag(Ks + (16 * j + r) * PK + 32 * kk + 4 * g));
            }
            // D tile rows = 16w + 4g + i (r index "row"), cols = 16j + r (s index)
            f32x4 kkg;
            const f32x4 gr = ld4_now(s_gam + 16 * w + 4 * g), br = ld4_now(s_bet + 16 * w + 4 * g);
            const float gc = s_gam[16 * j + r];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int row = 16 * w + 4 * g + i, col = 16 * j + r;
                kkg[i] = col < row ? acc[i] * __expf(gr[i] - gc) : 0.f;
                Am[row * AP + col] = br[i] * kkg[i];
            }
        }
    }
    __syncthreads();
    float* Tm = (float*)(lds + Lay::o_T1);  // T, fp32, row pitch AP
    if (hf == 0) {
        // T = (I + A)^-1 on waves 0..3; wave w holds column block w
        f32x4 tc[4];
        tri_inverse_cols(Am, Td, tc);  // one barrier inside
        const int s = 16 * w + r;
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int ii = 0; ii < 4; ++ii) Tm[(16 * i + 4 * g + ii) * AP + s] = tc[i][ii];
        // T^T[s][t] (tiled) for the backward's block adjoints
        if (a.TT) {
#pragma unroll
            for (int i = 0; i < 4; ++i) st4(a.TT + chunk * BLK * BLK + toff<E>(s, 16 * i + 4 * g, BLK), tc[i]);
        }
        if (w8 == 0) s_bG[l] = s_bet[l] * s_Gam[l];
    } else {
        __syncthreads();  // matches the barrier inside tri_inverse_cols
    }
    __syncthreads();

    // Row fragment (m = t, k = s) of T Diag(c): fp32, scaled, split
    auto tfrag = [&](int t, int k0, const float* c) {
        const float* p = Tm + t * AP + k0 + 4 * g;
        return split8<E>(ld4(p) * ld4_now(c + k0 + 4 * g), ld4(p + 16) * ld4_now(c + k0 + 16 + 4 * g));
    };
    // W^T[d][t] = sum_s K^T[d][s] (T Diag(beta Gam))[t][s]  -> stored as W[t][d] (tiled);
    // backward also row-major in LDS (Ws, where Am was)
    E* Wout = a.W + chunk * BLK * DK;
    E* Ws = (E*)(lds + Lay::o_A);
    // a wave's tiles below all lie in token block w8 & 3 (tile & 3 and tile % 4
    // with tile = w8 + 8i), so its split T rows are formed once per loop
    const int tbw = w8 & 3;
    const Frag2<E> tw[2] = {tfrag(16 * tbw + r, 0, s_bG), tfrag(16 * tbw + r, 32, s_bG)};
#pragma unroll
    for (int tile = w8; tile < ND * 4; tile += 8) {
        const int db = tile >> 2, tb = tbw;
        f32x4 acc = zero4();
#pragma unroll
        for (int j = 0; j < 2; ++j) mma2(acc, ldfrag_tr(Ks, PK, 32 * j, 16 * db, l), tw[j]);
        if (a.W) st4(Wout + toff<E>(16 * tb + r, 16 * db + 4 * g, DK), acc);
        if constexpr (BWD) st4(Ws + (16 * tb + r) * PK + 16 * db + 4 * g, acc);
    }
    // Ut[t][v] = sum_s (T Diag(beta))[t][s] V[s][v]  -> stored negated as fp32 -Ut^T[v][t]
    // (tiled), so that the scan forms -U = W S - Ut by accumulating onto it
    // (the forward scan's operands W, Ut and K^T are not written for a
    // backward that reads saved states: a null W, UtT, KhT)
    float* Uout = a.UtT + chunk * BLK * DV;
    if (a.UtT) {
        const Frag2<E> tu[2] = {tfrag(16 * tbw + r, 0, s_bet), tfrag(16 * tbw + r, 32, s_bet)};
#pragma unroll
        for (int tile = w8; tile < 4 * (DV / 16); tile += 8) {
            const int tb = tbw, vb = tile / 4;
            f32x4 acc = zero4();
#pragma unroll
            for (int j = 0; j < 2; ++j) mma2(acc, tu[j], ldfrag_tr(Vs, PV, 32 * j, 16 * vb, l));
            *(f32x4*)(Uout + toff<float>(16 * vb + r, 16 * tb + 4 * g, BLK)) = -acc;
        }
    }
    // K^T[d][t] (tiled): its fragment (db, j) is the B fragment of K over tokens
    // 32j.., columns 16db..  (the decay exp(gamma_C - gamma_t) is applied to U
    // in the scan, so the keys are stored exactly)
    E* KTout = a.KhT + chunk * BLK * DK;
    if (a.KhT) {
#pragma unroll
        for (int f = w8; f < 2 * ND; f += 8) st_fragT(KTout, f, l, ldfrag_tr(Ks, PK, 32 * (f & 1), 16 * (f >> 1), l));
    }
    if constexpr (BWD) {
        static_assert(Lay::BWD_FITS, "Q where V was, W where Am was, dO where T1, T2 were");
        constexpr int PQ = PK, PO = PV, NVB = DV / 16;
        E* Qs = (E*)(lds + Lay::o_V);
        E* dOs = (E*)(lds + Lay::o_T1);
        E* PsT = (E*)(lds + Lay::o_P);
        __syncthreads();  // V, T1, T2 no longer read: Q and dO take their places
        store_rows<E, BLK, DK, PQ, NT>(qx, Qs);
        store_rows<E, BLK, DV, PO, NT>(ox, dOs);
        __syncthreads();
        // W^T (tiled; A: m = d, k = t) and Kh (tiled; A: m = t, k = d): fragments (w, kk)
        E* WT = a.WT + chunk * BLK * DK;
#pragma unroll
        for (int f = w8; f < 2 * ND; f += 8) st_fragT(WT, f, l, ldfrag_tr(Ws, PQ, 32 * (f & 1), 16 * (f >> 1), l));
        const int s = 16 * w + r;
        Frag<E> fk[KK];
#pragma unroll
        for (int kk = 0; kk < KK; ++kk) fk[kk] = ldfrag(Ks + s * PK + 32 * kk + 4 * g);
        {
            // K, exact (the reverse scan applies exp(gamma_C - gamma_t) to K dS)
            E* Kt = a.Kh + chunk * BLK * DK;
#pragma unroll
            for (int kk = 0; kk < KK; ++kk) {
                if ((kk & 1) != hf) continue;  // static indices: fk stays in registers
                st_fragT(Kt, w * KK + kk, l, fk[kk]);
            }
        }
        // P[tb][w] (rows t, cols s = 16w + r), s <= t; both halves form the same tiles
        f32x4 P[4];
        const float gs = s_gam[s];
#pragma unroll
        for (int tb = 0; tb < 4; ++tb) {
            f32x4 acc = zero4();
            if (tb >= w) {
#pragma unroll
                for (int kk = 0; kk < KK; ++kk) mma(acc, ldfrag(Qs + (16 * tb + r) * PQ + 32 * kk + 4 * g), fk[kk]);
                const f32x4 gt = ld4_now(s_gam + 16 * tb + 4 * g);
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int t = 16 * tb + 4 * g + i;
                    acc[i] = (s <= t) ? acc[i] * __expf(gt[i] - gs) : 0.f;
                }
            }
            P[tb] = acc;
        }
        // dvloc^T[v][s] = sum_t P[t][s] dO[t][v] (this half's value blocks)
        Frag<E> fp[2];
        fp[0] = frag_from_acc<E>(P[0], P[1]);
        fp[1] = frag_from_acc<E>(P[2], P[3]);
        E* dvlT = a.dvlT + chunk * BLK * DV;  // the reverse scan adds it to dU in fp32
#pragma unroll
        for (int vb = hf; vb < NVB; vb += 2) {
            f32x4 acc = zero4();
#pragma unroll
            for (int j = 0; j < 2; ++j) mma(acc, fp[j], ldfrag_tr(dOs, PO, 32 * j, 16 * vb, l));
            st4(dvlT + toff<E>(16 * vb + r, 16 * w + 4 * g, BLK), acc);
        }
        __syncthreads();  // K no longer read: P^T may take its place
        if (hf == 0) {
#pragma unroll
            for (int tb = 0; tb < 4; ++tb) st4(PsT + s * PT + 16 * tb + 4 * g, P[tb]);
        }
        __syncthreads();
        // Z = Diag(Gam) Q - P W in place of Q: tiles (tb, db), rows t = 16tb + 4g + i, column d = 16db + r
        // (a wave's tiles share token block w8 & 3: its P^T operands are read once)
        const Frag<E> pz[2] = {ldfrag_tr(PsT, PT, 0, 16 * tbw, l), ldfrag_tr(PsT, PT, 32, 16 * tbw, l)};
#pragma unroll
        for (int tile = w8; tile < 4 * ND; tile += 8) {
            const int tb = tbw, db = tile >> 2;
            f32x4 acc = zero4();
#pragma unroll
            for (int j = 0; j < 2; ++j) mma(acc, pz[j], ldfrag_tr(Ws, PQ, 32 * j, 16 * db, l));
            const f32x4 Gt = ld4_now(s_Gam + 16 * tb + 4 * g);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                E& q = Qs[(16 * tb + 4 * g + i) * PQ + 16 * db + r];
                q = from_f<E>(Gt[i] * to_f(q) - acc[i]);
            }
        }
        __syncthreads();
        // R[d][v] = sum_t Z[t][d] dO[t][v]   (fp32, accumulator-tiled)
        E* Rt = a.Rt + chunk * DK * DV;
        // (a wave's tiles share d-block w8 % ND, ND dividing 8: its Z^T operands are read once)
        static_assert(8 % ND == 0, "d-block per wave");
        const int dbw = w8 % ND;
        const Frag<E> zq[2] = {ldfrag_tr(Qs, PQ, 0, 16 * dbw, l), ldfrag_tr(Qs, PQ, 32, 16 * dbw, l)};
        for (int tile = w8; tile < ND * NVB; tile += 8) {
            const int db = dbw, vb = tile / ND;
            f32x4 acc = zero4();
#pragma unroll
            for (int j = 0; j < 2; ++j) mma(acc, zq[j], ldfrag_tr(dOs, PO, 32 * j, 16 * vb, l));
            st4(Rt + atoff(db, vb, DK, l), acc);
        }
    }
}

// ---------------------------------------------------------------------------
// scan: one work-group per (16-wide value slice, head, batch), sequential over
// the blocks.  The fp32 state slice S[0:DK][v0:v0+16] lives in accumulator
// tiles of the consumer wave.  Writes the state entering each block and U_n^T.
// ---------------------------------------------------------------------------
// The scans keep Ut and dU in fp32 (see "Precision" above).  The
// Gated DeltaNet scans multiply the exact keys by e * U; KDA's (per-channel
// decay, PCD) multiply the decayed keys, streamed as a bf16 hi/lo pair.
template <bool PCD, typename E> using ScanWsT = float;
// Factor of the key units in a ring slot: two for the KDA pair (bf16 only).
template <bool PCD, typename E> constexpr int key_parts() { return PCD && sizeof(E) == 2 ? 2 : 1; }

// Consumer waves per scan work-group (NCW).  With two (bf16, dk >= 64, where
// each takes whole 32-row fragments of the key dimension) consumer c keeps
// the state rows [c dk/2, (c+1) dk/2) of the slice and forms its half of each
// contraction over d; the two partial sums meet in LDS (one more work-group
// barrier per block), so a block's matrix-core chain runs on two SIMDs
// instead of one.  Where that chain bounds the scan (the Gated DeltaNet pair
// scan: 42.2 -> 35.4 us per 2048-token chunk at H = 16) two are used; where
// the operand stream does (the Gated DeltaNet forward scan: 28.5 -> 30.2 us
// with two), or the extra barrier costs more than it saves (KDA's scans:
// 51 -> 66 us and 64 -> 69 us), one.
template <typename E, int DK> constexpr bool scan_can_split() { return sizeof(E) == 2 && DK >= 64; }

template <typename E, int DK, typename UE = E, int NCW = 1> struct ScanFwdOps {
    Frag<E> w[4][DK / 32 / NCW];   // W rows (A: m = t, k = d), this consumer's key range
    Frag<E> kh[DK / 16 / NCW][2];  // K^T (GDN) or Kh^T (KDA, hi half) rows (A: m = d, k = t), same range
    Frag<E> kl[DK / 16 / NCW][2];  // KDA: lo half of Kh^T
    Frag<UE> ut[2];           // -Ut^T[v0 + r][token pair-tiles 2j, 2j+1] (accumulator layout)
    float GC;                 // GDN: Gam_C = exp(gamma_C), from the small unit
};

// Store ROWS x 16 accumulator tiles (rows 16 rb + 4 g + i, column c0 + r)
// into a row-major matrix with row stride ld, staged through LDS
// (tile[ROWS][16]) so that each lane writes whole 16-byte row pieces instead
// of scattered elements.
template <typename E, int ROWS>
__device__ __forceinline__ void store_rows16(E* dst, size_t ld, const f32x4 (&X)[ROWS / 16], E* tile, int c0, int r,
                                             int g, int nrows = ROWS) {
    const int l = 16 * g + r;
#pragma unroll
    for (int rb = 0; rb < ROWS / 16; ++rb)
#pragma unroll
        for (int i = 0; i < 4; ++i) tile[(16 * rb + 4 * g + i) * 16 + r] = from_f<E>(X[rb][i]);
    // only this wave uses the tile; LDS operations of one wave execute in order
    asm volatile("" ::: "memory");
    constexpr int VEC = 16 / sizeof(E), PER_ROW = 16 / VEC;
#pragma unroll
    for (int c = l; c < ROWS * PER_ROW; c += 64) {
        const int d = c / PER_ROW, part = c % PER_ROW;
        if (d < nrows) *(uint4*)(dst + (size_t)d * ld + c0 + part * VEC) = *(const uint4*)(tile + d * 16 + part * VEC);
    }
    asm volatile("" ::: "memory");
}

// Store a state slice (accumulator tiles: rows d = 16 db + 4g + i, column
// v0 + r) into the tiled key-major h[d][v] (R = DK, C = DV).  A lane's values
// belong to four different lane units of that layout, so the slice has to be
// transposed; two ways follow.
// Without LDS: fs[kk] (the state's B fragment over rows 32kk.., from
// frag_from_acc) is also the A fragment of the state's transpose; its product
// with the 32 x 16 selector [I; 0] (half 0) or [0; I] (half 1) is the
// transposed tile of rows 32kk + 16 half.., in which lane (r, g) holds
// S[32kk + 16 half + r][v0 + 4g + i], i < 4: exactly this lane's four elements
// of the tiled h fragment.  Each product has one nonzero term, so the stored
// values are the bf16-rounded state.
template <typename E> __device__ __forceinline__ Frag<E> state_sel(int half, int l);
template <> __device__ __forceinline__ Frag<bf16> state_sel<bf16>(int half, int l) {
    const int r = l & 15, g = l >> 4;
    Frag<bf16> f;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const int k = i < 4 ? 4 * g + i : 16 + 4 * g + (i - 4);
        f.v[i] = (bf16)(k == r + 16 * half ? 1.f : 0.f);
    }
    return f;
}
template <> __device__ __forceinline__ Frag<float> state_sel<float>(int half, int l) {
    const int r = l & 15, g = l >> 4;
    Frag<float> f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        f.lo[i] = (half == 0 && 4 * g + i == r) ? 1.f : 0.f;
        f.hi[i] = (half == 1 && 4 * g + i == r) ? 1.f : 0.f;
    }
    return f;
}
template <typename E, int DK, int DV, int C = 0, int NCW = 1>
__device__ __forceinline__ void store_state_sel(E* h, const Frag<E> (&fs)[DK / 32 / NCW], int v0, int l) {
    const int r = l & 15, g = l >> 4;
    const Frag<E> sel[2] = {state_sel<E>(0, l), state_sel<E>(1, l)};
#pragma unroll
    for (int kk = 0; kk < DK / 32 / NCW; ++kk)
#pragma unroll
        for (int half = 0; half < 2; ++half) {
            f32x4 c = zero4();
            mma(c, fs[kk], sel[half]);
            E* dst = h + toff<E>(32 * (C * (DK / 32 / NCW) + kk) + 16 * half + r, v0 + 4 * g, DV);
            if constexpr (sizeof(E) == 2) *(bf16x4*)dst = bf16x4{(bf16)c[0], (bf16)c[1], (bf16)c[2], (bf16)c[3]};
            else *(f32x4*)dst = c;
        }
}

// Through LDS (bf16), a wave-private tile T[16 v][DK + 8]:
// each lane writes the two bf16x4 halves of fs[kk] (four consecutive rows d
// of its column v0 + r) as 8-byte runs of row r, and reads back with the
// transposing LDS read, which hands lane (r, g) T[4g + i][16 db + r] =
// S[16 db + r][v0 + 4g + i]: its four elements of the tiled h fragment.  Eight
// 8-byte writes and eight transposing reads per block, no matrix-core work on
// the recurrence's chain; fp32 states take the selector path.  Measured per
// 2048-token chunk: with three producer waves (KDA's scans) this path is the
// faster one for both halves of the pair scan (42.2 -> 39.2 us); with seven
// (the Gated DeltaNet pair, whose producers keep LDS busier) it is for the
// recompute's h (29.1 -> 28.1 us) but not for the reverse scan's dh, where
// the selector products are (both halves through LDS: 31.5 us).
// state_store() picks accordingly.
constexpr int state_tile_bytes(int dk, int es) { return 16 * (dk + 8) * es; }
// With two consumers (C, NCW = 2) each writes and reads back the columns of
// its own key range of the shared tile.
// The two halves of that store, for a wave that writes the tile and another
// that reads it back: the row writes of this consumer's key range ...
template <int DK, int C = 0, int NCW = 1>
__device__ __forceinline__ void state_tile_write(const Frag<bf16> (&fs)[DK / 32 / NCW], bf16* tile, int l) {
    constexpr int PS = DK + 8, KKC = DK / 32 / NCW;
    const int r = l & 15, g = l >> 4;
#pragma unroll
    for (int kk = 0; kk < KKC; ++kk) {
        const bf16x8 v = fs[kk].v;
        const int c0 = 32 * (C * KKC + kk);
        *(bf16x4*)(tile + r * PS + c0 + 4 * g) = bf16x4{v[0], v[1], v[2], v[3]};
        *(bf16x4*)(tile + r * PS + c0 + 16 + 4 * g) = bf16x4{v[4], v[5], v[6], v[7]};
    }
}
// ... and the transposing reads and stores of key blocks [db0, db0 + NDB)
// (any wave: the read's lane mapping is a wave's).
template <int DK, int DV, int NDB>
__device__ __forceinline__ void state_tile_readout(bf16* h, const bf16* tile, int db0, int v0, int l) {
    constexpr int PS = DK + 8;
    const int r = l & 15, g = l >> 4, j = (l >> 2) & 3, q = l & 3;
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
        const int d0 = 16 * (db0 + db);
        const bf16x4 x = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(tile + (4 * g + j) * PS + d0 + 4 * q));
        *(bf16x4*)(h + toff<bf16>(d0 + r, v0 + 4 * g, DV)) = x;
    }
}

template <typename E, int DK, int DV, int C = 0, int NCW = 1>
__device__ __forceinline__ void store_state_tr(E* h, const Frag<E> (&fs)[DK / 32 / NCW], E* tile, int v0, int l) {
    if constexpr (sizeof(E) == 2) {
        constexpr int NDC = DK / 16 / NCW;
        state_tile_write<DK, C, NCW>(fs, tile, l);
        // LDS operations of one wave complete in order
        asm volatile("" ::: "memory");
        state_tile_readout<DK, DV, NDC>(h, tile, C * NDC, v0, l);
        asm volatile("" ::: "memory");
    } else {
        static_assert(NCW == 1, "fp32 states run with one consumer");
        store_state_sel<E, DK, DV>(h, fs, v0, l);
    }
}

template <typename E, int DK, int DV, bool VIA_LDS, int C = 0, int NCW = 1>
__device__ __forceinline__ void state_store(E* h, const Frag<E> (&fs)[DK / 32 / NCW], E* tile, int v0, int l) {
    if constexpr (VIA_LDS) store_state_tr<E, DK, DV, C, NCW>(h, fs, tile, v0, l);
    else store_state_sel<E, DK, DV, C, NCW>(h, fs, v0, l);
}

// One block of the recurrence.  HNAT selects the layout of the saved states:
// false -> tiled h^T[v][d] (read by the forward's out kernel), true -> tiled
// h[d][v] (read by the backward).  Consumer C of NCW holds the state rows
// 16 db of its key range (db = C ND/NCW ..), and the operands of that range.
template <typename E, int DK, int NU, typename UE, int KP = 1, int C = 0, int NCW = 1>
__device__ __forceinline__ void scan_fwd_from_ring_kh(ScanFwdOps<E, DK, UE, NCW>& o, const char* slot, int l);

// The two consumers' partial sums X[4] (accumulator tiles over the 64 tokens)
// of a contraction over their key halves, added in one fixed order so that
// both hold the same values.  Both write, wait for their LDS writes, meet at
// the work-group barrier (the producers take part in it), and read.
template <int C>
__device__ __forceinline__ void consumers_exchange(f32x4 (&X)[4], f32x4* xch, int l) {
#pragma unroll
    for (int tb = 0; tb < 4; ++tb) xch[(4 * C + tb) * 64 + l] = X[tb];
    __builtin_amdgcn_s_waitcnt(lgkmcnt0_imm());
    ring_barrier();
#pragma unroll
    for (int tb = 0; tb < 4; ++tb) {
        const f32x4 other = xch[(4 * (1 - C) + tb) * 64 + l];
        X[tb] = C == 0 ? X[tb] + other : other + X[tb];
    }
}

template <typename E, int DK, int DV, bool HNAT, int NU, bool PCD = false, int C = 0, int NCW = 1, bool HTILE = false>
__device__ __forceinline__ void scan_fwd_step(ScanFwdOps<E, DK, ScanWsT<PCD, E>, NCW>& o, f32x4 (&S)[DK / 16 / NCW],
                                              const GdnScanArgs<E>& a, size_t chunk, int vb, int l, E* tile,
                                              const char* slot, f32x4* xch) {
    constexpr int KK = DK / 32, NDC = DK / 16 / NCW, KKC = KK / NCW;
    using UE = ScanWsT<PCD, E>;
    Frag<E> fs[KKC];
#pragma unroll
    for (int kk = 0; kk < KKC; ++kk) fs[kk] = frag_from_acc<E>(S[2 * kk], S[2 * kk + 1]);
    // state entering block n (this consumer's rows)
    if (a.hT) {
        E* hT = a.hT + chunk * DK * DV;
        if constexpr (HNAT) {
            // through LDS (Gated DeltaNet), by selector products (KDA, whose
            // slots need all of the LDS)
            state_store<E, DK, DV, !PCD, C, NCW>(hT, fs, tile, 16 * vb, l);
        } else {
#pragma unroll
            for (int kk = 0; kk < KKC; ++kk) st8T(hT, vb * KK + C * KKC + kk, l, S[2 * kk], S[2 * kk + 1]);
        }
    }
    // a forward that saves its states: the same state operand also in the
    // backward's layout (the values the backward's recompute stores), through
    // the wave's LDS tile where the work-group has one (HTILE)
    if (a.hN) state_store<E, DK, DV, HTILE, C, NCW>(a.hN + chunk * DK * DV, fs, tile, 16 * vb, l);

    // -U = W S - Ut, accumulated onto the stored -Ut  (tiles: rows t = 16tb + 4g + i, col v0 + r);
    // with two consumers each forms W S over its key half, the first onto -Ut
    f32x4 U[4];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
        U[2 * j] = C == 0 ? o.ut[j].lo : zero4();
        U[2 * j + 1] = C == 0 ? o.ut[j].hi : zero4();
    }
#pragma unroll
    for (int tb = 0; tb < 4; ++tb) {
#pragma unroll
        for (int kk = 0; kk < KKC; ++kk) mma(U[tb], o.w[tb][kk], fs[kk]);
    }
    // the Kh^T reads go out while the products above run
    asm volatile("" ::: "memory");
    scan_fwd_from_ring_kh<E, DK, NU, UE, key_parts<PCD, E>(), C, NCW>(o, slot, l);
    if constexpr (NCW == 2) consumers_exchange<C>(U, xch, l);
#pragma unroll
    for (int tb = 0; tb < 4; ++tb) U[tb] = -U[tb];
    // U^T tiled (R = DV, C = BLK): fragment (vb, j) is this pair of tiles (consumer j stores it),
    // in the element type (read by the output kernel and the block adjoints, not by the state)
    if (a.UT) {
        E* UT = (E*)a.UT + chunk * BLK * DV;
#pragma unroll
        for (int j = 0; j < 2; ++j)
            if (NCW == 1 || j == C) st8T(UT, 2 * vb + j, l, U[2 * j], U[2 * j + 1]);
    }
    if (PCD && C == 0 && a.Utok) {
        // U token-major for the output kernel (rows of valid tokens), staged
        // in the slot's W units: the W S products above have read them, and
        // the producers refill this slot only in a later round
        const size_t bh = chunk / a.NC;
        const int n = (int)(chunk % a.NC), bb = (int)(bh / a.H), hh = (int)(bh % a.H);
        const size_t ldv = (size_t)a.H * DV;
        E* dst = a.Utok + ((size_t)bb * a.T + (size_t)n * BLK) * ldv + (size_t)hh * DV;
        store_rows16<E, BLK>(dst, ldv, U, (E*)slot, 16 * vb, l & 15, l >> 4, min(BLK, a.T - n * BLK));
    }
    if constexpr (PCD) {
        // S <- Diag(exp(b_C)) S + Kh^T U (KDA: row d of S scaled by its own
        // channel's factor, from the slot's last unit); Kh and U both split
        Frag2<E> fu[2];
        fu[0] = split_acc<E>(U[0], U[1]);
        fu[1] = split_acc<E>(U[2], U[3]);
        const float* ecs = (const float*)(slot + (NU - 1) * RING_UNIT) + 4 * (l >> 4);
#pragma unroll
        for (int db = 0; db < NDC; ++db) {
            f32x4 acc = S[db] * *(const f32x4*)(ecs + 16 * (C * NDC + db));
#pragma unroll
            for (int j = 0; j < 2; ++j) mma2(acc, pair_of(o.kh[db][j], o.kl[db][j]), fu[j]);
            S[db] = acc;
        }
    } else {
        // S <- Gam_C S + K^T (e * U), e_t = exp(gamma_C - gamma_t) on the rows
        // of the U tiles (from the slot's small unit, whose last slot holds
        // Gam_C: e_63 = 1), e * U split
        const f32x4* es = (const f32x4*)(slot + NU * RING_UNIT) + (l >> 4);
#pragma unroll
        for (int tb = 0; tb < 4; ++tb) {
            f32x4 et = es[4 * tb];
            if (tb == 3) et[3] = (l >> 4) == 3 ? 1.f : et[3];
            U[tb] = U[tb] * et;
        }
        Frag2<E> fu[2];
        fu[0] = split_acc<E>(U[0], U[1]);
        fu[1] = split_acc<E>(U[2], U[3]);
#pragma unroll
        for (int db = 0; db < NDC; ++db) {
            f32x4 acc = S[db] * o.GC;
#pragma unroll
            for (int j = 0; j < 2; ++j) mma2(acc, o.kh[db][j], fu[j]);
            S[db] = acc;
        }
    }
}

// Operands of one block from a ring slot (see clr_ring.h for the layout).
template <typename E, int DK, int NU, typename UE, int KP = 1, int C = 0, int NCW = 1>
__device__ __forceinline__ void scan_fwd_from_ring(ScanFwdOps<E, DK, UE, NCW>& o, const char* slot, int l, int s = 0) {
    constexpr int KK = DK / 32, KKC = KK / NCW, NWF = 4 * KK, NKF = 2 * (DK / 16) * KP;
    // units per fragment of W / K and of Ut; Ut starts after the W and K units
    constexpr int UPF = sizeof(E) == 2 ? 1 : 2, UPFU = sizeof(UE) == 2 ? 1 : 2;
    static_assert((NWF + NKF) * UPF % UPFU == 0, "fragment alignment");
#pragma unroll
    for (int tb = 0; tb < 4; ++tb)
#pragma unroll
        for (int kk = 0; kk < KKC; ++kk) o.w[tb][kk] = ring_frag(slot, tb * KK + C * KKC + kk, l, (E*)nullptr);
    if constexpr (C == 0) {
#pragma unroll
        for (int j = 0; j < 2; ++j) o.ut[j] = ring_frag(slot, (NWF + NKF) * UPF / UPFU + 2 * s + j, l, (UE*)nullptr);
    }
    o.GC = ring_small<NU>(slot, BLK - 1);
}
// K^T (Kh^T) operands of a block (read after the W S products have been issued).
template <typename E, int DK, int NU, typename UE, int KP, int C, int NCW>
__device__ __forceinline__ void scan_fwd_from_ring_kh(ScanFwdOps<E, DK, UE, NCW>& o, const char* slot, int l) {
    constexpr int KK = DK / 32, NWF = 4 * KK, NKF = 2 * (DK / 16), NDC = DK / 16 / NCW;
#pragma unroll
    for (int db = 0; db < NDC; ++db)
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            o.kh[db][j] = ring_frag(slot, NWF + 2 * (C * NDC + db) + j, l, (E*)nullptr);
            if constexpr (KP == 2) o.kl[db][j] = ring_frag(slot, NWF + NKF + 2 * (C * NDC + db) + j, l, (E*)nullptr);
        }
}

// Work-group: the consumer waves (NCW) run the recurrence, the
// other waves stream the operands of the next blocks into the LDS ring
// (clr_ring.h).  All operands are tiled, so ring unit u of a block is the
// contiguous 1-KB run u of
// [W | K^T (Kh^T) | Ut^T fragments (vb, 0..1)]  (Ut fp32 for the Gated
// DeltaNet scans: two units per fragment); the small unit holds gamma.
// With PCD (per-channel decay, KDA) one more unit holds exp(b_C) for every key
// channel, as fp32 (256 floats, padded), and the state-store tile also
// stages U for its token-major store.
// Producer waves: the Gated DeltaNet scans stream faster with more of them
// (three -> seven with one consumer: 27 -> 20.5 us per 2048-token chunk at
// H = 16), so their work-groups fill eight waves; KDA's scans, whose
// consumer does more per block (the token-major U), keep three.
template <int NCW> constexpr int scan_np_fast = 8 - NCW;
template <int NP, int NCW> constexpr int scan_threads = 64 * (NP + NCW);

// NVS value slices per work-group (B_V = 16 NVS): the slices share the W and
// K^T units of a slot and each has its own Ut units and consumer wave.
template <typename E, int DK, int DV, bool HNAT, bool PCD = false, int NCW_ = 1, int NVS = 1> struct ScanFwdGeom {
    static_assert(NVS == 1 || (NCW_ == 1 && !HNAT && !PCD && DV % (16 * NVS) == 0), "value-slice groups");
    static constexpr int UPF = sizeof(E) == 2 ? 1 : 2;  // 1-KB units per fragment
    static constexpr int UPFU = sizeof(ScanWsT<PCD, E>) == 2 ? 1 : 2;  // ... of Ut
    static constexpr int ND = DK / 16, KK = DK / 32, NWU = 4 * KK * UPF, NKU = 2 * ND * UPF * key_parts<PCD, E>();
    static constexpr int NU = NWU + NKU + 2 * UPFU * NVS + (PCD ? 1 : 0);
    static constexpr int SLOT = RingGeom<NU>::SLOT;
    // the state-store tile (KDA stores the state without one, and stages its
    // token-major U in the slot: its slots need all of the LDS)
    // (the Gated DeltaNet forward scan of one slice keeps one too, for the
    // states a forward that saves its activations also stores in that layout)
    static constexpr int TILE = (HNAT || (NVS == 1 && sizeof(E) == 2)) && !PCD ? state_tile_bytes(DK, sizeof(E)) : 16;
    static_assert(BLK * 16 * (int)sizeof(E) <= NWU * RING_UNIT, "U staging fits the W units");
    static constexpr int NCW = NCW_;
    static_assert(NCW == 1 || (NCW == 2 && scan_can_split<E, DK>()), "consumer split");
    static constexpr int XCH = NCW == 2 ? 2 * 4 * 64 * 16 : 0;  // the consumers' exchange
    static constexpr int PF = (160 * 1024 - TILE - XCH) / SLOT;  // ring, tile, exchange within the CU's LDS
    static constexpr int P = PF > 4 ? 4 : (PF < 2 ? 2 : PF);
    static constexpr int LDS = P * SLOT + TILE + XCH;  // ring, then the state-store tile, then the exchange
};

// Consumer C of the forward scan body.
template <typename E, int DK, int DV, bool HNAT, bool PCD, int NP, int NCW, int C, int NVS = 1>
__device__ __forceinline__ void gdn_scan_fwd_consume(const GdnScanArgs<E>& a, const char* ring, E* tile, f32x4* xch,
                                                     size_t bh, int vb, int l, int s = 0) {
    using SG = ScanFwdGeom<E, DK, DV, HNAT, PCD, NCW, NVS>;
    using UT_ = ScanWsT<PCD, E>;
    constexpr int NDC = DK / 16 / NCW, NU = SG::NU, P = SG::P;
    using G = RingGeom<NU, NP>;
    const int n0 = a.n0, NB = (a.n1 < a.NC ? a.n1 : a.NC) - a.n0;
    const int r = l & 15, g = l >> 4, v0 = 16 * vb;
    f32x4 S[NDC];
    const float* Sin = a.S_in ? a.S_in + bh * DK * DV : nullptr;
#pragma unroll
    for (int db = 0; db < NDC; ++db)
#pragma unroll
        for (int i = 0; i < 4; ++i)
            S[db][i] = Sin ? Sin[(size_t)(16 * (C * NDC + db) + 4 * g + i) * DV + v0 + r] : 0.f;
    ring_barrier();
    for (int n = 0; n < NB; ++n) {
        ScanFwdOps<E, DK, UT_, NCW> o;
        const char* slot = ring + (n % P) * G::SLOT;
        scan_fwd_from_ring<E, DK, NU, UT_, key_parts<PCD, E>(), C, NCW>(o, slot, l, s);
        constexpr bool HTILE = !HNAT && NVS == 1 && !PCD && sizeof(E) == 2;  // the tile ScanFwdGeom keeps
        scan_fwd_step<E, DK, DV, HNAT, NU, PCD, C, NCW, HTILE>(o, S, a, bh * a.NC + n0 + n, vb, l, tile, slot, xch);
        ring_barrier();
    }
    if (a.S_out) {
        float* So = a.S_out + bh * DK * DV;
#pragma unroll
        for (int db = 0; db < NDC; ++db)
#pragma unroll
            for (int i = 0; i < 4; ++i) So[(size_t)(16 * (C * NDC + db) + 4 * g + i) * DV + v0 + r] = S[db][i];
    }
}

// Scan body for work-group `wgi` of the scan grid; `smem` holds
// ScanFwdGeom::LDS bytes (16-byte aligned).
template <typename E, int DK, int DV, bool HNAT, bool PCD = false, int NP = NPROD, int NCW = 1, int NVS = 1>
__device__ __forceinline__ void gdn_scan_fwd_body(const GdnScanArgs<E>& a, int wgi, char* smem) {
    const int H = a.H, NC = a.NC;
    // blocks n0 .. n0 + NB - 1 of each head are scanned (ring index j = n - n0)
    const int n0 = a.n0, NB = (a.n1 < NC ? a.n1 : NC) - a.n0;
    int b, h, vg;  // value-slice group vg: slices NVS vg .. NVS vg + NVS - 1
    if (!scan_coords(wgi, DV / 16 / NVS, a.BH, H, b, h, vg)) return;
    const int vb = NVS * vg;  // the group's first slice
    const int w = threadIdx.x >> 6, l = threadIdx.x & 63;
    using SG = ScanFwdGeom<E, DK, DV, HNAT, PCD, NCW, NVS>;
    using UT_ = ScanWsT<PCD, E>;
    constexpr int UPFU = SG::UPFU, NWU = SG::NWU, NKU = SG::NKU, NU = SG::NU, P = SG::P;
    constexpr int UE = UNIT_ELEMS<E>, LE = LANE_ELEMS<E>;
    using G = RingGeom<NU, NP>;
    char* ring = smem;
    E* tile = (E*)(smem + P * G::SLOT);
    f32x4* xch = (f32x4*)(smem + P * G::SLOT + SG::TILE);
    const size_t bh = (size_t)b * H + h;

    // lane 0's address of unit u of workspace block c (lane l reads 16 l bytes further)
    auto unit_ptr = [&](size_t c, int u) -> const char* {
        if (u < NWU) return (const char*)(a.W + c * BLK * DK + u * UE);
        if (u < NWU + NKU) {
            const int k = u - NWU;  // KDA: the lo half follows the hi half
            if (PCD && k >= NKU / 2 && key_parts<PCD, E>() == 2)
                return (const char*)(a.KhT_lo + c * BLK * DK + (k - NKU / 2) * UE);
            return (const char*)(a.KhT + c * BLK * DK + k * UE);
        }
        if (PCD && u == NU - 1) return (const char*)(a.eC + c * 256);
        return (const char*)((const UT_*)a.UtT + c * BLK * DV + (size_t)(2 * vb * UPFU) * UNIT_ELEMS<UT_> +
                             (size_t)(u - NWU - NKU) * UNIT_ELEMS<UT_>);
    };
    // lane 0's address of the small unit (4 bytes per lane)
    auto small_ptr = [&](size_t c) -> const char* {
        return PCD ? (const char*)(a.eC + c * 256) : (const char*)(a.eg + c * BLK);
    };
    const int pre = NB < P - 1 ? NB : P - 1;
    if (w >= NCW * NVS) {  // producers
        const int pid = w - NCW * NVS;
        auto issue = [&](int n) {
            const size_t c = bh * NC + n0 + n;
            auto src = [&](int u) -> const void* { return unit_ptr(c, u) + 16 * l; };
            ring_issue<NU, decltype(src), NP>(ring + (n % P) * G::SLOT, pid, src, small_ptr(c) + 4 * l);
        };
        for (int n = 0; n < pre; ++n) issue(n);
        ring_wait<G::NU_MIN>(pre - 1);  // block 0 has landed
        ring_barrier();
        for (int n = 0; n < NB; ++n) {
            if (n + P - 1 < NB) issue(n + P - 1);
            if constexpr (NCW == 2) ring_barrier();  // the consumers' exchange within block n
            const int last = (n + P - 1 < NB ? n + P - 1 : NB - 1);
            ring_wait<G::NU_MIN>(last - (n + 1));  // block n + 1 has landed
            ring_barrier();
        }
        return;
    }
    if constexpr (NVS > 1) {  // one consumer per slice of the group
        gdn_scan_fwd_consume<E, DK, DV, HNAT, PCD, NP, NCW, 0, NVS>(a, ring, tile, xch, bh, vb + w, l, w);
    } else {
        if (w == 0) gdn_scan_fwd_consume<E, DK, DV, HNAT, PCD, NP, NCW, 0>(a, ring, tile, xch, bh, vb, l);
        if constexpr (NCW == 2)
            if (w == 1) gdn_scan_fwd_consume<E, DK, DV, HNAT, PCD, NP, NCW, 1>(a, ring, tile, xch, bh, vb, l);
    }
}

template <typename E, int DK, int DV, bool HNAT, bool PCD = false, int NP = NPROD, int NVS = 1>
__global__ __launch_bounds__((scan_threads<NP, NVS>)) void gdn_scan_fwd_kernel(GdnScanArgs<E> a) {
    __shared__ __align__(16) char smem[ScanFwdGeom<E, DK, DV, HNAT, PCD, 1, NVS>::LDS];
    gdn_scan_fwd_body<E, DK, DV, HNAT, PCD, NP, 1, NVS>(a, blockIdx.x, smem);
}
// ---------------------------------------------------------------------------
// out: one work-group (4 waves) per (block, head, batch); wave w owns tokens
// 16w..16w+15 of the block.  Computes O^T tiles so that each lane writes four
// contiguous output values.  Q and K are staged row-major in LDS (all loads
// in flight at once); the tiled h^T / U^T fragments of the next value slice
// are loaded while the current one is computed.
// ---------------------------------------------------------------------------
template <typename E, int DK, int DV>
__global__ __launch_bounds__(256) void gdn_out_kernel(GdnOutArgs<E> a) {
    const int n = a.n0 + blockIdx.x, h = blockIdx.y, b = blockIdx.z;
    const int tid = threadIdx.x, w = tid >> 6, l = tid & 63, r = l & 15, g = l >> 4;
    const int T = a.T, H = a.H, NC = a.NC;
    const size_t tok0 = (size_t)b * T + (size_t)n * BLK;
    const size_t chunk = ((size_t)b * H + h) * NC + n;
    const float* gam = a.gam + chunk * BLK;
    const size_t ldk = (size_t)H * DK;
    const int nvalid = min(BLK, T - n * BLK);
    constexpr int PK = RP<E, DK>, KK = DK / 32, NV = DV / 16;
    static_assert(NV % 2 == 0, "value slices are processed in pairs");
    __shared__ __align__(16) E Qs[BLK * PK], Ks[BLK * PK];

    const E* hT = a.hT + chunk * DK * DV;
    const E* UT = a.UT + chunk * BLK * DV;
    Frag<E> fh[2][KK];
    Frag<E> fu[2][2];
    auto load_slice = [&](int buf, int vb) {
#pragma unroll
        for (int kk = 0; kk < KK; ++kk) fh[buf][kk] = ldfragT(hT, vb * KK + kk, l);
#pragma unroll
        for (int j = 0; j < 2; ++j) fu[buf][j] = ldfragT(UT, 2 * vb + j, l);
    };
    const auto qx = load_rows<E, BLK, DK>(a.q + tok0 * ldk + (size_t)h * DK, ldk, nvalid);
    const auto kx = load_rows<E, BLK, DK>(a.k + tok0 * ldk + (size_t)h * DK, ldk, nvalid);
    load_slice(0, 0);
    store_rows<E, BLK, DK, PK>(qx, Qs);
    store_rows<E, BLK, DK, PK>(kx, Ks);
    __syncthreads();

    // Q as B operand: Bt[t][d] = Q[t][d]
    const int t_lane = 16 * w + r;  // this lane's token (column of every O^T / P^T tile)
    Frag<E> fq[KK];
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) fq[kk] = ldfrag(Qs + t_lane * PK + 32 * kk + 4 * g);
    const float gt = gam[t_lane];
    // gamma at rows 16 sb + 4g + i, all read before use
    f32x4 gs[4];
#pragma unroll
    for (int sb = 0; sb < 4; ++sb) gs[sb] = ld4_now(gam + 16 * sb + 4 * g);
    // P^T[s][t] = (k_s . q_t) exp(gamma_t - gamma_s) for s <= t
    f32x4 P[4];
#pragma unroll
    for (int sb = 0; sb < 4; ++sb) {
        f32x4 acc = zero4();
        if (sb <= w) {
#pragma unroll
            for (int kk = 0; kk < KK; ++kk) mma(acc, ldfrag(Ks + (16 * sb + r) * PK + 32 * kk + 4 * g), fq[kk]);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int s2 = 16 * sb + 4 * g + i;
                acc[i] = (s2 <= t_lane) ? acc[i] * __expf(gt - gs[sb][i]) : 0.f;
            }
        }
        P[sb] = acc;
    }
    // P U: P split, U in the element type (U telescopes over repeated keys;
    // an fp64 emulation of the block algorithm on the stress input puts o at
    // 7e-3 with U rounded here against 2e-3 with U kept split: the products
    // that carry U into the state stay split)
    Frag2<E> fp[2];
    fp[0] = split_acc<E>(P[0], P[1]);
    fp[1] = split_acc<E>(P[2], P[3]);
    const float Gt = __expf(gt);
    E* ob = a.o + tok0 * H * DV + (size_t)h * DV;
    auto compute_slice = [&](int buf, int vb) {
        f32x4 acc = zero4();
#pragma unroll
        for (int kk = 0; kk < KK; ++kk) mma(acc, fh[buf][kk], fq[kk]);
        acc = acc * Gt;
#pragma unroll
        for (int j = 0; j < 2; ++j)
            if (2 * j <= w) mma2(acc, fu[buf][j], fp[j]);
        if (t_lane < nvalid) st4(ob + (size_t)t_lane * H * DV + 16 * vb + 4 * g, acc);
    };
#pragma unroll
    for (int vb = 0; vb < NV; vb += 2) {
        load_slice(1, vb + 1);
        compute_slice(0, vb);
        if (vb + 2 < NV) load_slice(0, vb + 2);
        compute_slice(1, vb + 1);
    }
}

}  // namespace clr
