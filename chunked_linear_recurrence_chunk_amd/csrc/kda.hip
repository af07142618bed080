// kda.hip -- Kimi Delta Attention (the diagonal-plus-low-rank member of the
// StateFlow paper's Sec. 2.1: a per-key-channel decay followed by the delta
// rule's erase and write), chunk forward and backward on gfx950.
//
// Key-major state S [dk][dv]:  S_t = (I - beta_t k_t k_t^T) Diag(e^{g_t}) S_{t-1} + beta_t k_t v_t^T,
// o_t = S_t^T q_t.  Per 64-token block, with b = cumsum(g) per channel, S0 the
// state entering the block and dS1 the gradient of the state leaving it:
//   M[t][s] = sum_d k_t[d] k_s[d] e^{b_t[d] - b_s[d]}  (s < t),   A = Diag(beta) M,
//   T = (I + A)^-1,  W = T Diag(beta) (K e^b),  Ut = T Diag(beta) V,  U = Ut - W S0,
//   O = (Q e^b) S0 + (P * tril) U,   P[t][s] = sum_d q_t[d] k_s[d] e^{b_t[d] - b_s[d]},
//   S1 = Diag(e^{b_C}) S0 + (K e^{b_C - b})^T U.
// Forward:   kda_prep (e^{b_C}, W, Kh^T, -Ut^T; gla_kernels.h), the delta-rule
//            scan with a per-channel decay (gdn_kernels.h), and the GLA output
//            kernel on U (the output has the GLA form with U in place of V).
// Backward:  kda_prep, then
//   kda_prep2       W^T, Kh = K e^{b_C - b}, dvloc = P^T dO, R = (Q e^b)^T dO - W^T dvloc
//   scan pair       forward recompute (S0 of every block, U token-major) and the
//                   reverse scan dU = dvloc + Kh dS1, dS0 = Diag(e^{b_C}) dS1 + R - W^T (Kh dS1)
//   kda_bwd_wy      dW = -dU S0^T, dT = dW X^T + dU Y^T (X = Diag(beta) K e^b, Y = Diag(beta) V),
//                   dA = -T^T dT T^T (strictly lower), dM = Diag(beta) dA, dX = T^T dW,
//                   dv = beta T^T dU, dbeta = rowsum(dX * K e^b) + rowsum(T^T dU * V) + rowsum(dA * M)
//   GLA intra (KDA) dq, dk, dg from the P and M pair terms, the state terms and dX.
#include "gdn_bwd_kernels.h"
#include "gla_kernels.h"

namespace clr {

template <typename E> struct KdaPrep2Args {
    const E *q, *k, *dO, *g;
    const E* W;
    float* Rt;
    E *WT, *Kh;
    float* dvlT;  // fp32 (the reverse scan adds it to Kh dS)
    int T, H, NC;
    E* Kh_lo = nullptr;  // lo half of the decayed keys (bf16 inputs)
};

// ---------------------------------------------------------------------------
// prep2: one work-group (8 waves) per (block, head, batch); wave w8 owns the
// 16 tokens 16w.. (w = w8 & 3) as s (columns of P, rows of Kh and dvloc) and
// half hf = w8 >> 2 of the output tiles.  Both halves form the same P tiles.  P is formed per
// pair of 16-token tiles against a reference row of b between the two tiles
// (the end of tile w off the diagonal, its middle on it), as in the GLA kernels.
// ---------------------------------------------------------------------------
template <typename E, int DK, int DV>
__global__ __launch_bounds__(512) void kda_prep2_kernel(KdaPrep2Args<E> a) {
    constexpr int NT = 512;
    const int n = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
    const int tid = threadIdx.x, w8 = tid >> 6, w = w8 & 3, hf = w8 >> 2, l = tid & 63, r = l & 15, g = l >> 4;
    const int T = a.T, H = a.H, NC = a.NC;
    const size_t tok0 = (size_t)b * T + (size_t)n * BLK;
    const size_t chunk = ((size_t)b * H + h) * NC + n;
    const int nvalid = min(BLK, T - n * BLK);
    const size_t ldk = (size_t)H * DK, ldv = (size_t)H * DV;
    constexpr int PQ = RP<E, DK>, PO = RP<E, DV>, PB = DK + 4, KK = DK / 32, ND = DK / 16, NVB = DV / 16;

    __shared__ __align__(16) E Qs[BLK * PQ], Ks[BLK * PQ], dOs[BLK * PO], Ws[BLK * PQ], dvlt[DV * PT];
    __shared__ __align__(16) float Bs[BLK * PB];
    __shared__ float seg[256];

    {
        const auto kx = load_rows<E, BLK, DK, NT>(a.k + tok0 * ldk + (size_t)h * DK, ldk, nvalid);
        const auto gx = load_gate<false, E, DK, NT>(a.g, tok0, h, H, nvalid);
        const auto qx = load_rows<E, BLK, DK, NT>(a.q + tok0 * ldk + (size_t)h * DK, ldk, nvalid);
        const auto ox = load_rows<E, BLK, DV, NT>(a.dO + tok0 * ldv + (size_t)h * DV, ldv, nvalid);
        const auto wx = load_tiled<E, BLK, DK, NT>(a.W + chunk * BLK * DK);
        store_rows<E, BLK, DK, PQ, NT>(kx, Ks);
        store_rows<E, BLK, DK, PQ, NT>(gx, Qs);  // g staged where Q goes
        store_rows<E, BLK, DV, PO, NT>(ox, dOs);
        store_untiled<E, BLK, DK, PQ, NT>(wx, Ws);
        __syncthreads();
        gate_cumsum<E, DK, PQ, PB>(Qs, Bs, seg, nvalid);
        __syncthreads();
        store_rows<E, BLK, DK, PQ, NT>(qx, Qs);
        __syncthreads();
    }
    const float* bC = Bs + (BLK - 1) * PB;
    // W^T (tiled; A: m = d, k = t)
    E* WT = a.WT + chunk * BLK * DK;
#pragma unroll
    for (int f = w8; f < 2 * ND; f += 8) st_fragT(WT, f, l, ldfrag_tr(Ws, PQ, 32 * (f & 1), 16 * (f >> 1), l));
    // Kh[t][d] = K[t][d] e^{b_C[d] - b_t[d]} (tiled; A: m = t, k = d): fragments (w, kk)
    const int s = 16 * w + r;
    {
        // as a hi/lo pair: the reverse scan multiplies it by the split dS
        E* Kh = a.Kh + chunk * BLK * DK;
        E* Khl = a.Kh_lo + chunk * BLK * DK;
#pragma unroll
        for (int kk = hf; kk < KK; kk += 2) {
            const Frag2<E> x = frag_row_decay2(Ks, PQ, s, 32 * kk, Bs + s * PB, bC, -1.f);
            st_fragT(Kh, w * KK + kk, l, x.hi);
            if constexpr (sizeof(E) == 2) st_fragT(Khl, w * KK + kk, l, x.lo);
        }
    }
    // P[tb][w] (rows t, cols s), s <= t
    f32x4 P[4];
    {
        const float* refE = Bs + (16 * w + 15) * PB;
        const float* refD = Bs + (16 * w + 7) * PB;
        Frag<E> fkE[KK], fkD[KK];
#pragma unroll
        for (int kk = 0; kk < KK; ++kk) {
            fkE[kk] = frag_row_decay(Ks, PQ, s, 32 * kk, Bs + s * PB, refE, -1.f);
            fkD[kk] = frag_row_decay(Ks, PQ, s, 32 * kk, Bs + s * PB, refD, -1.f);
        }
#pragma unroll
        for (int tb = 0; tb < 4; ++tb) {
            f32x4 acc = zero4();
            if (tb >= w) {
                const int t = 16 * tb + r;
                const float* ref = tb > w ? refE : refD;
#pragma unroll
                for (int kk = 0; kk < KK; ++kk)
                    mma(acc, frag_row_decay(Qs, PQ, t, 32 * kk, Bs + t * PB, ref, 1.f), tb > w ? fkE[kk] : fkD[kk]);
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    if (16 * tb + 4 * g + i < s) acc[i] = 0.f;
            }
            P[tb] = acc;
        }
    }
    // dvloc^T[v][s] = sum_t P[t][s] dO[t][v]
    Frag<E> fp[2];
    fp[0] = frag_from_acc<E>(P[0], P[1]);
    fp[1] = frag_from_acc<E>(P[2], P[3]);
    float* dvlT = a.dvlT + chunk * BLK * DV;
#pragma unroll
    for (int vb = hf; vb < NVB; vb += 2) {
        f32x4 acc = zero4();
#pragma unroll
        for (int j = 0; j < 2; ++j) mma(acc, fp[j], ldfrag_tr(dOs, PO, 32 * j, 16 * vb, l));
        *(f32x4*)(dvlT + toff<float>(16 * vb + r, 16 * w + 4 * g, BLK)) = acc;
        st4(dvlt + (16 * vb + r) * PT + 16 * w + 4 * g, acc);
    }
    __syncthreads();
    // Qs <- Q e^b (factors <= 1)
    scale_exp_rows<E, DK, PQ, PB, NT>(Qs, Bs, Qs);
    __syncthreads();
    // R[d][v] = sum_t (Q e^b)^T[d][t] dO[t][v] - sum_t W^T[d][t] dvloc[t][v]   (fp32, accumulator-tiled)
    float* Rt = a.Rt + chunk * DK * DV;
    for (int tile = w8; tile < ND * NVB; tile += 8) {
        const int db = tile % ND, vb = tile / ND;
        f32x4 acc = zero4(), acc2 = zero4();
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            mma(acc, ldfrag_tr(Qs, PQ, 32 * j, 16 * db, l), ldfrag_tr(dOs, PO, 32 * j, 16 * vb, l));
            mma(acc2, ldfrag_tr(Ws, PQ, 32 * j, 16 * db, l), ldfrag(dvlt + (16 * vb + r) * PT + 32 * j + 4 * g));
        }
        *(f32x4*)(Rt + atoff(db, vb, DK, l)) = acc - acc2;
    }
}

template <typename E> struct KdaWyArgs {
    const E *v, *beta;
    const E* h;        // S0 per block (tiled [d][v])
    const float* dUT;  // dU^T per block (tiled [v][t], fp32)
    const E* TT;       // per block, from the prep: T^T (tiled)
    const float* M;    //   the decayed Gram product (accumulator tiles)
    const E* Kd;       //   K e^b (row-major [64][dk])
    E *dv, *dbeta;
    float *dM, *dX;    // per block: [64][64] and [64][dk], fp32
    int T, H, NC;
};

template <typename E, int DK, int DV> struct KdaWyLds {
    static constexpr int PK = RP<E, DK>, PV = RP<E, DV>;
    // persistent
    static constexpr size_t o_Kd = 0;                               // E[64][PK]    K e^b
    static constexpr size_t o_TT = o_Kd + sizeof(E) * BLK * PK;     // E[64][PT]    TT[s][t] = T[t][s]
    static constexpr size_t o_V = o_TT + sizeof(E) * BLK * PT;      // E[64][PV]; then dTT E[64][PT]
    // phase B: dUTs E[DV][PT], dWs E[64][PK]; dT^T takes V's place once the dT
    // products have read V (the total stays within 80 KB: two work-groups per CU)
    static constexpr size_t pB_dUT = o_V + sizeof(E) * BLK * PV, pB_dW = pB_dUT + sizeof(E) * DV * PT;
    static constexpr bool ALIAS = PT <= PV;  // else (small dv) a region of its own
    static constexpr size_t pB_dTT = ALIAS ? o_V : pB_dW + sizeof(E) * BLK * PK;
    static constexpr size_t total = pB_dW + sizeof(E) * BLK * PK + (ALIAS ? 0 : sizeof(E) * BLK * PT);
};

// ---------------------------------------------------------------------------
// WY adjoints: one work-group (8 waves) per (block, head, batch).  Wave w8:
// token block w = w8 & 3, half hf = w8 >> 2 (the halves split the column
// blocks of the adjoint tiles and the feature / value loops).  T, M and
// K e^b come from the prep of the same call.
// ---------------------------------------------------------------------------
template <typename E, int DK, int DV>
__global__ __launch_bounds__(512) void kda_bwd_wy_kernel(KdaWyArgs<E> a) {
    using Lay = KdaWyLds<E, DK, DV>;
    constexpr int NT = 512;
    constexpr int PK = Lay::PK, PV = Lay::PV, KK = DK / 32, KV = DV / 32, ND = DK / 16;
    constexpr int NDH = ND / 2, NVH = DV / 32;
    static_assert(Lay::total <= 150 * 1024, "LDS budget");
    __shared__ __align__(16) char lds[Lay::total];
    __shared__ float s_bet[BLK], s_g2[2][BLK], s_v2[2][BLK], s_k2[2][BLK];
    E* Kd = (E*)(lds + Lay::o_Kd);
    E* TT = (E*)(lds + Lay::o_TT);
    E* Vs = (E*)(lds + Lay::o_V);

    const int n = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
    const int tid = threadIdx.x, w8 = tid >> 6, w = w8 & 3, hf = w8 >> 2, l = tid & 63, r = l & 15, g = l >> 4;
    const int T = a.T, H = a.H, NC = a.NC;
    const size_t tok0 = (size_t)b * T + (size_t)n * BLK;
    const size_t chunk = ((size_t)b * H + h) * NC + n;
    const int nvalid = min(BLK, T - n * BLK);
    const size_t ldv = (size_t)H * DV;
    const E* S0 = a.h + chunk * DK * DV;

    // ---------------- phase 0: operands -------------------------------------
    E* dUTs = (E*)(lds + Lay::pB_dUT);
    E* dWs = (E*)(lds + Lay::pB_dW);
    E* dTT = (E*)(lds + Lay::pB_dTT);
    {
        const auto dux = load_tiled<float, DV, BLK, NT>(a.dUT + chunk * BLK * DV);
        const auto kx = load_rows<E, BLK, DK, NT>(a.Kd + chunk * BLK * DK, DK, BLK);
        const auto tx = load_tiled<E, BLK, BLK, NT>(a.TT + chunk * BLK * BLK);
        const auto vx = load_rows<E, BLK, DV, NT>(a.v + tok0 * ldv + (size_t)h * DV, ldv, nvalid);
        if (tid < BLK) s_bet[tid] = tid < nvalid ? to_f(a.beta[(tok0 + tid) * H + h]) : 0.f;
        store_rows<E, BLK, DK, PK, NT>(kx, Kd);
        store_untiled<E, BLK, BLK, PT, NT>(tx, TT);
        store_rows<E, BLK, DV, PV, NT>(vx, Vs);
        store_untiled_round<E, DV, BLK, PT, NT>(dux, dUTs);
    }
    __syncthreads();

    // ---------------- phase B: WY adjoints ------------------------------------
    // M tiles (w, cb) of this half, cb = hf and hf + 2, in flight during the dW and dT products
    f32x4 mtt[2];
#pragma unroll
    for (int u = 0; u < 2; ++u) mtt[u] = *(const f32x4*)(a.M + chunk * BLK * BLK + (4 * w + hf + 2 * u) * 256 + l * 4);
    const int tw = 16 * w + r;  // this lane's token as the column of transposed tiles
    // dW^T[db][w] = -(S0 dU^T): rows d, cols t = tw; stored as dW[t][d]
    {
        Frag<E> fdu[KV], fh[KV];
#pragma unroll
        for (int kk = 0; kk < KV; ++kk) {
            fdu[kk] = ldfrag_tr(dUTs, PT, 32 * kk, 16 * w, l);
            fh[kk] = ldfragT(S0, (hf * NDH) * KV + kk, l);
        }
#pragma unroll
        for (int jd = 0; jd < NDH; ++jd) {
            const int db = hf * NDH + jd;
            f32x4 acc = zero4();
#pragma unroll
            for (int kk = 0; kk < KV; ++kk) mma(acc, fh[kk], fdu[kk]);
            if (jd + 1 < NDH) {
#pragma unroll
                for (int kk = 0; kk < KV; ++kk) fh[kk] = ldfragT(S0, (db + 1) * KV + kk, l);
            }
            st4(dWs + tw * PK + 16 * db + 4 * g, -acc);
        }
    }
    __syncthreads();
    // dT[w][sb] = beta_s (dU V^T + dW (K e^b)^T): rows t, cols s; stored as dT^T[s][t]
    // (where V was, after every wave's V reads)
    {
        Frag<E> fdu[KV], fdw[KK];
#pragma unroll
        for (int kk = 0; kk < KV; ++kk) fdu[kk] = ldfrag_tr(dUTs, PT, 32 * kk, 16 * w, l);
#pragma unroll
        for (int kk = 0; kk < KK; ++kk) fdw[kk] = ldfrag(dWs + (16 * w + r) * PK + 32 * kk + 4 * g);
        f32x4 dts[2];
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            const int sb = hf + 2 * u;
            f32x4 acc = zero4();
#pragma unroll
            for (int kk = 0; kk < KV; ++kk) mma(acc, fdu[kk], ldfrag(Vs + (16 * sb + r) * PV + 32 * kk + 4 * g));
#pragma unroll
            for (int kk = 0; kk < KK; ++kk) mma(acc, fdw[kk], ldfrag(Kd + (16 * sb + r) * PK + 32 * kk + 4 * g));
            dts[u] = acc * s_bet[16 * sb + r];
        }
        __syncthreads();
#pragma unroll
        for (int u = 0; u < 2; ++u) st4(dTT + (16 * (hf + 2 * u) + r) * PT + 16 * w + 4 * g, dts[u]);
    }
    // V rows of this lane's token for the V term of dbeta (V is no longer in LDS)
    Raw4<E> vrow[NVH];
    const E* vtok = a.v + (tok0 + min(tw, nvalid - 1)) * ldv + (size_t)h * DV;
#pragma unroll
    for (int jv = 0; jv < NVH; ++jv) vrow[jv] = ldraw4(vtok + 16 * (hf * NVH + jv) + 4 * g);
    __syncthreads();
    // X^T[sb][w] = dT^T T (rows s, cols t = tw);  dA[w][cb] = -X T^T (rows t, cols c),
    // strictly lower;  dM = beta_t dA;  the Gram term of dbeta, sum_c dA[t][c] M[t][c]
    {
        f32x4 XT[4];
#pragma unroll
        for (int sb = 0; sb < 4; ++sb) {
            f32x4 acc = zero4();
#pragma unroll
            for (int j = 0; j < 2; ++j)
                mma(acc, ldfrag(dTT + (16 * sb + r) * PT + 32 * j + 4 * g), ldfrag(TT + tw * PT + 32 * j + 4 * g));
            XT[sb] = acc;
        }
        Frag<E> fx[2];
        fx[0] = frag_from_acc<E>(XT[0], XT[1]);
        fx[1] = frag_from_acc<E>(XT[2], XT[3]);
        float* dMb = a.dM + chunk * BLK * BLK;
        float gram[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int cb = 0; cb < 4; ++cb) {
            if ((cb & 1) != hf) continue;
            f32x4 acc = zero4();
            const f32x4 mt = mtt[cb >> 1];  // M tile (w, cb): rows 16w + 4g + i, column 16cb + r
            if (cb <= w) {
#pragma unroll
                for (int j = 0; j < 2; ++j) mma(acc, fx[j], ldfrag_tr(TT, PT, 32 * j, 16 * cb, l));  // T rows 16cb + r
            }
            const int c = 16 * cb + r;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int row = 16 * w + 4 * g + i;
                const float dA = c < row ? -acc[i] : 0.f;
                gram[i] += dA * mt[i];
                dMb[row * BLK + c] = dA * s_bet[row];
            }
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const float x = row16_sum(gram[i]);
            if (r == 0) s_g2[hf][16 * w + 4 * g + i] = x;
        }
    }
    // dV^T[vb][w] = beta_s (dU^T T): rows v, cols s = tw;  the V term of dbeta
    const float bet_tw = s_bet[tw];
    {
        float dbv = 0.f;
#pragma unroll
        for (int jv = 0; jv < NVH; ++jv) {
            const int vb = hf * NVH + jv;
            f32x4 acc = zero4();
#pragma unroll
            for (int j = 0; j < 2; ++j)
                mma(acc, ldfrag(dUTs + (16 * vb + r) * PT + 32 * j + 4 * g), ldfrag(TT + tw * PT + 32 * j + 4 * g));
            const f32x4 vv = cvt4(vrow[jv]);
            dbv += vv[0] * acc[0] + vv[1] * acc[1] + vv[2] * acc[2] + vv[3] * acc[3];
            if (tw < nvalid) st4(a.dv + (tok0 + tw) * ldv + (size_t)h * DV + 16 * vb + 4 * g, acc * bet_tw);
        }
        dbv += __shfl_xor(dbv, 16, 64);
        dbv += __shfl_xor(dbv, 32, 64);
        if (g == 0) s_v2[hf][tw] = dbv;
    }
    // dX^T[db][w] = dW^T T: rows d, cols s = tw (stored token-major, fp32);  the X term of dbeta
    {
        float dbk = 0.f;
        float* dXb = a.dX + chunk * BLK * DK;
#pragma unroll
        for (int jd = 0; jd < NDH; ++jd) {
            const int db = hf * NDH + jd;
            f32x4 acc = zero4();
#pragma unroll
            for (int j = 0; j < 2; ++j) mma(acc, ldfrag_tr(dWs, PK, 32 * j, 16 * db, l), ldfrag(TT + tw * PT + 32 * j + 4 * g));
            const f32x4 kv = ld4(Kd + tw * PK + 16 * db + 4 * g);
            dbk += kv[0] * acc[0] + kv[1] * acc[1] + kv[2] * acc[2] + kv[3] * acc[3];
            *(f32x4*)(dXb + (size_t)tw * DK + 16 * db + 4 * g) = acc;
        }
        dbk += __shfl_xor(dbk, 16, 64);
        dbk += __shfl_xor(dbk, 32, 64);
        if (g == 0) s_k2[hf][tw] = dbk;
    }
    __syncthreads();
    if (tid < nvalid) {  // combine the halves (fixed order)
        const int t = tid;
        const float db = (s_v2[0][t] + s_v2[1][t]) + (s_k2[0][t] + s_k2[1][t]) + (s_g2[0][t] + s_g2[1][t]);
        a.dbeta[(tok0 + t) * H + h] = from_f<E>(db);
    }
}

// ---------------------------------------------------------------------------
// Host-side launchers
// ---------------------------------------------------------------------------
template <typename E, int DK, int DV>
hipError_t launch_kda_fwd_t(const GdnLaunch& L, hipStream_t st) {
    const dim3 gblk(L.NC, L.H, L.B);
    const GdnWs& ws = L.ws;
    KdaPrepArgs<E> pa{(const E*)L.k, (const E*)L.v, (const E*)L.g, (const E*)L.beta, L.T, L.H, L.NC,
                      ws.eCk, (E*)ws.W, (E*)ws.KhT, (float*)ws.UtT, (E*)ws.KhT_lo};
    pa.range = ws.range;
    launch("kda_prep", kda_prep_kernel<E, DK, DV>, gblk, dim3(512), st, pa);
    GdnScanArgs<E> sa{nullptr, (const E*)ws.W, (const E*)ws.KhT, (const E*)ws.UtT, L.S_in, L.S_out,
                      (E*)ws.hT, nullptr, L.H, L.NC, L.B * L.H};
    sa.eC = ws.eCk;
    // saved activations: U token-major in the caller's buffer, and the states
    // once more in the backward's layout (the values its recompute stores)
    E* Utok = L.saved_U ? (E*)L.saved_U : (E*)ws.Utok;
    sa.Utok = Utok;
    sa.hN = (E*)L.saved_h;
    sa.T = L.T;
    sa.KhT_lo = (const E*)ws.KhT_lo;
    launch("kda_scan_fwd", gdn_scan_fwd_kernel<E, DK, DV, false, true, scan_np_fast<1>>,
           dim3(scan_grid(DV / 16, L.B * L.H)), dim3(scan_threads<scan_np_fast<1>, 1>), st, sa);
    if (L.o) {
        GlaOutArgs<E> oa{(const E*)L.q, (const E*)L.k, (const E*)Utok, (const E*)L.g, (const E*)ws.hT,
                         (E*)L.o, L.T, L.H, L.NC};
        launch("kda_out", gla_out_kernel<E, DK, DV, false>, gblk, dim3(512), st, oa);
    }
    return hipGetLastError();
}

template <typename E, int DK, int DV>
hipError_t launch_kda_bwd_t(const GdnLaunch& L, hipStream_t st) {
    const dim3 gblk(L.NC, L.H, L.B);
    const GdnWs& ws = L.ws;
    // with saved states and U the forward recompute (and the operands only it
    // reads: Ut, Kh^T) drops out
    const bool saved = L.saved_h != nullptr;
    KdaPrepArgs<E> pa{(const E*)L.k, (const E*)L.v, (const E*)L.g, (const E*)L.beta, L.T, L.H, L.NC,
                      ws.eCk, (E*)ws.W, saved ? nullptr : (E*)ws.KhT, saved ? nullptr : (float*)ws.UtT,
                      saved ? nullptr : (E*)ws.KhT_lo};
    pa.range = ws.range;
    pa.TT = (E*)ws.TT;
    pa.M = ws.KKG;
    pa.Kd = (E*)ws.Kd;
    launch("kda_prep_bwd", kda_prep_kernel<E, DK, DV>, gblk, dim3(512), st, pa);
    KdaPrep2Args<E> p2{(const E*)L.q, (const E*)L.k, (const E*)L.dO, (const E*)L.g, (const E*)ws.W,
                       (float*)ws.Rt, (E*)ws.WT, (E*)ws.Kh, (float*)ws.dvlT, L.T, L.H, L.NC};
    p2.Kh_lo = (E*)ws.Kh_lo;
    launch("kda_prep2", kda_prep2_kernel<E, DK, DV>, gblk, dim3(512), st, p2);
    GdnScanArgs<E> sa{nullptr, (const E*)ws.W, (const E*)ws.KhT, (const E*)ws.UtT, L.S_in, nullptr,
                      (E*)ws.hT, nullptr, L.H, L.NC, L.B * L.H};
    sa.eC = ws.eCk;
    sa.Utok = (E*)ws.Utok;
    sa.T = L.T;
    sa.KhT_lo = (const E*)ws.KhT_lo;
    GdnScanBwdArgs<E> sb{nullptr, (const E*)ws.Kh, (const E*)ws.WT, (const E*)ws.dvlT, ws.Rt,
                         L.dS_out, L.dS_in, (E*)ws.dhT, (E*)ws.dUT, L.H, L.NC, L.B * L.H};
    sb.eC = ws.eCk;
    sb.Kh_lo = (const E*)ws.Kh_lo;
    const int G = (int)scan_grid(DV / 16, L.B * L.H);
    if (saved)
        launch("kda_scan_rev", gdn_scan_rev_kernel<E, DK, DV, true, scan_np_fast<1>, 1>, dim3(G),
               dim3(scan_threads<scan_np_fast<1>, 1>), st, sb);
    else
        launch("kda_scan_pair", gdn_scan_pair_kernel<E, DK, DV, true, scan_np_fast<1>, 1>, dim3(2 * G),
               dim3(scan_threads<scan_np_fast<1>, 1>), st, sa, sb, G);
    const E* hT = saved ? (const E*)L.saved_h : (const E*)ws.hT;
    const E* Utok = saved ? (const E*)L.saved_U : (const E*)ws.Utok;
    KdaWyArgs<E> wa{(const E*)L.v, (const E*)L.beta, hT, (const float*)ws.dUT, (const E*)ws.TT, ws.KKG,
                    (const E*)ws.Kd, (E*)L.dv_, (E*)L.dbeta, ws.dM, ws.dX, L.T, L.H, L.NC};
    launch("kda_bwd_wy", kda_bwd_wy_kernel<E, DK, DV>, gblk, dim3(512), st, wa);
    GlaIntraArgs<E> ia{(const E*)L.q, (const E*)L.k, Utok, (const E*)L.dO, (const E*)L.g,
                       hT, (const E*)ws.dhT, nullptr, (E*)L.dq, (E*)L.dk_, nullptr, (E*)L.dg,
                       L.T, L.H, L.NC};
    ia.dM = ws.dM;
    ia.dX = ws.dX;
    ia.beta = (const E*)L.beta;
    launch("kda_bwd_intra", gla_bwd_intra_kernel<E, DK, DV, false, true>, gblk, dim3(512), st, ia);
    return hipGetLastError();
}

hipError_t launch_kda_fwd(const GdnLaunch& L, hipStream_t st) {
#define CLR_CASE(E, DK, DV) \
    if (L.dk == DK && L.dv == DV) return launch_kda_fwd_t<E, DK, DV>(L, st);
    if (L.bf16) {
        CLR_FOR_GDN_SHAPES(bf16)
    } else {
        CLR_FOR_KDA_SHAPES_F32(float)
    }
#undef CLR_CASE
    return hipErrorInvalidValue;
}

hipError_t launch_kda_bwd(const GdnLaunch& L, hipStream_t st) {
#define CLR_CASE(E, DK, DV) \
    if (L.dk == DK && L.dv == DV) return launch_kda_bwd_t<E, DK, DV>(L, st);
    if (L.bf16) {
        CLR_FOR_GDN_SHAPES(bf16)
    } else {
        CLR_FOR_GDN_BWD_SHAPES_F32(float)
    }
#undef CLR_CASE
    return hipErrorInvalidValue;
}

}  // namespace clr
