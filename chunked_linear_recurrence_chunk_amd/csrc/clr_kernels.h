// clr_kernels.h -- kernel argument blocks and host launchers (internal).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>

#include "clr_device.h"
#include "clr_launch.h"

namespace clr {

// Head sizes (dk, dv) instantiated for the delta-rule kernels.
#define CLR_FOR_GDN_SHAPES(E) \
    CLR_CASE(E, 32, 32)       \
    CLR_CASE(E, 64, 64)       \
    CLR_CASE(E, 128, 128)
// fp32 backward: the block kernels' LDS tiles fit for d <= 64.
#define CLR_FOR_GDN_BWD_SHAPES_F32(E) \
    CLR_CASE(E, 32, 32)               \
    CLR_CASE(E, 64, 64)
// fp32 KDA forward: the prep kernel's LDS tiles fit for d <= 64.
#define CLR_FOR_KDA_SHAPES_F32(E) \
    CLR_CASE(E, 32, 32)           \
    CLR_CASE(E, 64, 64)

// Workspace of the Gated DeltaNet path.  Block-major: index
// ((b * H + h) * NC + n) selects the 64-token block n of head h in batch b.
// UtT and dUT are fp32; UT is in the element type, and so are Rt and dvlT for
// Gated DeltaNet (fp32 for KDA) (see gdn_kernels.h, "Precision").  Gated
// DeltaNet: KhT / Kh hold the keys themselves; KDA: the per-channel decayed
// keys, as a bf16 hi/lo pair for bf16 inputs.
struct GdnWs {
    float* gam;   // [.., 64]       in-block cumulative log gate
    float* eg;    // [.., 64]       exp(gamma_C - gamma_t) for t < 63, exp(gamma_C) at t = 63 (GDN scans)
    void* W;      // [.., 64, dk]   W = T Diag(beta Gam) K           (token-major)
    void* KhT;    // [.., dk, 64]   K^T (GDN), (K * exp(b_C - b))^T (KDA)
    void* UtT;    // [.., dv, 64]   -(T Diag(beta) V)^T
    void* KhT_lo; // [.., dk, 64]   KDA, bf16 inputs: lo half of the decayed keys Kh^T
    void* hT;     // [.., dv, dk]   state entering the block, transposed
    void* UT;     // [.., dv, 64]   U^T (delta-rule new values)
    float* Smid;  // [B, H, dk, dv] state at the split point of a split forward
    // KDA forward only
    float* eCk;   // [.., 256]      exp(b_C) per key channel (padded)
    int* range;   // [..]           per block: 1 if the gates leave the diagonal tiles' bound
    void* Utok;   // [B, T, H, dv]  U, token-major
    // backward only
    void* Rt;     // [.., dv, dk]   R^T, R = (Diag(Gam) Q)^T dO - W^T dvloc  (GDN: element type; KDA: fp32)
    void* WT;     // [.., dk, 64]   W^T
    void* Kh;     // [.., 64, dk]   K (GDN), K * exp(b_C - b) (KDA)   (token-major)
    void* Kh_lo;  // [.., 64, dk]   KDA, bf16 inputs: lo half of Kh
    void* dvlT;   // [.., dv, 64]   dvloc^T, dvloc = (Q K^T * G * tril)^T dO
    void* dhT;    // [.., dk, dv]   gradient w.r.t. the state leaving the block (GDN: bf16 hi part)
    void* dhT_lo; // [.., dk, dv]   GDN, bf16 inputs: the lo part of that gradient
    void* dUT;    // [.., dv, 64]   dU^T
    void* TT;     // [.., 64, 64]   T^T (tiled), T = (I + A)^-1
    float* KKG;   // [.., 16, 256]  KDA: M, the decayed Gram product, accumulator tiles (rb, cb) at (4 rb + cb) * 256
    // KDA backward only
    void* Kd;     // [.., 64, dk]   K e^b (row-major)
    float* dM;    // [.., 64, 64]   Diag(beta) dA, the adjoint of the decayed Gram product (fp32)
    float* dX;    // [.., 64, dk]   T^T dW (fp32)
};

struct GdnLaunch {
    int B, T, H, NC, dk, dv;
    bool bf16;
    const void *q, *k, *v, *g, *beta;
    const float* S_in;
    void* o;
    float* S_out;
    // backward
    const void* dO;
    const float* dS_out;
    void *dq, *dk_, *dv_, *dg, *dbeta;
    float* dS_in;
    GdnWs ws;
    bool no_split = false;  // never take the two-stream split forward
    // saved forward activations (Gated DeltaNet): per block the entering state
    // in the backward's layout (tiled h[d][v]) and U^T (tiled), both in the
    // element type.  The forward writes them; the backward reads them in place
    // of its forward recompute.  Null: not saved / recompute.
    void* saved_h = nullptr;
    void* saved_U = nullptr;
};

template <typename E> struct GdnPrepArgs {
    const E *k, *v, *g, *beta;
    int T, H, NC;
    float* gam;
    E *W, *KhT;
    float* UtT;
    float* eg;
    int n0 = 0;  // first block of the launch (grid x covers blocks n0 ..)
    // backward only (nullable): T^T (tiled [s][t])
    E* TT = nullptr;
    // backward only: the reverse scan's operands (q, dO in; W^T, Kh, dvloc^T, R out)
    const E *q = nullptr, *dO = nullptr;
    E *WT = nullptr, *Kh = nullptr;
    E* dvlT = nullptr;  // in the element type
    E* Rt = nullptr;  // in the element type (accumulator-tiled, 256 elements per 16 x 16 tile)
};

// UtT and UT are fp32.  KDA (eC set): KhT is the hi half of the decayed keys
// and KhT_lo their lo half (bf16 inputs).
template <typename E> struct GdnScanArgs {
    const float* eg;  // GDN: per block exp(gamma_C - gamma_t), t < 63, and exp(gamma_C) at 63
    const E *W, *KhT;
    const void* UtT;
    const float* S_in;
    float* S_out;
    E* hT;
    void* UT;
    int H, NC, BH;
    int n0 = 0, n1 = 1 << 30;  // blocks [n0, min(n1, NC)) are scanned
    // per-channel decay (KDA): exp(b_C) per block, padded to 256 floats, and
    // U written token-major [B, T, H, dv] (rows of valid tokens only)
    const float* eC = nullptr;
    E* Utok = nullptr;
    int T = 0;
    const E* KhT_lo = nullptr;
    // Gated DeltaNet forward that saves its states for the backward: the state
    // entering each block also in the backward's layout (tiled h[d][v])
    E* hN = nullptr;
};

template <typename E> struct GdnOutArgs {
    const E *q, *k;
    const float* gam;
    const E* hT;
    const E* UT;  // U^T in the element type (the forward scan's store)
    E* o;
    int T, H, NC;
    int n0 = 0;  // first block of the launch
};

hipError_t launch_gdn_fwd(const GdnLaunch& L, hipStream_t st);
// KDA forward (g per key channel); kernels in gla.hip.
hipError_t launch_kda_fwd(const GdnLaunch& L, hipStream_t st);
hipError_t launch_kda_bwd(const GdnLaunch& L, hipStream_t st);
hipError_t launch_gdn_bwd(const GdnLaunch& L, hipStream_t st);

// ---------------------------------------------------------------------------
// GLA
// ---------------------------------------------------------------------------
#define CLR_FOR_GLA_SHAPES(E) \
    CLR_CASE(E, 32, 32)       \
    CLR_CASE(E, 64, 64)       \
    CLR_CASE(E, 128, 128)     \
    CLR_CASE(E, 128, 256)

struct GlaWs {
    int* range;   // [..]          per block: 1 if the gates leave the diagonal tiles' bound
    float* eC;    // [.., dk]      exp(b_C): the block's total decay per channel (fp32)
    void* KhT;    // [.., dk, 64]  (K * exp(b_C - b))^T, tiled
    void* hT;     // fwd: [.., dv, dk] state entering the block as h^T, tiled;
                  // bwd: [.., dk, dv] key-major h, tiled
    // backward only
    void* QgT;    // [.., dk, 64]  (Q * exp(b))^T, tiled
    void* Kh;     // [.., 64, dk]  K * exp(b_C - b), tiled
    void* dh;     // [.., dk, dv]  key-major gradient w.r.t. the state leaving the block, tiled
    void* dVs;    // [.., 64, dv]  Kh dh (state part of dV), token-major
};

struct GlaLaunch {
    int B, T, H, NC, dk, dv;
    bool bf16;
    bool scalar_gate;  // Mamba-2 member: g and dg are [B, T, H], broadcast over dk
    const void *q, *k, *v, *g;
    const float* S_in;
    void* o;
    float* S_out;
    const void* dO;
    const float* dS_out;
    void *dq, *dk_, *dv_, *dg;
    float* dS_in;
    GlaWs ws;
    // saved activations (gla_fwd_save / gla_bwd_saved and the Mamba-2 pair):
    // per block the entering state, tiled [d][v]
    void* saved_h = nullptr;
};

hipError_t launch_gla_fwd(const GlaLaunch& L, hipStream_t st);
hipError_t launch_gla_bwd(const GlaLaunch& L, hipStream_t st);

// Probe of the fragment abstraction: C[16][16] = A[16][32] * Bt[16][32]^T
// (dtype 0 = fp32, 1 = bf16), computed with ldfrag/mma.
hipError_t launch_probe_mma(int bf16, const void* A, const void* Bt, float* C, hipStream_t st);

}  // namespace clr
