// clr_api.hip -- the C ABI: host-side validation, workspace layout and launch
// sequencing.  See include/clr.h for the contract.
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <string.h>

#include "clr.h"
#include "clr_kernels.h"

using namespace clr;

namespace {

constexpr size_t ALIGN = 256;
inline size_t align_up(size_t x) { return (x + ALIGN - 1) / ALIGN * ALIGN; }

bool gdn_shape_ok(int dk, int dv) {
    return (dk == 32 && dv == 32) || (dk == 64 && dv == 64) || (dk == 128 && dv == 128);
}
bool gla_shape_ok(int dk, int dv) { return gdn_shape_ok(dk, dv) || (dk == 128 && dv == 256); }

size_t esize(int dtype) { return dtype == CLR_BF16 ? 2 : 4; }

// Basic shape validation shared by every entry point.  The fp32 backward
// kernels are instantiated for dk = dv = 32 only.
int check_shape(const clr_shape_t* s, bool gla, bool bwd) {
    if (!s) return CLR_EINVAL;
    if (s->B < 1 || s->H < 1 || s->T < 0 || s->dk < 1 || s->dv < 1) return CLR_EINVAL;
    if (s->dtype != CLR_F32 && s->dtype != CLR_BF16) return CLR_ENOTSUP;
    if (gla ? !gla_shape_ok(s->dk, s->dv) : !gdn_shape_ok(s->dk, s->dv)) return CLR_ENOTSUP;
    if (bwd && s->dtype == CLR_F32 && !(s->dk == 32 && s->dv == 32)) return CLR_ENOTSUP;
    // 64-bit element counts must stay addressable
    const double tok = (double)s->B * s->T * s->H * (s->dk > s->dv ? s->dk : s->dv);
    if (tok > 9.0e15) return CLR_EINVAL;
    return CLR_OK;
}

// Workspace carve-up.  Each sub-buffer starts on a 256-byte boundary.
struct Carver {
    char* base;
    size_t off = 0;
    void* take(size_t bytes) {
        void* p = base ? base + off : nullptr;
        off = align_up(off + bytes);
        return p;
    }
};

size_t nblocks(const clr_shape_t* s) {
    const size_t NC = ((size_t)s->T + BLK - 1) / BLK;
    return (size_t)s->B * s->H * NC;
}

GdnWs carve_gdn(const clr_shape_t* s, bool bwd, char* base, size_t* total) {
    Carver c{base};
    const size_t nb = nblocks(s), es = esize(s->dtype), dk = s->dk, dv = s->dv;
    GdnWs w{};
    w.gam = (float*)c.take(nb * BLK * 4);
    w.W = c.take(nb * BLK * dk * es);
    w.KhT = c.take(nb * BLK * dk * es);
    w.UtT = c.take(nb * BLK * dv * es);
    w.hT = c.take(nb * dk * dv * es);
    w.UT = c.take(nb * BLK * dv * es);
    w.Smid = (float*)c.take((size_t)s->B * s->H * dk * dv * 4);
    if (bwd) {
        w.Rt = (float*)c.take(nb * dk * dv * 4);
        w.WT = c.take(nb * BLK * dk * es);
        w.Kh = c.take(nb * BLK * dk * es);
        w.dvlT = c.take(nb * BLK * dv * es);
        w.dhT = c.take(nb * dk * dv * es);
        w.dUT = c.take(nb * BLK * dv * es);
    }
    if (total) *total = c.off;
    return w;
}

GlaWs carve_gla(const clr_shape_t* s, bool bwd, char* base, size_t* total) {
    Carver c{base};
    const size_t nb = nblocks(s), es = esize(s->dtype), dk = s->dk, dv = s->dv;
    GlaWs w{};
    w.eC = (float*)c.take(nb * dk * 4);
    w.KhT = c.take(nb * BLK * dk * es);
    w.hT = c.take(nb * dk * dv * es);
    if (bwd) {
        w.QgT = c.take(nb * BLK * dk * es);
        w.Kh = c.take(nb * BLK * dk * es);
        w.dh = c.take(nb * dk * dv * es);
        w.dVs = c.take(nb * BLK * dv * es);
    }
    if (total) *total = c.off;
    return w;
}

// Pointer checks: alignment and pairwise overlap of [p, p + n).
struct Buf {
    const void* p;
    size_t n;
    bool out;
};

bool aligned16(const void* p) { return ((uintptr_t)p & 15) == 0; }

int check_bufs(const Buf* b, int nb) {
    for (int i = 0; i < nb; ++i) {
        if (!b[i].p || b[i].n == 0) continue;
        if (!aligned16(b[i].p)) return CLR_EINVAL;
    }
    for (int i = 0; i < nb; ++i) {
        if (!b[i].p || b[i].n == 0) continue;
        for (int j = i + 1; j < nb; ++j) {
            if (!b[j].p || b[j].n == 0) continue;
            if (!b[i].out && !b[j].out) continue;  // inputs may alias each other
            const uintptr_t a0 = (uintptr_t)b[i].p, a1 = a0 + b[i].n;
            const uintptr_t c0 = (uintptr_t)b[j].p, c1 = c0 + b[j].n;
            if (a0 < c1 && c0 < a1) return CLR_EINVAL;
        }
    }
    return CLR_OK;
}

int hip_status(hipError_t e) { return e == hipSuccess ? CLR_OK : CLR_EHIP; }

// T == 0: the state passes through unchanged.
int passthrough(const float* src, float* dst, size_t n, hipStream_t st) {
    if (!dst) return CLR_OK;
    hipError_t e = src ? hipMemcpyAsync(dst, src, n * 4, hipMemcpyDeviceToDevice, st)
                       : hipMemsetAsync(dst, 0, n * 4, st);
    return hip_status(e);
}

}  // namespace

extern "C" {

int clr_version(void) { return 100; }

const char* clr_status_string(int s) {
    switch (s) {
        case CLR_OK: return "ok";
        case CLR_EINVAL: return "invalid argument";
        case CLR_ENOTSUP: return "unsupported dtype or head size";
        case CLR_EWORKSPACE: return "workspace missing or too small";
        case CLR_EHIP: return "HIP error";
        default: return "unknown status";
    }
}

size_t clr_workspace_bytes(const clr_shape_t* s, int op) {
    if (op < CLR_OP_GDN_FWD || op > CLR_OP_M2_BWD) return 0;
    // the Mamba-2 member runs on the GLA kernels
    const bool gla = op != CLR_OP_GDN_FWD && op != CLR_OP_GDN_BWD;
    const bool bwd = op == CLR_OP_GDN_BWD || op == CLR_OP_GLA_BWD || op == CLR_OP_M2_BWD;
    if (check_shape(s, gla, bwd) != CLR_OK) return 0;
    size_t total = 0;
    if (gla) carve_gla(s, bwd, nullptr, &total);
    else carve_gdn(s, bwd, nullptr, &total);
    return total;
}

// Which member of the family an entry point computes.
enum Kind { K_GDN, K_GLA, K_M2 };

static int fwd_common(Kind kind, const clr_shape_t* s, const void* q, const void* k, const void* v,
                      const void* g, const void* beta, const float* S_in, void* o, float* S_out,
                      void* ws, size_t ws_bytes, void* stream) {
    const bool gla = kind != K_GDN;
    int rc = check_shape(s, gla, false);
    if (rc) return rc;
    if (!q || !k || !v || !g) return CLR_EINVAL;
    if (gla ? beta != nullptr : beta == nullptr) return CLR_EINVAL;
    const size_t es = esize(s->dtype);
    const size_t ntok = (size_t)s->B * s->T * s->H, nst = (size_t)s->B * s->H * s->dk * s->dv;
    Buf bufs[] = {{q, ntok * s->dk * es, false}, {k, ntok * s->dk * es, false},
                  {v, ntok * s->dv * es, false}, {g, ntok * (kind == K_GLA ? s->dk : 1) * es, false},
                  {beta, ntok * es, false},      {S_in, nst * 4, false},
                  {o, ntok * s->dv * es, true},  {S_out, nst * 4, true},
                  {ws, ws_bytes, true}};
    // g and beta rows of GDN are only 2/4-byte aligned per token but the
    // tensors themselves must start 16-byte aligned.
    if ((rc = check_bufs(bufs, 9))) return rc;
    const size_t need = clr_workspace_bytes(s, gla ? CLR_OP_GLA_FWD : CLR_OP_GDN_FWD);
    hipStream_t st = (hipStream_t)stream;
    if (s->T == 0) return passthrough(S_in, S_out, nst, st);
    if (!ws || ws_bytes < need || ((uintptr_t)ws & (ALIGN - 1))) return CLR_EWORKSPACE;
    const int NC = (s->T + BLK - 1) / BLK;
    if (!gla) {
        GdnLaunch L{};
        L.B = s->B; L.T = s->T; L.H = s->H; L.NC = NC; L.dk = s->dk; L.dv = s->dv;
        L.bf16 = s->dtype == CLR_BF16;
        L.q = q; L.k = k; L.v = v; L.g = g; L.beta = beta; L.S_in = S_in; L.o = o; L.S_out = S_out;
        L.ws = carve_gdn(s, false, (char*)ws, nullptr);
        return hip_status(launch_gdn_fwd(L, st));
    } else {
        GlaLaunch L{};
        L.B = s->B; L.T = s->T; L.H = s->H; L.NC = NC; L.dk = s->dk; L.dv = s->dv;
        L.bf16 = s->dtype == CLR_BF16;
        L.scalar_gate = kind == K_M2;
        L.q = q; L.k = k; L.v = v; L.g = g; L.S_in = S_in; L.o = o; L.S_out = S_out;
        L.ws = carve_gla(s, false, (char*)ws, nullptr);
        return hip_status(launch_gla_fwd(L, st));
    }
}

int gdn_fwd(const clr_shape_t* s, const void* q, const void* k, const void* v, const void* g,
            const void* beta, const float* S_in, void* o, float* S_out, void* ws, size_t ws_bytes,
            void* stream) {
    return fwd_common(K_GDN, s, q, k, v, g, beta, S_in, o, S_out, ws, ws_bytes, stream);
}

int gla_fwd(const clr_shape_t* s, const void* q, const void* k, const void* v, const void* g,
            const void* beta, const float* S_in, void* o, float* S_out, void* ws, size_t ws_bytes,
            void* stream) {
    return fwd_common(K_GLA, s, q, k, v, g, beta, S_in, o, S_out, ws, ws_bytes, stream);
}

int mamba2_fwd(const clr_shape_t* s, const void* q, const void* k, const void* v, const void* g,
               const void* beta, const float* S_in, void* o, float* S_out, void* ws, size_t ws_bytes,
               void* stream) {
    return fwd_common(K_M2, s, q, k, v, g, beta, S_in, o, S_out, ws, ws_bytes, stream);
}

static int bwd_common(Kind kind, const clr_shape_t* s, const void* q, const void* k, const void* v,
                      const void* g, const void* beta, const float* S_in, const void* dO,
                      const float* dS_out, void* dq, void* dk, void* dv, void* dg, void* dbeta,
                      float* dS_in, void* ws, size_t ws_bytes, void* stream) {
    const bool gla = kind != K_GDN;
    int rc = check_shape(s, gla, true);
    if (rc) return rc;
    if (!q || !k || !v || !g || !dO || !dq || !dk || !dv || !dg || !dS_in) return CLR_EINVAL;
    if (gla ? (beta != nullptr || dbeta != nullptr) : (beta == nullptr || dbeta == nullptr))
        return CLR_EINVAL;
    const size_t es = esize(s->dtype);
    const size_t ntok = (size_t)s->B * s->T * s->H, nst = (size_t)s->B * s->H * s->dk * s->dv;
    const size_t gn = ntok * (kind == K_GLA ? s->dk : 1) * es;
    Buf bufs[] = {{q, ntok * s->dk * es, false},  {k, ntok * s->dk * es, false},
                  {v, ntok * s->dv * es, false},  {g, gn, false},
                  {beta, ntok * es, false},       {S_in, nst * 4, false},
                  {dO, ntok * s->dv * es, false}, {dS_out, nst * 4, false},
                  {dq, ntok * s->dk * es, true},  {dk, ntok * s->dk * es, true},
                  {dv, ntok * s->dv * es, true},  {dg, gn, true},
                  {dbeta, ntok * es, true},       {dS_in, nst * 4, true},
                  {ws, ws_bytes, true}};
    if ((rc = check_bufs(bufs, 15))) return rc;
    const size_t need = clr_workspace_bytes(s, gla ? CLR_OP_GLA_BWD : CLR_OP_GDN_BWD);
    hipStream_t st = (hipStream_t)stream;
    if (s->T == 0) return passthrough(dS_out, dS_in, nst, st);
    if (!ws || ws_bytes < need || ((uintptr_t)ws & (ALIGN - 1))) return CLR_EWORKSPACE;
    const int NC = (s->T + BLK - 1) / BLK;
    if (!gla) {
        GdnLaunch L{};
        L.B = s->B; L.T = s->T; L.H = s->H; L.NC = NC; L.dk = s->dk; L.dv = s->dv;
        L.bf16 = s->dtype == CLR_BF16;
        L.q = q; L.k = k; L.v = v; L.g = g; L.beta = beta; L.S_in = S_in;
        L.dO = dO; L.dS_out = dS_out; L.dq = dq; L.dk_ = dk; L.dv_ = dv; L.dg = dg; L.dbeta = dbeta;
        L.dS_in = dS_in;
        L.ws = carve_gdn(s, true, (char*)ws, nullptr);
        return hip_status(launch_gdn_bwd(L, st));
    } else {
        GlaLaunch L{};
        L.B = s->B; L.T = s->T; L.H = s->H; L.NC = NC; L.dk = s->dk; L.dv = s->dv;
        L.bf16 = s->dtype == CLR_BF16;
        L.scalar_gate = kind == K_M2;
        L.q = q; L.k = k; L.v = v; L.g = g; L.S_in = S_in;
        L.dO = dO; L.dS_out = dS_out; L.dq = dq; L.dk_ = dk; L.dv_ = dv; L.dg = dg; L.dS_in = dS_in;
        L.ws = carve_gla(s, true, (char*)ws, nullptr);
        return hip_status(launch_gla_bwd(L, st));
    }
}

int gdn_bwd(const clr_shape_t* s, const void* q, const void* k, const void* v, const void* g,
            const void* beta, const float* S_in, const void* dO, const float* dS_out, void* dq,
            void* dk, void* dv, void* dg, void* dbeta, float* dS_in, void* ws, size_t ws_bytes,
            void* stream) {
    return bwd_common(K_GDN, s, q, k, v, g, beta, S_in, dO, dS_out, dq, dk, dv, dg, dbeta, dS_in, ws,
                      ws_bytes, stream);
}

int gla_bwd(const clr_shape_t* s, const void* q, const void* k, const void* v, const void* g,
            const void* beta, const float* S_in, const void* dO, const float* dS_out, void* dq,
            void* dk, void* dv, void* dg, void* dbeta, float* dS_in, void* ws, size_t ws_bytes,
            void* stream) {
    return bwd_common(K_GLA, s, q, k, v, g, beta, S_in, dO, dS_out, dq, dk, dv, dg, dbeta, dS_in, ws,
                      ws_bytes, stream);
}

int mamba2_bwd(const clr_shape_t* s, const void* q, const void* k, const void* v, const void* g,
               const void* beta, const float* S_in, const void* dO, const float* dS_out, void* dq,
               void* dk, void* dv, void* dg, void* dbeta, float* dS_in, void* ws, size_t ws_bytes,
               void* stream) {
    return bwd_common(K_M2, s, q, k, v, g, beta, S_in, dO, dS_out, dq, dk, dv, dg, dbeta, dS_in, ws,
                      ws_bytes, stream);
}

int clr_probe_mma(int dtype, const void* A, const void* Bt, float* C, void* stream) {
    if (dtype != CLR_F32 && dtype != CLR_BF16) return CLR_ENOTSUP;
    if (!A || !Bt || !C || !aligned16(A) || !aligned16(Bt) || !aligned16(C)) return CLR_EINVAL;
    return hip_status(launch_probe_mma(dtype == CLR_BF16, A, Bt, C, (hipStream_t)stream));
}

}  // extern "C"
