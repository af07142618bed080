// clr_api.hip -- the C ABI: host-side validation, workspace layout and launch
// sequencing.  See include/clr.h for the contract.
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <string.h>

#include <mutex>
#include <vector>

#include "clr.h"
#include "clr_conv.h"
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
// kernels are instantiated for dk = dv <= 64.
int check_shape(const clr_shape_t* s, bool gla, bool bwd) {
    if (!s) return CLR_EINVAL;
    if (s->B < 1 || s->H < 1 || s->T < 0 || s->dk < 1 || s->dv < 1) return CLR_EINVAL;
    if (s->dtype != CLR_F32 && s->dtype != CLR_BF16) return CLR_ENOTSUP;
    if (s->chunk != 0 && s->chunk != BLK) return CLR_ENOTSUP;  // the kernels' block size
    if (gla ? !gla_shape_ok(s->dk, s->dv) : !gdn_shape_ok(s->dk, s->dv)) return CLR_ENOTSUP;
    if (bwd && s->dtype == CLR_F32 && (s->dk > 64 || s->dv > 64)) return CLR_ENOTSUP;
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
    // Ut and dU are fp32 (split operands); U, R and dvloc in the element type (gdn_kernels.h, "Precision")
    w.gam = (float*)c.take(nb * BLK * 4);
    w.eg = (float*)c.take(nb * BLK * 4);
    w.W = c.take(nb * BLK * dk * es);
    w.KhT = c.take(nb * BLK * dk * es);
    w.UtT = c.take(nb * BLK * dv * 4);
    w.hT = c.take(nb * dk * dv * es);
    w.UT = c.take(nb * BLK * dv * es);
    w.Smid = (float*)c.take((size_t)s->B * s->H * dk * dv * 4);
    if (bwd) {
        w.Rt = c.take(nb * dk * dv * es);  // R in the element type
        w.WT = c.take(nb * BLK * dk * es);
        w.Kh = c.take(nb * BLK * dk * es);
        w.dvlT = c.take(nb * BLK * dv * es);  // dvloc in the element type
        w.dhT = c.take(nb * dk * dv * es);
        if (es == 2) w.dhT_lo = c.take(nb * dk * dv * es);  // the lo part of dh (bf16 pair)
        w.dUT = c.take(nb * BLK * dv * 4);
        w.TT = c.take(nb * BLK * BLK * es);
    }
    if (total) *total = c.off;
    return w;
}

// Saved forward activations of the Gated DeltaNet layer: per block the
// entering state (tiled h[d][v]) and U^T (tiled [dv][64]), element type.
size_t saved_carve(const clr_shape_t* s, char* base, void** h, void** U) {
    Carver c{base};
    const size_t nb = nblocks(s), es = esize(s->dtype);
    void* ph = c.take(nb * s->dk * s->dv * es);
    void* pu = c.take(nb * BLK * s->dv * es);
    if (h) *h = ph;
    if (U) *U = pu;
    return c.off;
}

// The fp32 KDA forward and backward are instantiated for d <= 64.
bool kda_f32_unsupported(const clr_shape_t* s, bool bwd) {
    (void)bwd;
    return s->dtype == CLR_F32 && s->dk > 64;
}

// KDA: the Gated DeltaNet forward layouts the scan reads, exp(b_C) per key
// channel (padded to 256 floats) and U token-major; the backward adds the
// reverse-scan operands and the WY adjoints dM, dX.
GdnWs carve_kda(const clr_shape_t* s, bool bwd, char* base, size_t* total) {
    Carver c{base};
    const size_t nb = nblocks(s), es = esize(s->dtype), dk = s->dk, dv = s->dv;
    GdnWs w{};
    w.range = (int*)c.take(nb * 4);  // first, where clr_range_status finds it
    // Ut, dvloc and dU fp32; the decayed keys as a bf16 hi/lo pair (gdn_kernels.h, "Precision")
    w.W = c.take(nb * BLK * dk * es);
    w.KhT = c.take(nb * BLK * dk * es);
    if (es == 2) w.KhT_lo = c.take(nb * BLK * dk * es);
    w.UtT = c.take(nb * BLK * dv * 4);
    w.hT = c.take(nb * dk * dv * es);
    w.eCk = (float*)c.take(nb * 256 * 4);
    w.Utok = c.take((size_t)s->B * s->T * s->H * dv * es);
    if (bwd) {
        w.Rt = c.take(nb * dk * dv * 4);
        w.WT = c.take(nb * BLK * dk * es);
        w.Kh = c.take(nb * BLK * dk * es);
        if (es == 2) w.Kh_lo = c.take(nb * BLK * dk * es);
        w.dvlT = c.take(nb * BLK * dv * 4);
        w.dhT = c.take(nb * dk * dv * es);
        w.dUT = c.take(nb * BLK * dv * 4);
        w.dM = (float*)c.take(nb * BLK * BLK * 4);
        w.dX = (float*)c.take(nb * BLK * dk * 4);
        w.TT = c.take(nb * BLK * BLK * es);
        w.KKG = (float*)c.take(nb * BLK * BLK * 4);  // M, the decayed Gram product
        w.Kd = c.take(nb * BLK * dk * es);
    }
    if (total) *total = c.off;
    return w;
}

GlaWs carve_gla(const clr_shape_t* s, bool bwd, char* base, size_t* total) {
    Carver c{base};
    const size_t nb = nblocks(s), es = esize(s->dtype), dk = s->dk, dv = s->dv;
    GlaWs w{};
    w.range = (int*)c.take(nb * 4);  // first, where clr_range_status finds it
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

int conv_check_shape(const clr_conv_shape_t* s) {
    if (!s) return CLR_EINVAL;
    if (s->B < 1 || s->T < 0 || s->C < 8 || s->W < 1) return CLR_EINVAL;
    if (s->dtype != CLR_F32 && s->dtype != CLR_BF16) return CLR_ENOTSUP;
    if (s->C % 8 || s->W > 4 || (s->act != 0 && s->act != 1)) return CLR_ENOTSUP;
    if ((double)s->B * s->T * s->C > 9.0e15) return CLR_EINVAL;
    return CLR_OK;
}

template <typename E>
ConvArgs<E> conv_args(const clr_conv_shape_t* s, const void* x, const float* w, const float* bias,
                             const void* state_in) {
    ConvArgs<E> a{};
    a.B = s->B; a.T = s->T; a.C = s->C; a.W = s->W; a.act = s->act;
    a.x = (const E*)x; a.w = w; a.bias = bias; a.state_in = (const E*)state_in;
    return a;
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
        case CLR_ESCRATCH: return "needs more scratch than the allocation-free entry point holds";
        case CLR_ERANGE: return "gates beyond the diagonal tiles' decay bound";
        default: return "unknown status";
    }
}

size_t clr_saved_bytes(const clr_shape_t* s) {
    // the saved activations feed gdn_bwd_saved: the backward's shapes
    if (check_shape(s, false, true) != CLR_OK) return 0;
    return saved_carve(s, nullptr, nullptr, nullptr);
}

size_t clr_saved_bytes_op(const clr_shape_t* s, int op) {
    switch (op) {
        case CLR_OP_GDN_FWD: case CLR_OP_GDN_BWD: return clr_saved_bytes(s);
        case CLR_OP_KDA_FWD: case CLR_OP_KDA_BWD:
            // KDA: the Gated DeltaNet layout (states, then U token-major in the U space)
            if (check_shape(s, false, false) != CLR_OK || kda_f32_unsupported(s, true) || s->T == 0) return 0;
            return saved_carve(s, nullptr, nullptr, nullptr);
        case CLR_OP_GLA_FWD: case CLR_OP_GLA_BWD: case CLR_OP_M2_FWD: case CLR_OP_M2_BWD:
            // GLA and Mamba-2: per block the entering state, tiled [d][v]
            if (check_shape(s, true, true) != CLR_OK) return 0;
            return align_up(nblocks(s) * s->dk * s->dv * esize(s->dtype));
        default: return 0;
    }
}

size_t clr_workspace_bytes(const clr_shape_t* s, int op) {
    if (op == CLR_OP_KDA_FWD || op == CLR_OP_KDA_BWD) {
        const bool bwd = op == CLR_OP_KDA_BWD;
        if (check_shape(s, false, false) != CLR_OK || kda_f32_unsupported(s, bwd)) return 0;
        size_t total = 0;
        carve_kda(s, bwd, nullptr, &total);
        return total;
    }
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

// The per-block range records sit at the start of the GLA, KDA and Mamba-2
// workspaces (carve_gla, carve_kda); the prep kernels rewrite them every call.
int clr_range_status(const clr_shape_t* s, int op, const void* ws, void* stream) {
    if (op < CLR_OP_GDN_FWD || op > CLR_OP_KDA_BWD) return CLR_EINVAL;
    const bool kda = op == CLR_OP_KDA_FWD || op == CLR_OP_KDA_BWD;
    const bool gla = !kda && op != CLR_OP_GDN_FWD && op != CLR_OP_GDN_BWD;
    const bool bwd = op == CLR_OP_GDN_BWD || op == CLR_OP_GLA_BWD || op == CLR_OP_M2_BWD || op == CLR_OP_KDA_BWD;
    if (const int rc = check_shape(s, gla, kda ? false : bwd)) return rc;
    if (kda && kda_f32_unsupported(s, bwd)) return CLR_ENOTSUP;
    if (!kda && !gla) return CLR_OK;
    if (!ws || ((uintptr_t)ws & (ALIGN - 1))) return CLR_EWORKSPACE;
    const size_t nb = nblocks(s);
    if (nb == 0) return CLR_OK;
    std::vector<int> flags(nb);
    hipStream_t st = (hipStream_t)stream;
    if (hipMemcpyAsync(flags.data(), ws, nb * sizeof(int), hipMemcpyDeviceToHost, st) != hipSuccess ||
        hipStreamSynchronize(st) != hipSuccess)
        return CLR_EHIP;
    for (const int f : flags)
        if (f) return CLR_ERANGE;
    return CLR_OK;
}

// ---------------------------------------------------------------------------
// Allocation-free Gated DeltaNet forward: gdn_fwd with its workspace in the
// library's own device array.  The array's host-side name is not a device
// address; each device's address is taken once, with that device current,
// by hipGetSymbolAddress and kept, and only that address reaches a kernel.
// Nothing in it has to start at zero: the forward writes every workspace
// element before reading it.
// ---------------------------------------------------------------------------
static __device__ __align__(256) char scratch[CLR_NOALLOC_SCRATCH_BYTES];

namespace {
constexpr int MAX_DEVICES = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[MAX_DEVICES];  // device address of `scratch`, per device (null until taken)

int scratch_address(void** out) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= MAX_DEVICES) return CLR_EHIP;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void* p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return CLR_EHIP;
        g_scratch_ptr[dev] = p;
    }
    *out = g_scratch_ptr[dev];
    return CLR_OK;
}
}  // namespace

// Which member of the family an entry point computes.
enum Kind { K_GDN, K_GLA, K_M2, K_KDA };
// the op whose saved-activation size a member's saving pair uses
static int saved_op(Kind kind) {
    return kind == K_GDN ? CLR_OP_GDN_BWD : kind == K_GLA ? CLR_OP_GLA_BWD : kind == K_M2 ? CLR_OP_M2_BWD : CLR_OP_KDA_BWD;
}

static int fwd_common(Kind kind, const clr_shape_t* s, const void* q, const void* k, const void* v,
                      const void* g, const void* beta, const float* S_in, void* o, float* S_out,
                      void* ws, size_t ws_bytes, void* stream, bool noalloc = false,
                      void* saved = nullptr, size_t saved_bytes = 0, bool save = false) {
    const bool gla = kind == K_GLA || kind == K_M2;  // GLA kernels and head sizes
    const bool has_beta = kind == K_GDN || kind == K_KDA;
    int rc = check_shape(s, gla, false);
    if (rc) return rc;
    if (kind == K_KDA && kda_f32_unsupported(s, false)) return CLR_ENOTSUP;
    // per-token tensors are empty when T == 0 and may then be NULL
    const bool tok = s->T > 0;
    if (tok && (!q || !k || !v || !g)) return CLR_EINVAL;
    if (has_beta ? (tok && beta == nullptr) : beta != nullptr) return CLR_EINVAL;
    const size_t es = esize(s->dtype);
    const size_t ntok = (size_t)s->B * s->T * s->H, nst = (size_t)s->B * s->H * s->dk * s->dv;
    Buf bufs[] = {{q, ntok * s->dk * es, false}, {k, ntok * s->dk * es, false},
                  {v, ntok * s->dv * es, false}, {g, ntok * ((kind == K_GLA || kind == K_KDA) ? s->dk : 1) * es, false},
                  {beta, ntok * es, false},      {S_in, nst * 4, false},
                  {o, ntok * s->dv * es, true},  {S_out, nst * 4, true},
                  {ws, ws_bytes, true},          {saved, saved_bytes, true}};
    // g and beta rows of GDN are only 2/4-byte aligned per token but the
    // tensors themselves must start 16-byte aligned.
    if ((rc = check_bufs(bufs, 10))) return rc;
    if (save) {  // *_fwd_save: the saved activations feed the member's *_bwd_saved
        if ((rc = kind == K_KDA ? check_shape(s, false, false) : check_shape(s, gla, true))) return rc;
        if (kind == K_KDA && kda_f32_unsupported(s, true)) return CLR_ENOTSUP;
        const size_t need_s = clr_saved_bytes_op(s, saved_op(kind));
        if (need_s && (!saved || saved_bytes < need_s || ((uintptr_t)saved & (ALIGN - 1)))) return CLR_EWORKSPACE;
    }
    const size_t need = clr_workspace_bytes(s, kind == K_KDA ? CLR_OP_KDA_FWD : gla ? CLR_OP_GLA_FWD : CLR_OP_GDN_FWD);
    if (noalloc && need > (size_t)CLR_NOALLOC_SCRATCH_BYTES) return CLR_ESCRATCH;
    hipStream_t st = (hipStream_t)stream;
    if (s->T == 0) return passthrough(S_in, S_out, nst, st);
    if (noalloc) {  // the static scratch in place of a workspace (all arguments checked above)
        if ((rc = scratch_address(&ws))) return rc;
        ws_bytes = CLR_NOALLOC_SCRATCH_BYTES;
    }
    if (!ws || ws_bytes < need || ((uintptr_t)ws & (ALIGN - 1))) return CLR_EWORKSPACE;
    const int NC = (s->T + BLK - 1) / BLK;
    if (kind == K_KDA) {
        GdnLaunch L{};
        L.B = s->B; L.T = s->T; L.H = s->H; L.NC = NC; L.dk = s->dk; L.dv = s->dv;
        L.bf16 = s->dtype == CLR_BF16;
        L.q = q; L.k = k; L.v = v; L.g = g; L.beta = beta; L.S_in = S_in; L.o = o; L.S_out = S_out;
        L.ws = carve_kda(s, false, (char*)ws, nullptr);
        if (save) saved_carve(s, (char*)saved, &L.saved_h, &L.saved_U);
        return hip_status(launch_kda_fwd(L, st));
    }
    if (!gla) {
        GdnLaunch L{};
        L.B = s->B; L.T = s->T; L.H = s->H; L.NC = NC; L.dk = s->dk; L.dv = s->dv;
        L.bf16 = s->dtype == CLR_BF16;
        L.q = q; L.k = k; L.v = v; L.g = g; L.beta = beta; L.S_in = S_in; L.o = o; L.S_out = S_out;
        L.ws = carve_gdn(s, false, (char*)ws, nullptr);
        L.no_split = noalloc;
        if (save) saved_carve(s, (char*)saved, &L.saved_h, &L.saved_U);
        return hip_status(launch_gdn_fwd(L, st));
    } else {
        GlaLaunch L{};
        L.B = s->B; L.T = s->T; L.H = s->H; L.NC = NC; L.dk = s->dk; L.dv = s->dv;
        L.bf16 = s->dtype == CLR_BF16;
        L.scalar_gate = kind == K_M2;
        L.q = q; L.k = k; L.v = v; L.g = g; L.S_in = S_in; L.o = o; L.S_out = S_out;
        L.ws = carve_gla(s, false, (char*)ws, nullptr);
        if (save) L.saved_h = saved;
        return hip_status(launch_gla_fwd(L, st));
    }
}

int gdn_fwd(const clr_shape_t* s, const void* q, const void* k, const void* v, const void* g,
            const void* beta, const float* S_in, void* o, float* S_out, void* ws, size_t ws_bytes,
            void* stream) {
    return fwd_common(K_GDN, s, q, k, v, g, beta, S_in, o, S_out, ws, ws_bytes, stream);
}

// gdn_fwd with the static scratch as its workspace (validated first; no split schedule)
int gdn_fwd_noalloc(const clr_shape_t* s, const void* q, const void* k, const void* v, const void* g,
                    const void* beta, const float* S_in, void* o, float* S_out, void* stream) {
    return fwd_common(K_GDN, s, q, k, v, g, beta, S_in, o, S_out, nullptr, 0, stream, /*noalloc=*/true);
}

int gdn_fwd_save(const clr_shape_t* s, const void* q, const void* k, const void* v, const void* g,
                 const void* beta, const float* S_in, void* o, float* S_out, void* saved, size_t saved_bytes,
                 void* ws, size_t ws_bytes, void* stream) {
    return fwd_common(K_GDN, s, q, k, v, g, beta, S_in, o, S_out, ws, ws_bytes, stream, false, saved, saved_bytes,
                      /*save=*/true);
}

int gla_fwd(const clr_shape_t* s, const void* q, const void* k, const void* v, const void* g,
            const void* beta, const float* S_in, void* o, float* S_out, void* ws, size_t ws_bytes,
            void* stream) {
    return fwd_common(K_GLA, s, q, k, v, g, beta, S_in, o, S_out, ws, ws_bytes, stream);
}

int gla_fwd_save(const clr_shape_t* s, const void* q, const void* k, const void* v, const void* g,
                 const void* beta, const float* S_in, void* o, float* S_out, void* saved, size_t saved_bytes,
                 void* ws, size_t ws_bytes, void* stream) {
    return fwd_common(K_GLA, s, q, k, v, g, beta, S_in, o, S_out, ws, ws_bytes, stream, false, saved, saved_bytes,
                      /*save=*/true);
}

int mamba2_fwd_save(const clr_shape_t* s, const void* q, const void* k, const void* v, const void* g,
                    const void* beta, const float* S_in, void* o, float* S_out, void* saved, size_t saved_bytes,
                    void* ws, size_t ws_bytes, void* stream) {
    return fwd_common(K_M2, s, q, k, v, g, beta, S_in, o, S_out, ws, ws_bytes, stream, false, saved, saved_bytes,
                      /*save=*/true);
}

int kda_fwd_save(const clr_shape_t* s, const void* q, const void* k, const void* v, const void* g,
                 const void* beta, const float* S_in, void* o, float* S_out, void* saved, size_t saved_bytes,
                 void* ws, size_t ws_bytes, void* stream) {
    return fwd_common(K_KDA, s, q, k, v, g, beta, S_in, o, S_out, ws, ws_bytes, stream, false, saved, saved_bytes,
                      /*save=*/true);
}

int kda_fwd(const clr_shape_t* s, const void* q, const void* k, const void* v, const void* g,
            const void* beta, const float* S_in, void* o, float* S_out, void* ws, size_t ws_bytes,
            void* stream) {
    return fwd_common(K_KDA, s, q, k, v, g, beta, S_in, o, S_out, ws, ws_bytes, stream);
}

int mamba2_fwd(const clr_shape_t* s, const void* q, const void* k, const void* v, const void* g,
               const void* beta, const float* S_in, void* o, float* S_out, void* ws, size_t ws_bytes,
               void* stream) {
    return fwd_common(K_M2, s, q, k, v, g, beta, S_in, o, S_out, ws, ws_bytes, stream);
}

static int bwd_common(Kind kind, const clr_shape_t* s, const void* q, const void* k, const void* v,
                      const void* g, const void* beta, const float* S_in, const void* dO,
                      const float* dS_out, void* dq, void* dk, void* dv, void* dg, void* dbeta,
                      float* dS_in, void* ws, size_t ws_bytes, void* stream,
                      const void* saved = nullptr, size_t saved_bytes = 0, bool use_saved = false) {
    const bool gla = kind == K_GLA || kind == K_M2;  // GLA kernels and head sizes
    const bool has_beta = kind == K_GDN || kind == K_KDA;
    int rc = kind == K_KDA ? check_shape(s, false, false) : check_shape(s, gla, true);
    if (rc) return rc;
    if (kind == K_KDA && kda_f32_unsupported(s, true)) return CLR_ENOTSUP;
    // per-token tensors are empty when T == 0 and may then be NULL
    const bool tok = s->T > 0;
    if (!dS_in || (tok && (!q || !k || !v || !g || !dO || !dq || !dk || !dv || !dg))) return CLR_EINVAL;
    if (has_beta ? (tok && (beta == nullptr || dbeta == nullptr)) : (beta != nullptr || dbeta != nullptr))
        return CLR_EINVAL;
    const size_t es = esize(s->dtype);
    const size_t ntok = (size_t)s->B * s->T * s->H, nst = (size_t)s->B * s->H * s->dk * s->dv;
    const size_t gn = ntok * ((kind == K_GLA || kind == K_KDA) ? s->dk : 1) * es;
    Buf bufs[] = {{q, ntok * s->dk * es, false},  {k, ntok * s->dk * es, false},
                  {v, ntok * s->dv * es, false},  {g, gn, false},
                  {beta, ntok * es, false},       {S_in, nst * 4, false},
                  {dO, ntok * s->dv * es, false}, {dS_out, nst * 4, false},
                  {dq, ntok * s->dk * es, true},  {dk, ntok * s->dk * es, true},
                  {dv, ntok * s->dv * es, true},  {dg, gn, true},
                  {dbeta, ntok * es, true},       {dS_in, nst * 4, true},
                  {ws, ws_bytes, true},           {saved, saved_bytes, false}};
    if ((rc = check_bufs(bufs, 16))) return rc;
    if (use_saved) {
        const size_t need_s = clr_saved_bytes_op(s, saved_op(kind));
        if (need_s && (!saved || saved_bytes < need_s || ((uintptr_t)saved & (ALIGN - 1)))) return CLR_EWORKSPACE;
    }
    const size_t need = clr_workspace_bytes(s, kind == K_KDA ? CLR_OP_KDA_BWD : gla ? CLR_OP_GLA_BWD : CLR_OP_GDN_BWD);
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
        if (kind == K_KDA) {
            L.ws = carve_kda(s, true, (char*)ws, nullptr);
            if (use_saved) saved_carve(s, (char*)saved, &L.saved_h, &L.saved_U);
            return hip_status(launch_kda_bwd(L, st));
        }
        L.ws = carve_gdn(s, true, (char*)ws, nullptr);
        if (use_saved) saved_carve(s, (char*)saved, &L.saved_h, &L.saved_U);
        return hip_status(launch_gdn_bwd(L, st));
    } else {
        GlaLaunch L{};
        L.B = s->B; L.T = s->T; L.H = s->H; L.NC = NC; L.dk = s->dk; L.dv = s->dv;
        L.bf16 = s->dtype == CLR_BF16;
        L.scalar_gate = kind == K_M2;
        L.q = q; L.k = k; L.v = v; L.g = g; L.S_in = S_in;
        L.dO = dO; L.dS_out = dS_out; L.dq = dq; L.dk_ = dk; L.dv_ = dv; L.dg = dg; L.dS_in = dS_in;
        L.ws = carve_gla(s, true, (char*)ws, nullptr);
        if (use_saved) L.saved_h = const_cast<void*>(saved);
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

int gdn_bwd_saved(const clr_shape_t* s, const void* q, const void* k, const void* v, const void* g,
                  const void* beta, const float* S_in, const void* dO, const float* dS_out, const void* saved,
                  size_t saved_bytes, void* dq, void* dk, void* dv, void* dg, void* dbeta, float* dS_in, void* ws,
                  size_t ws_bytes, void* stream) {
    return bwd_common(K_GDN, s, q, k, v, g, beta, S_in, dO, dS_out, dq, dk, dv, dg, dbeta, dS_in, ws, ws_bytes,
                      stream, saved, saved_bytes, /*use_saved=*/true);
}

int kda_bwd(const clr_shape_t* s, const void* q, const void* k, const void* v, const void* g,
            const void* beta, const float* S_in, const void* dO, const float* dS_out, void* dq,
            void* dk, void* dv, void* dg, void* dbeta, float* dS_in, void* ws, size_t ws_bytes,
            void* stream) {
    return bwd_common(K_KDA, s, q, k, v, g, beta, S_in, dO, dS_out, dq, dk, dv, dg, dbeta, dS_in, ws,
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

int kda_bwd_saved(const clr_shape_t* s, const void* q, const void* k, const void* v, const void* g,
                  const void* beta, const float* S_in, const void* dO, const float* dS_out, const void* saved,
                  size_t saved_bytes, void* dq, void* dk, void* dv, void* dg, void* dbeta, float* dS_in, void* ws,
                  size_t ws_bytes, void* stream) {
    return bwd_common(K_KDA, s, q, k, v, g, beta, S_in, dO, dS_out, dq, dk, dv, dg, dbeta, dS_in, ws, ws_bytes,
                      stream, saved, saved_bytes, /*use_saved=*/true);
}

int gla_bwd_saved(const clr_shape_t* s, const void* q, const void* k, const void* v, const void* g,
                  const void* beta, const float* S_in, const void* dO, const float* dS_out, const void* saved,
                  size_t saved_bytes, void* dq, void* dk, void* dv, void* dg, void* dbeta, float* dS_in, void* ws,
                  size_t ws_bytes, void* stream) {
    return bwd_common(K_GLA, s, q, k, v, g, beta, S_in, dO, dS_out, dq, dk, dv, dg, dbeta, dS_in, ws, ws_bytes,
                      stream, saved, saved_bytes, /*use_saved=*/true);
}

int mamba2_bwd_saved(const clr_shape_t* s, const void* q, const void* k, const void* v, const void* g,
                     const void* beta, const float* S_in, const void* dO, const float* dS_out, const void* saved,
                     size_t saved_bytes, void* dq, void* dk, void* dv, void* dg, void* dbeta, float* dS_in,
                     void* ws, size_t ws_bytes, void* stream) {
    return bwd_common(K_M2, s, q, k, v, g, beta, S_in, dO, dS_out, dq, dk, dv, dg, dbeta, dS_in, ws, ws_bytes,
                      stream, saved, saved_bytes, /*use_saved=*/true);
}

size_t clr_shortconv_workspace_bytes(const clr_conv_shape_t* s) {
    if (conv_check_shape(s) != CLR_OK) return 0;
    const size_t P = (size_t)s->B * conv_bwd_tile_groups(s->B, s->T, s->C, CONV_BWD_TT);
    return align_up(P * s->C * (s->W + 1) * 4 + 4);
}

int shortconv_fwd(const clr_conv_shape_t* s, const void* x, const float* w, const float* bias,
                  const void* state_in, void* y, void* state_out, void* stream) {
    int rc = conv_check_shape(s);
    if (rc) return rc;
    if (!w || (s->T > 0 && (!x || !y))) return CLR_EINVAL;  // x, y are empty (may be NULL) when T == 0
    const size_t es = esize(s->dtype), n = (size_t)s->B * s->T * s->C, ns = (size_t)s->B * (s->W - 1) * s->C;
    Buf bufs[] = {{x, n * es, false}, {w, (size_t)s->C * s->W * 4, false}, {bias, (size_t)s->C * 4, false},
                  {state_in, ns * es, false}, {y, n * es, true}, {state_out, ns * es, true}};
    if ((rc = check_bufs(bufs, 6))) return rc;
    hipStream_t st = (hipStream_t)stream;
    if (s->T == 0) {
        if (!state_out || ns == 0) return CLR_OK;
        return hip_status(state_in ? hipMemcpyAsync(state_out, state_in, ns * es, hipMemcpyDeviceToDevice, st)
                                   : hipMemsetAsync(state_out, 0, ns * es, st));
    }
    if (s->dtype == CLR_BF16) {
        ConvArgs<bf16> a = conv_args<bf16>(s, x, w, bias, state_in);
        a.y = (bf16*)y; a.state_out = (bf16*)state_out;
        return hip_status(launch_shortconv_fwd(a, st));
    }
    ConvArgs<float> a = conv_args<float>(s, x, w, bias, state_in);
    a.y = (float*)y; a.state_out = (float*)state_out;
    return hip_status(launch_shortconv_fwd(a, st));
}

int shortconv_bwd(const clr_conv_shape_t* s, const void* x, const float* w, const float* bias,
                  const void* state_in, const void* dy, const float* dstate_out, void* dx, float* dw,
                  float* dbias, float* dstate_in, int accumulate, void* ws, size_t ws_bytes, void* stream) {
    int rc = conv_check_shape(s);
    if (rc) return rc;
    if (!w || !dw || (s->W > 1 && !dstate_in) || (s->T > 0 && (!x || !dy || !dx))) return CLR_EINVAL;
    if (accumulate != 0 && accumulate != 1) return CLR_EINVAL;
    const size_t es = esize(s->dtype), n = (size_t)s->B * s->T * s->C, ns = (size_t)s->B * (s->W - 1) * s->C;
    const size_t nw = (size_t)s->C * s->W * 4, nb = (size_t)s->C * 4;
    Buf bufs[] = {{x, n * es, false},          {w, nw, false},           {bias, nb, false},
                  {state_in, ns * es, false},  {dy, n * es, false},      {dstate_out, ns * 4, false},
                  {dx, n * es, true},          {dw, nw, true},           {dbias, nb, true},
                  {dstate_in, ns * 4, true},   {ws, ws_bytes, true}};
    if ((rc = check_bufs(bufs, 11))) return rc;
    hipStream_t st = (hipStream_t)stream;
    if (s->T == 0) {
        hipError_t e = hipSuccess;
        if (dstate_in && ns)
            e = dstate_out ? hipMemcpyAsync(dstate_in, dstate_out, ns * 4, hipMemcpyDeviceToDevice, st)
                           : hipMemsetAsync(dstate_in, 0, ns * 4, st);
        if (e == hipSuccess && !accumulate) e = hipMemsetAsync(dw, 0, nw, st);
        if (e == hipSuccess && !accumulate && dbias) e = hipMemsetAsync(dbias, 0, nb, st);
        return hip_status(e);
    }
    if (!ws || ws_bytes < clr_shortconv_workspace_bytes(s) || ((uintptr_t)ws & (ALIGN - 1))) return CLR_EWORKSPACE;
    if (s->dtype == CLR_BF16) {
        ConvArgs<bf16> a = conv_args<bf16>(s, x, w, bias, state_in);
        a.dy = (const bf16*)dy; a.dstate_out = dstate_out; a.dx = (bf16*)dx;
        a.dstate_in = dstate_in; a.dw = dw; a.dbias = dbias; a.part = (float*)ws;
        return hip_status(launch_shortconv_bwd(a, accumulate, st));
    }
    ConvArgs<float> a = conv_args<float>(s, x, w, bias, state_in);
    a.dy = (const float*)dy; a.dstate_out = dstate_out; a.dx = (float*)dx;
    a.dstate_in = dstate_in; a.dw = dw; a.dbias = dbias; a.part = (float*)ws;
    return hip_status(launch_shortconv_bwd(a, accumulate, st));
}

int clr_probe_mma(int dtype, const void* A, const void* Bt, float* C, void* stream) {
    if (dtype != CLR_F32 && dtype != CLR_BF16) return CLR_ENOTSUP;
    if (!A || !Bt || !C || !aligned16(A) || !aligned16(Bt) || !aligned16(C)) return CLR_EINVAL;
    return hip_status(launch_probe_mma(dtype == CLR_BF16, A, Bt, C, (hipStream_t)stream));
}

}  // extern "C"
