/*
 * clr_c_driver.c -- a plain C11 consumer of the layer's C ABI (include/clr.h),
 * for the test suite.  It uses only that header, the HIP runtime API (device
 * memory, copies, one stream) and libc: no C++, no PyTorch.
 *
 *   clr_c_driver check
 *       Host-only checks that need no GPU: version, status strings, workspace
 *       sizes, and the errors every entry point returns before launching
 *       anything (null pointers, bad sizes, unsupported shapes, small
 *       workspace, overlapping outputs).  Exit 0 when all hold.
 *
 *   clr_c_driver run IN OUT
 *       Runs one Gated DeltaNet layer over N sequence chunks (B = 1) in the
 *       StateFlow order (StateFlow paper, Sec. 3.1, Eqs. 5 and 7): forward
 *       i = 0..N-1 with S_{i+1}^in = S_i^out, then backward i = N-1..0 with
 *       dS_i^out = dS_{i+1}^in, keeping only each chunk's incoming state.
 *       IN:  int32 magic 0x434c5231 ("CLR1"), B, T, H, dk, dv, dtype, N; then
 *            q, k, v, g, beta, dO in the element type (raw bits), then S_in and
 *            dS_out as float32.
 *       OUT: o, dq, dk, dv, dg, dbeta in the element type, then S_out and dS_in
 *            as float32.
 *       Exit 0 on success; on a library or HIP error, the status text on
 *       stderr and exit 2.
 *
 *   clr_c_driver run-saved IN OUT
 *       The same chain with gdn_fwd_save / gdn_bwd_saved: each chunk's
 *       forward keeps its activations in a buffer of clr_saved_bytes, which
 *       that chunk's backward reads instead of recomputing them.
 */
#include <hip/hip_runtime_api.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "clr.h"

#define MAGIC 0x434c5231

static int fail(const char* what, int st) {
    fprintf(stderr, "%s: status %d (%s)\n", what, st, clr_status_string(st));
    return 2;
}

#define HIPCHK(x)                                                                  \
    do {                                                                           \
        hipError_t e_ = (x);                                                       \
        if (e_ != hipSuccess) {                                                    \
            fprintf(stderr, "%s: %s\n", #x, hipGetErrorString(e_));                \
            return 2;                                                              \
        }                                                                          \
    } while (0)

/* ------------------------------------------------------------------------- */
/* host-only checks                                                           */
/* ------------------------------------------------------------------------- */

static int expect(int got, int want, const char* what) {
    if (got != want) {
        fprintf(stderr, "check failed: %s returned %d (%s), expected %d\n", what, got, clr_status_string(got), want);
        return 1;
    }
    return 0;
}

static int run_checks(void) {
    int bad = 0;
    if (clr_version() <= 0) {
        fprintf(stderr, "check failed: clr_version\n");
        bad++;
    }
    for (int s = CLR_OK; s <= CLR_ERANGE; ++s) {
        const char* t = clr_status_string(s);
        if (!t || !t[0]) {
            fprintf(stderr, "check failed: empty status string for %d\n", s);
            bad++;
        }
    }
    clr_shape_t sh = {1, 256, 2, 128, 128, CLR_BF16, 64};
    const size_t wf = clr_workspace_bytes(&sh, CLR_OP_GDN_FWD), wb = clr_workspace_bytes(&sh, CLR_OP_GDN_BWD);
    if (wf == 0 || wb < wf) {
        fprintf(stderr, "check failed: workspace sizes fwd %zu bwd %zu\n", wf, wb);
        bad++;
    }
    clr_shape_t odd = sh;
    odd.chunk = 32;
    if (clr_workspace_bytes(&odd, CLR_OP_GDN_FWD) != 0) {
        fprintf(stderr, "check failed: workspace size of a block size that is not built\n");
        bad++;
    }
    /* Fake, distinct, 256-byte aligned addresses: every call below must be
     * rejected on the host, so none of them is ever dereferenced. */
    char* base = (char*)(uintptr_t)0x100000000ull;
    const size_t tok = (size_t)sh.B * sh.T * sh.H;
    const size_t span = tok * 128 * 2;
    void* q = base;
    void* k = base + 1 * span;
    void* v = base + 2 * span;
    void* g = base + 3 * span;
    void* beta = base + 4 * span;
    void* o = base + 5 * span;
    float* S_out = (float*)(base + 6 * span);
    void* ws = base + 8 * span;
    bad += expect(gdn_fwd(&sh, NULL, k, v, g, beta, NULL, o, S_out, ws, wf, NULL), CLR_EINVAL, "gdn_fwd(q = NULL)");
    bad += expect(gdn_fwd(&sh, q, k, v, g, beta, NULL, o, S_out, ws, wf - 256, NULL), CLR_EWORKSPACE,
                  "gdn_fwd(small workspace)");
    bad += expect(gdn_fwd(&sh, q, k, v, g, beta, NULL, o, S_out, NULL, wf, NULL), CLR_EWORKSPACE, "gdn_fwd(ws = NULL)");
    bad += expect(gdn_fwd(&sh, q, k, v, g, beta, NULL, q, S_out, ws, wf, NULL), CLR_EINVAL, "gdn_fwd(o aliases q)");
    bad += expect(gdn_fwd(&sh, (char*)q + 2, k, v, g, beta, NULL, o, S_out, ws, wf, NULL), CLR_EINVAL,
                  "gdn_fwd(misaligned q)");
    clr_shape_t d256 = sh;
    d256.dk = d256.dv = 256;
    bad += expect(gdn_fwd(&d256, q, k, v, g, beta, NULL, o, S_out, ws, wf, NULL), CLR_ENOTSUP, "gdn_fwd(d = 256)");
    clr_shape_t neg = sh;
    neg.T = -1;
    bad += expect(gdn_fwd(&neg, q, k, v, g, beta, NULL, o, S_out, ws, wf, NULL), CLR_EINVAL, "gdn_fwd(T < 0)");
    bad += expect(gdn_fwd(&odd, q, k, v, g, beta, NULL, o, S_out, ws, wf, NULL), CLR_ENOTSUP, "gdn_fwd(chunk = 32)");
    bad += expect(gla_fwd(&sh, q, k, v, g, beta, NULL, o, S_out, ws, wf, NULL), CLR_EINVAL, "gla_fwd(beta != NULL)");
    /* backward: distinct outputs, one of them missing */
    void* dO = base + 9 * span;
    void* dq = base + 10 * span;
    void* dk = base + 11 * span;
    void* dv = base + 12 * span;
    void* dg = base + 13 * span;
    void* db = base + 14 * span;
    float* dS_in = (float*)(base + 15 * span);
    void* wsb = base + 16 * span;
    bad += expect(gdn_bwd(&sh, q, k, v, g, beta, NULL, dO, NULL, NULL, dk, dv, dg, db, dS_in, wsb, wb, NULL),
                  CLR_EINVAL, "gdn_bwd(dq = NULL)");
    bad += expect(gdn_bwd(&sh, q, k, v, g, beta, NULL, dO, NULL, dq, dk, dv, dg, db, dS_in, wsb, wf - 256, NULL),
                  CLR_EWORKSPACE, "gdn_bwd(forward-sized workspace)");
    bad += expect(gdn_bwd(&sh, q, k, v, g, beta, NULL, dO, NULL, dq, dq, dv, dg, db, dS_in, wsb, wb, NULL),
                  CLR_EINVAL, "gdn_bwd(dk aliases dq)");
    return bad ? 1 : 0;
}

/* ------------------------------------------------------------------------- */
/* the chunk chain on the GPU                                                 */
/* ------------------------------------------------------------------------- */

static int read_all(FILE* f, void* p, size_t n) { return fread(p, 1, n, f) == n ? 0 : 1; }
static int write_all(FILE* f, const void* p, size_t n) { return fwrite(p, 1, n, f) == n ? 0 : 1; }

static int run_chain(const char* in_path, const char* out_path, int save) {
    FILE* f = fopen(in_path, "rb");
    if (!f) {
        perror(in_path);
        return 2;
    }
    int32_t hd[8];
    if (read_all(f, hd, sizeof hd) || hd[0] != MAGIC) {
        fprintf(stderr, "%s: bad header\n", in_path);
        fclose(f);
        return 2;
    }
    const int B = hd[1], T = hd[2], H = hd[3], DK = hd[4], DV = hd[5], dtype = hd[6], N = hd[7];
    if (B != 1 || N < 1 || T % N || (dtype != CLR_F32 && dtype != CLR_BF16)) {
        fprintf(stderr, "unsupported run: B %d T %d N %d dtype %d\n", B, T, N, dtype);
        fclose(f);
        return 2;
    }
    const size_t es = dtype == CLR_BF16 ? 2 : 4;
    const size_t nk = (size_t)T * H * DK, nv = (size_t)T * H * DV, nt = (size_t)T * H, ns = (size_t)H * DK * DV;
    /* host copies, in file order */
    const size_t sizes[8] = {nk * es, nk * es, nv * es, nt * es, nt * es, nv * es, ns * 4, ns * 4};
    void* h[8];
    for (int i = 0; i < 8; ++i) {
        h[i] = malloc(sizes[i] ? sizes[i] : 1);
        if (!h[i] || read_all(f, h[i], sizes[i])) {
            fprintf(stderr, "%s: short read\n", in_path);
            fclose(f);
            return 2;
        }
    }
    fclose(f);

    hipStream_t st;
    HIPCHK(hipStreamCreate(&st));
    /* device inputs: q k v g beta dO S_in dS_out */
    void* d[8];
    for (int i = 0; i < 8; ++i) {
        HIPCHK(hipMalloc(&d[i], sizes[i] ? sizes[i] : 16));
        HIPCHK(hipMemcpyAsync(d[i], h[i], sizes[i], hipMemcpyHostToDevice, st));
    }
    /* device outputs: o dq dk dv dg dbeta (element type) */
    const size_t osz[6] = {nv * es, nk * es, nk * es, nv * es, nt * es, nt * es};
    void* od[6];
    for (int i = 0; i < 6; ++i) HIPCHK(hipMalloc(&od[i], osz[i] ? osz[i] : 16));
    /* boundary states S_0 .. S_N (S_0 = S_in) and the backward's two dS buffers */
    float* S;
    float* dS[2];
    HIPCHK(hipMalloc((void**)&S, (size_t)(N + 1) * ns * 4));
    HIPCHK(hipMalloc((void**)&dS[0], ns * 4));
    HIPCHK(hipMalloc((void**)&dS[1], ns * 4));
    HIPCHK(hipMemcpyAsync(S, d[6], ns * 4, hipMemcpyDeviceToDevice, st));

    const int L = T / N;
    clr_shape_t sh = {B, L, H, DK, DV, dtype, 64};
    size_t wsz = clr_workspace_bytes(&sh, CLR_OP_GDN_BWD);
    const size_t wf = clr_workspace_bytes(&sh, CLR_OP_GDN_FWD);
    if (wf > wsz) wsz = wf;
    if (wsz == 0) return fail("clr_workspace_bytes", CLR_EINVAL);
    void* ws;
    HIPCHK(hipMalloc(&ws, wsz));
    /* saved activations: one buffer per chunk, each held until that chunk's backward */
    const size_t nsv = save ? clr_saved_bytes(&sh) : 0;
    if (save && nsv == 0) return fail("clr_saved_bytes", CLR_ENOTSUP);
    char* sv = NULL;
    if (save) HIPCHK(hipMalloc((void**)&sv, (size_t)N * nsv));

    /* byte offset of chunk i in a [1, T, H, d] tensor */
#define OFF(base, i, d_) ((char*)(base) + (size_t)(i) * L * H * (d_) * es)
    for (int i = 0; i < N; ++i) {
        const int s = save ? gdn_fwd_save(&sh, OFF(d[0], i, DK), OFF(d[1], i, DK), OFF(d[2], i, DV), OFF(d[3], i, 1),
                                          OFF(d[4], i, 1), S + (size_t)i * ns, OFF(od[0], i, DV),
                                          S + (size_t)(i + 1) * ns, sv + (size_t)i * nsv, nsv, ws, wsz, st)
                           : gdn_fwd(&sh, OFF(d[0], i, DK), OFF(d[1], i, DK), OFF(d[2], i, DV), OFF(d[3], i, 1),
                                     OFF(d[4], i, 1), S + (size_t)i * ns, OFF(od[0], i, DV),
                                     S + (size_t)(i + 1) * ns, ws, wsz, st);
        if (s != CLR_OK) return fail(save ? "gdn_fwd_save" : "gdn_fwd", s);
    }
    HIPCHK(hipMemcpyAsync(dS[N & 1], d[7], ns * 4, hipMemcpyDeviceToDevice, st));
    for (int i = N - 1; i >= 0; --i) {
        /* dS[(i + 1) & 1] holds dS_{i+1}^in = dS_i^out; the call writes dS_i^in */
        const int s =
            save ? gdn_bwd_saved(&sh, OFF(d[0], i, DK), OFF(d[1], i, DK), OFF(d[2], i, DV), OFF(d[3], i, 1),
                                 OFF(d[4], i, 1), NULL, OFF(d[5], i, DV), dS[(i + 1) & 1], sv + (size_t)i * nsv, nsv,
                                 OFF(od[1], i, DK), OFF(od[2], i, DK), OFF(od[3], i, DV), OFF(od[4], i, 1),
                                 OFF(od[5], i, 1), dS[i & 1], ws, wsz, st)
                 : gdn_bwd(&sh, OFF(d[0], i, DK), OFF(d[1], i, DK), OFF(d[2], i, DV), OFF(d[3], i, 1),
                           OFF(d[4], i, 1), S + (size_t)i * ns, OFF(d[5], i, DV), dS[(i + 1) & 1],
                           OFF(od[1], i, DK), OFF(od[2], i, DK), OFF(od[3], i, DV), OFF(od[4], i, 1),
                           OFF(od[5], i, 1), dS[i & 1], ws, wsz, st);
        if (s != CLR_OK) return fail(save ? "gdn_bwd_saved" : "gdn_bwd", s);
    }
#undef OFF
    HIPCHK(hipStreamSynchronize(st));
    HIPCHK(hipGetLastError());

    FILE* g = fopen(out_path, "wb");
    if (!g) {
        perror(out_path);
        return 2;
    }
    int werr = 0;
    for (int i = 0; i < 6; ++i) {
        void* buf = malloc(osz[i] ? osz[i] : 1);
        if (!buf) return 2;
        HIPCHK(hipMemcpy(buf, od[i], osz[i], hipMemcpyDeviceToHost));
        werr |= write_all(g, buf, osz[i]);
        free(buf);
    }
    float* sb = (float*)malloc(ns * 4);
    if (!sb) return 2;
    HIPCHK(hipMemcpy(sb, S + (size_t)N * ns, ns * 4, hipMemcpyDeviceToHost));
    werr |= write_all(g, sb, ns * 4);
    HIPCHK(hipMemcpy(sb, dS[0], ns * 4, hipMemcpyDeviceToHost));
    werr |= write_all(g, sb, ns * 4);
    free(sb);
    if (fclose(g) || werr) {
        fprintf(stderr, "%s: write failed\n", out_path);
        return 2;
    }

    for (int i = 0; i < 8; ++i) {
        HIPCHK(hipFree(d[i]));
        free(h[i]);
    }
    for (int i = 0; i < 6; ++i) HIPCHK(hipFree(od[i]));
    HIPCHK(hipFree(S));
    HIPCHK(hipFree(dS[0]));
    HIPCHK(hipFree(dS[1]));
    HIPCHK(hipFree(ws));
    if (sv) HIPCHK(hipFree(sv));
    HIPCHK(hipStreamDestroy(st));
    return 0;
}

int main(int argc, char** argv) {
    if (argc == 2 && !strcmp(argv[1], "check")) return run_checks();
    if (argc == 4 && !strcmp(argv[1], "run")) return run_chain(argv[2], argv[3], 0);
    if (argc == 4 && !strcmp(argv[1], "run-saved")) return run_chain(argv[2], argv[3], 1);
    fprintf(stderr, "usage: %s check | run IN OUT | run-saved IN OUT\n", argv[0]);
    return 64;
}
