/*
 * oracle_sanitize.c -- test driver: runs every fp64 oracle entry point on a
 * tiny problem under AddressSanitizer and UndefinedBehaviorSanitizer (built
 * by tests/test_oracle_sanitize.py with gcc -fsanitize=address,undefined
 * against oracle/clr_oracle.c and oracle/conv_oracle.c), and checks each
 * member's adjoints against central finite differences of
 *     L = sum_t <dO_t, o_t> + <dS_out, S_out>_F
 * (the gradient definition of the StateFlow paper's chunk backward, Sec. 3.1),
 * so that the sanitizers see the forward, the checkpointed backward and the
 * chunk boundary (T crosses the 64-token checkpoint).  Exit status 0 = pass.
 * Test infrastructure only; it declares the oracle's prototypes itself.
 */
#include <math.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

int ref_gdn_fwd(int, int, int, int, int, const double*, const double*, const double*, const double*,
                const double*, const double*, double*, double*);
int ref_gdn_bwd(int, int, int, int, int, const double*, const double*, const double*, const double*,
                const double*, const double*, const double*, const double*, double*, double*, double*,
                double*, double*, double*);
int ref_kda_fwd(int, int, int, int, int, const double*, const double*, const double*, const double*,
                const double*, const double*, double*, double*);
int ref_kda_bwd(int, int, int, int, int, const double*, const double*, const double*, const double*,
                const double*, const double*, const double*, const double*, double*, double*, double*,
                double*, double*, double*);
int ref_gla_fwd(int, int, int, int, int, const double*, const double*, const double*, const double*,
                const double*, double*, double*);
int ref_gla_bwd(int, int, int, int, int, const double*, const double*, const double*, const double*,
                const double*, const double*, const double*, double*, double*, double*, double*, double*);
int ref_m2_fwd(int, int, int, int, int, const double*, const double*, const double*, const double*,
               const double*, double*, double*);
int ref_m2_bwd(int, int, int, int, int, const double*, const double*, const double*, const double*,
               const double*, const double*, const double*, double*, double*, double*, double*, double*);
int ref_conv_fwd(int, int, int, int, int, const double*, const double*, const double*, const double*,
                 double*, double*);
int ref_conv_bwd(int, int, int, int, int, const double*, const double*, const double*, const double*,
                 const double*, const double*, double*, double*, double*, double*);

enum { B = 2, T = 70, H = 2, DK = 4, DV = 3 };
enum { NQ = B * T * H * DK, NV = B * T * H * DV, NT = B * T * H, NS = B * H * DK * DV };

static unsigned long long rng = 88172645463325252ull;
static double unif(void) {  /* xorshift64, uniform in (-1, 1) */
    rng ^= rng << 13;
    rng ^= rng >> 7;
    rng ^= rng << 17;
    return (double)(rng >> 11) / 4503599627370496.0 - 1.0;
}
static double* arr(size_t n, double lo, double hi) {
    double* p = malloc(n * sizeof(double));
    for (size_t i = 0; i < n; ++i) p[i] = lo + (hi - lo) * 0.5 * (unif() + 1.0);
    return p;
}
static double dot(const double* a, const double* b, size_t n) {
    double s = 0;
    for (size_t i = 0; i < n; ++i) s += a[i] * b[i];
    return s;
}

/* member: 0 GDN, 1 KDA, 2 GLA, 3 Mamba-2 */
static int member;
static double *q, *k, *v, *g, *beta, *S_in, *dO, *dS_out;

static double loss(void) {
    double* o = calloc(NV, sizeof(double));
    double* S = calloc(NS, sizeof(double));
    int rc = member == 0 ? ref_gdn_fwd(B, T, H, DK, DV, q, k, v, g, beta, S_in, o, S)
           : member == 1 ? ref_kda_fwd(B, T, H, DK, DV, q, k, v, g, beta, S_in, o, S)
           : member == 2 ? ref_gla_fwd(B, T, H, DK, DV, q, k, v, g, S_in, o, S)
                         : ref_m2_fwd(B, T, H, DK, DV, q, k, v, g, S_in, o, S);
    if (rc) { fprintf(stderr, "forward %d failed\n", member); exit(2); }
    const double L = dot(o, dO, NV) + dot(S, dS_out, NS);
    free(o);
    free(S);
    return L;
}

static int check(const char* name, double* x, const double* grad, size_t idx) {
    const double h = 1e-6, x0 = x[idx];
    x[idx] = x0 + h;
    const double lp = loss();
    x[idx] = x0 - h;
    const double lm = loss();
    x[idx] = x0;
    const double fd = (lp - lm) / (2 * h), err = fabs(fd - grad[idx]) / fmax(1.0, fabs(fd));
    if (err > 1e-6) {
        fprintf(stderr, "member %d: d%s[%zu] adjoint %.9g, finite difference %.9g\n", member, name, idx, grad[idx], fd);
        return 1;
    }
    return 0;
}

int main(void) {
    int bad = 0;
    for (member = 0; member < 4; ++member) {
        const int per_channel = member == 1 || member == 2;
        const size_t ng = per_channel ? (size_t)NQ : (size_t)NT;
        q = arr(NQ, -1, 1); k = arr(NQ, -0.5, 0.5); v = arr(NV, -1, 1);
        g = arr(ng, -0.3, -0.01); beta = arr(NT, 0.1, 0.9);
        S_in = arr(NS, -0.2, 0.2); dO = arr(NV, -1, 1); dS_out = arr(NS, -1, 1);
        double *dq = calloc(NQ, 8), *dk = calloc(NQ, 8), *dv = calloc(NV, 8), *dg = calloc(ng, 8);
        double *db = calloc(NT, 8), *dS = calloc(NS, 8);
        int rc = member == 0 ? ref_gdn_bwd(B, T, H, DK, DV, q, k, v, g, beta, S_in, dO, dS_out, dq, dk, dv, dg, db, dS)
               : member == 1 ? ref_kda_bwd(B, T, H, DK, DV, q, k, v, g, beta, S_in, dO, dS_out, dq, dk, dv, dg, db, dS)
               : member == 2 ? ref_gla_bwd(B, T, H, DK, DV, q, k, v, g, S_in, dO, dS_out, dq, dk, dv, dg, dS)
                             : ref_m2_bwd(B, T, H, DK, DV, q, k, v, g, S_in, dO, dS_out, dq, dk, dv, dg, dS);
        if (rc) { fprintf(stderr, "backward %d failed\n", member); return 2; }
        /* a token before the checkpoint, one after it, and the boundary state */
        const size_t tq[2] = {(size_t)(5 * H + 1) * DK + 2, (size_t)(((size_t)T + 66) * H + 0) * DK + 1};
        const size_t tv[2] = {(size_t)(7 * H + 1) * DV + 1, (size_t)((T + 68) * H + 1) * DV + 2};
        const size_t tt[2] = {(size_t)(3 * H + 0), (size_t)((T + 65) * H + 1)};
        for (int i = 0; i < 2; ++i) {
            bad |= check("q", q, dq, tq[i]);
            bad |= check("k", k, dk, tq[i]);
            bad |= check("v", v, dv, tv[i]);
            bad |= check("g", g, dg, per_channel ? tq[i] : tt[i]);
            if (member <= 1) bad |= check("beta", beta, db, tt[i]);
        }
        bad |= check("S_in", S_in, dS, 5);
        bad |= check("S_in", S_in, dS, NS - 2);
        free(q); free(k); free(v); free(g); free(beta); free(S_in); free(dO); free(dS_out);
        free(dq); free(dk); free(dv); free(dg); free(db); free(dS);
    }
    /* short convolution: forward and backward with a carried state */
    {
        enum { CB = 2, CT = 9, CC = 8, CW = 4 };
        double *x = arr(CB * CT * CC, -1, 1), *w = arr(CC * CW, -1, 1), *bias = arr(CC, -0.1, 0.1);
        double *st = arr(CB * (CW - 1) * CC, -1, 1), *dy = arr(CB * CT * CC, -1, 1);
        double *dst = arr(CB * (CW - 1) * CC, -1, 1);
        double *y = calloc(CB * CT * CC, 8), *so = calloc(CB * (CW - 1) * CC, 8);
        double *dx = calloc(CB * CT * CC, 8), *dw = calloc(CC * CW, 8), *dbias = calloc(CC, 8);
        double *dsi = calloc(CB * (CW - 1) * CC, 8);
        for (int act = 0; act < 2; ++act) {
            if (ref_conv_fwd(CB, CT, CC, CW, act, x, w, bias, st, y, so)) return 2;
            if (ref_conv_bwd(CB, CT, CC, CW, act, x, w, bias, st, dy, dst, dx, dw, dbias, dsi)) return 2;
        }
        free(x); free(w); free(bias); free(st); free(dy); free(dst); free(y); free(so);
        free(dx); free(dw); free(dbias); free(dsi);
    }
    if (bad) return 1;
    printf("oracle sanitize: ok\n");
    return 0;
}
