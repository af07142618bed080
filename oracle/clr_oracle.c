/*
 * clr_oracle.c -- fp64 CPU oracle for the gated linear recurrence layer.
 *
 * TEST INFRASTRUCTURE ONLY.  This file is the slow, obviously-correct
 * reference that the GPU path is checked against.  Only the test suite, the
 * smoke check and the benchmark's CPU-baseline leg may load it; the product
 * library never links, calls or falls back to it, and it shares no code,
 * header or constant with the GPU sources.
 *
 * What it computes (plain definition, one token at a time, in fp64):
 *
 *   The layer family is the matrix-state recurrence of the StateFlow paper
 *   ("StateFlow: Sequence Pipeline Parallelism for Long-Context Modeling with
 *   Linear Recurrence", Sec. 2.1, Eq. 1), S_t = S_{t-1} F_t + v_t k_t^T,
 *   y_t = S_t q_t, with the structured transitions named in the same section:
 *     - Gated DeltaNet: F_t is scalar-plus-low-rank,
 *         F_t = alpha_t (I - beta_t k_t k_t^T),  write term beta_t v_t k_t^T;
 *     - Gated Linear Attention: per-key-channel (diagonal) decay alpha_t,
 *         write term v_t k_t^T;
 *     - Mamba-2: F_t is a scalar times the identity, write term v_t k_t^T;
 *     - Kimi Delta Attention (KDA): F_t is diagonal-plus-low-rank, the delta
 *       rule's erase factor after a per-key-channel decay.
 *   Here the state is stored key-major, S in R^{dk x dv} (the transpose of the
 *   paper's value-major S), so the same maps read
 *     GDN:     S_t = alpha_t (I - beta_t k_t k_t^T) S_{t-1} + beta_t k_t v_t^T
 *     GLA:     S_t = Diag(alpha_t) S_{t-1} + k_t v_t^T     (alpha_t in R^dk)
 *     Mamba-2: S_t = alpha_t S_{t-1} + k_t v_t^T            (alpha_t scalar)
 *     KDA:     S_t = (I - beta_t k_t k_t^T) Diag(alpha_t) S_{t-1} + beta_t k_t v_t^T
 *     all: o_t = S_t^T q_t,   alpha_t = exp(g_t)  (g = log alpha <= 0).
 *
 *   The chunk entry points take a boundary state S_in and return S_out (the
 *   chunk forward of the StateFlow paper, Sec. 3.1, "Forward Computation"),
 *   and the backward takes dS_out and returns dS_in (Sec. 3.1, "Backward
 *   Computation"), so that chaining S_out -> S_in forward and dS_in -> dS_out
 *   backward over sequence chunks reproduces the unchunked run.
 *
 *   Gradients are the vector-Jacobian products of
 *       (q, k, v, g, beta, S_in) -> (o, S_out)
 *   for upstream (dO, dS_out), i.e. the gradient of
 *       L = sum_t <dO_t, o_t> + <dS_out, S_out>_F,
 *   obtained by hand-derived reverse-mode adjoints of the per-token update
 *   (derivation in the comments of gdn_token_bwd / gla_token_bwd).
 *
 * The backward recomputes the forward states from checkpoints taken every
 * CKPT tokens.  Recomputation repeats the forward's exact operation order, so
 * a sequence split into chunks (with state passing) gives bit-identical
 * results to the unsplit run.
 *
 * Layouts (all contiguous, row-major, fp64, host memory):
 *   q, k        [B, T, H, dk]
 *   v, o, dO    [B, T, H, dv]
 *   g           GDN, Mamba-2: [B, T, H]       GLA, KDA: [B, T, H, dk]
 *   beta        GDN, KDA: [B, T, H]  (GLA and Mamba-2 have none)
 *   S_in, S_out, dS_in, dS_out   [B, H, dk, dv]
 * S_in / dS_out may be NULL (zero); S_out may be NULL (not wanted).
 * Return 0 on success, -1 on bad arguments or allocation failure.
 */
#include <math.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define CKPT 64

static int g_threads = 0;

void ref_set_threads(int n) { g_threads = n; }

int ref_get_max_threads(void)
{
#ifdef _OPENMP
    return g_threads > 0 ? g_threads : omp_get_max_threads();
#else
    return 1;
#endif
}

/* Offsets of token t of head h in batch b, and of the state of (b, h). */
static size_t tok(int b, int t, int h, int T, int H, int d)
{
    return (((size_t)b * T + t) * H + h) * (size_t)d;
}
static size_t hd(int b, int t, int h, int T, int H)
{
    return ((size_t)b * T + t) * H + h;
}
static size_t st(int b, int h, int H, int dk, int dv)
{
    return ((size_t)b * H + h) * (size_t)dk * dv;
}

/* ------------------------------------------------------------------------ */
/* Gated DeltaNet                                                             */
/* ------------------------------------------------------------------------ */

/*
 * One GDN token, in delta form:
 *   a     = S^T k                 (dv)
 *   delta = v - alpha a           (dv)
 *   S    <- alpha S + beta k delta^T
 * which equals alpha (I - beta k k^T) S + beta k v^T.  a_out receives a.
 */
static void gdn_token_fwd(double *S, const double *kt, const double *vt,
                          double alpha, double beta, int dk, int dv,
                          double *a_out)
{
    for (int j = 0; j < dv; ++j) a_out[j] = 0.0;
    for (int i = 0; i < dk; ++i) {
        const double ki = kt[i];
        const double *Si = S + (size_t)i * dv;
        for (int j = 0; j < dv; ++j) a_out[j] += Si[j] * ki;
    }
    for (int i = 0; i < dk; ++i) {
        const double bki = beta * kt[i];
        double *Si = S + (size_t)i * dv;
        for (int j = 0; j < dv; ++j)
            Si[j] = alpha * Si[j] + bki * (vt[j] - alpha * a_out[j]);
    }
}

/* o = S^T q */
static void out_token(const double *S, const double *qt, int dk, int dv,
                      double *ot)
{
    for (int j = 0; j < dv; ++j) ot[j] = 0.0;
    for (int i = 0; i < dk; ++i) {
        const double qi = qt[i];
        const double *Si = S + (size_t)i * dv;
        for (int j = 0; j < dv; ++j) ot[j] += Si[j] * qi;
    }
}

static void load_state(double *S, const double *S_in, size_t off, size_t n)
{
    if (S_in) memcpy(S, S_in + off, n * sizeof(double));
    else memset(S, 0, n * sizeof(double));
}

int ref_gdn_fwd(int B, int T, int H, int dk, int dv,
                const double *q, const double *k, const double *v,
                const double *g, const double *beta, const double *S_in,
                double *o, double *S_out)
{
    if (B < 0 || T < 0 || H < 0 || dk <= 0 || dv <= 0) return -1;
    if (!q || !k || !v || !g || !beta || !o) return -1;
    const size_t ns = (size_t)dk * dv;
    int fail = 0;
#pragma omp parallel for schedule(dynamic, 1) num_threads(ref_get_max_threads()) reduction(|:fail)
    for (int bh = 0; bh < B * H; ++bh) {
        const int b = bh / H, h = bh % H;
        double *S = (double *)malloc(ns * sizeof(double));
        double *a = (double *)malloc((size_t)dv * sizeof(double));
        if (!S || !a) { free(S); free(a); fail |= 1; continue; }
        load_state(S, S_in, st(b, h, H, dk, dv), ns);
        for (int t = 0; t < T; ++t) {
            const double alpha = exp(g[hd(b, t, h, T, H)]);
            gdn_token_fwd(S, k + tok(b, t, h, T, H, dk), v + tok(b, t, h, T, H, dv),
                          alpha, beta[hd(b, t, h, T, H)], dk, dv, a);
            out_token(S, q + tok(b, t, h, T, H, dk), dk, dv, o + tok(b, t, h, T, H, dv));
        }
        if (S_out) memcpy(S_out + st(b, h, H, dk, dv), S, ns * sizeof(double));
        free(S);
        free(a);
    }
    return fail ? -1 : 0;
}

/*
 * Reverse-mode step for one GDN token.  On entry dS holds dL/dS_t from the
 * future (tokens > t) and Sp holds S_{t-1}; St holds S_t.  Derivation, with
 * S_t = alpha S_{t-1} + beta k delta^T, delta = v - alpha S_{t-1}^T k:
 *   dS_t   += q do^T                    (o_t = S_t^T q)
 *   dq      = S_t do
 *   ddelta  = beta dS_t^T k             -> dv = ddelta
 *   dbeta   = k^T dS_t delta
 *   dk      = beta dS_t delta - alpha S_{t-1} ddelta
 *   dalpha  = <dS_t, S_{t-1}> - (S_{t-1}^T k) . ddelta,  dg = alpha dalpha
 *   dS_{t-1} = alpha (dS_t - k ddelta^T)   ( = alpha (I - beta k k^T) dS_t )
 */
static void gdn_token_bwd(double *dS, const double *Sp, const double *St,
                          const double *qt, const double *kt, const double *vt,
                          const double *dot, double alpha, double beta,
                          int dk, int dv, double *dqt, double *dkt, double *dvt,
                          double *dg_out, double *dbeta_out, double *a,
                          double *delta, double *dd)
{
    /* dS_t += q do^T ; dq = S_t do */
    for (int i = 0; i < dk; ++i) {
        double *dSi = dS + (size_t)i * dv;
        const double *Si = St + (size_t)i * dv;
        double acc = 0.0;
        for (int j = 0; j < dv; ++j) {
            dSi[j] += qt[i] * dot[j];
            acc += Si[j] * dot[j];
        }
        dqt[i] = acc;
    }
    /* a = S_{t-1}^T k ; delta = v - alpha a */
    for (int j = 0; j < dv; ++j) a[j] = 0.0;
    for (int i = 0; i < dk; ++i)
        for (int j = 0; j < dv; ++j) a[j] += Sp[(size_t)i * dv + j] * kt[i];
    for (int j = 0; j < dv; ++j) delta[j] = vt[j] - alpha * a[j];
    /* ddelta = beta dS^T k */
    for (int j = 0; j < dv; ++j) dd[j] = 0.0;
    for (int i = 0; i < dk; ++i)
        for (int j = 0; j < dv; ++j) dd[j] += dS[(size_t)i * dv + j] * kt[i];
    for (int j = 0; j < dv; ++j) {
        dd[j] *= beta;
        dvt[j] = dd[j];
    }
    /* dbeta = k^T dS delta ; dk = beta dS delta - alpha S_{t-1} ddelta ;
       <dS, S_{t-1}> */
    double dbeta = 0.0, frob = 0.0, adot = 0.0;
    for (int i = 0; i < dk; ++i) {
        const double *dSi = dS + (size_t)i * dv;
        const double *Spi = Sp + (size_t)i * dv;
        double x = 0.0, y = 0.0;
        for (int j = 0; j < dv; ++j) {
            x += dSi[j] * delta[j];
            y += Spi[j] * dd[j];
            frob += dSi[j] * Spi[j];
        }
        dbeta += kt[i] * x;
        dkt[i] = beta * x - alpha * y;
    }
    for (int j = 0; j < dv; ++j) adot += a[j] * dd[j];
    *dbeta_out = dbeta;
    *dg_out = alpha * (frob - adot);
    /* dS_{t-1} = alpha (dS - k ddelta^T) */
    for (int i = 0; i < dk; ++i) {
        double *dSi = dS + (size_t)i * dv;
        for (int j = 0; j < dv; ++j) dSi[j] = alpha * (dSi[j] - kt[i] * dd[j]);
    }
}

int ref_gdn_bwd(int B, int T, int H, int dk, int dv,
                const double *q, const double *k, const double *v,
                const double *g, const double *beta, const double *S_in,
                const double *dO, const double *dS_out,
                double *dq, double *dk_, double *dv_, double *dg,
                double *dbeta, double *dS_in)
{
    if (B < 0 || T < 0 || H < 0 || dk <= 0 || dv <= 0) return -1;
    if (!q || !k || !v || !g || !beta || !dO) return -1;
    if (!dq || !dk_ || !dv_ || !dg || !dbeta || !dS_in) return -1;
    const size_t ns = (size_t)dk * dv;
    const int nck = T / CKPT + 1; /* checkpoints at t = 0, CKPT, 2 CKPT, ... */
    int fail = 0;
#pragma omp parallel for schedule(dynamic, 1) num_threads(ref_get_max_threads()) reduction(|:fail)
    for (int bh = 0; bh < B * H; ++bh) {
        const int b = bh / H, h = bh % H;
        double *ck = (double *)malloc((size_t)nck * ns * sizeof(double));
        double *seg = (double *)malloc((size_t)(CKPT + 1) * ns * sizeof(double));
        double *dS = (double *)malloc(ns * sizeof(double));
        double *tmp = (double *)malloc((size_t)4 * dv * sizeof(double));
        if (!ck || !seg || !dS || !tmp) {
            free(ck); free(seg); free(dS); free(tmp);
            fail |= 1;
            continue;
        }
        double *a = tmp, *delta = tmp + dv, *dd = tmp + 2 * dv;
        /* forward pass, keeping the state every CKPT tokens */
        double *S = seg; /* scratch while checkpointing */
        load_state(S, S_in, st(b, h, H, dk, dv), ns);
        for (int t = 0; t < T; ++t) {
            if (t % CKPT == 0) memcpy(ck + (size_t)(t / CKPT) * ns, S, ns * sizeof(double));
            gdn_token_fwd(S, k + tok(b, t, h, T, H, dk), v + tok(b, t, h, T, H, dv),
                          exp(g[hd(b, t, h, T, H)]), beta[hd(b, t, h, T, H)], dk, dv, a);
        }
        /* reverse pass, segment by segment */
        if (dS_out) memcpy(dS, dS_out + st(b, h, H, dk, dv), ns * sizeof(double));
        else memset(dS, 0, ns * sizeof(double));
        const int nseg = (T + CKPT - 1) / CKPT;
        for (int sgi = nseg - 1; sgi >= 0; --sgi) {
            const int t0 = sgi * CKPT;
            const int t1 = (t0 + CKPT < T) ? t0 + CKPT : T;
            /* seg[j] = S_{t0 + j - 1}, i.e. seg[0] = state before token t0 */
            memcpy(seg, ck + (size_t)sgi * ns, ns * sizeof(double));
            for (int t = t0; t < t1; ++t) {
                double *nx = seg + (size_t)(t - t0 + 1) * ns;
                memcpy(nx, seg + (size_t)(t - t0) * ns, ns * sizeof(double));
                gdn_token_fwd(nx, k + tok(b, t, h, T, H, dk), v + tok(b, t, h, T, H, dv),
                              exp(g[hd(b, t, h, T, H)]), beta[hd(b, t, h, T, H)], dk, dv, a);
            }
            for (int t = t1 - 1; t >= t0; --t) {
                const size_t ih = hd(b, t, h, T, H);
                gdn_token_bwd(dS, seg + (size_t)(t - t0) * ns, seg + (size_t)(t - t0 + 1) * ns,
                              q + tok(b, t, h, T, H, dk), k + tok(b, t, h, T, H, dk),
                              v + tok(b, t, h, T, H, dv), dO + tok(b, t, h, T, H, dv),
                              exp(g[ih]), beta[ih], dk, dv,
                              dq + tok(b, t, h, T, H, dk), dk_ + tok(b, t, h, T, H, dk),
                              dv_ + tok(b, t, h, T, H, dv), dg + ih, dbeta + ih, a, delta, dd);
            }
        }
        memcpy(dS_in + st(b, h, H, dk, dv), dS, ns * sizeof(double));
        free(ck); free(seg); free(dS); free(tmp);
    }
    return fail ? -1 : 0;
}

/* ------------------------------------------------------------------------ */
/* Gated Linear Attention (per-key-channel diagonal gate, no delta term)      */
/* ------------------------------------------------------------------------ */

/* S <- Diag(exp(g)) S + k v^T */
static void gla_token_fwd(double *S, const double *kt, const double *vt,
                          const double *gt, int dk, int dv)
{
    for (int i = 0; i < dk; ++i) {
        const double al = exp(gt[i]);
        double *Si = S + (size_t)i * dv;
        for (int j = 0; j < dv; ++j) Si[j] = al * Si[j] + kt[i] * vt[j];
    }
}

int ref_gla_fwd(int B, int T, int H, int dk, int dv,
                const double *q, const double *k, const double *v,
                const double *g, const double *S_in, double *o, double *S_out)
{
    if (B < 0 || T < 0 || H < 0 || dk <= 0 || dv <= 0) return -1;
    if (!q || !k || !v || !g || !o) return -1;
    const size_t ns = (size_t)dk * dv;
    int fail = 0;
#pragma omp parallel for schedule(dynamic, 1) num_threads(ref_get_max_threads()) reduction(|:fail)
    for (int bh = 0; bh < B * H; ++bh) {
        const int b = bh / H, h = bh % H;
        double *S = (double *)malloc(ns * sizeof(double));
        if (!S) { fail |= 1; continue; }
        load_state(S, S_in, st(b, h, H, dk, dv), ns);
        for (int t = 0; t < T; ++t) {
            gla_token_fwd(S, k + tok(b, t, h, T, H, dk), v + tok(b, t, h, T, H, dv),
                          g + tok(b, t, h, T, H, dk), dk, dv);
            out_token(S, q + tok(b, t, h, T, H, dk), dk, dv, o + tok(b, t, h, T, H, dv));
        }
        if (S_out) memcpy(S_out + st(b, h, H, dk, dv), S, ns * sizeof(double));
        free(S);
    }
    return fail ? -1 : 0;
}

/*
 * Reverse-mode step for one GLA token, S_t = Diag(alpha) S_{t-1} + k v^T:
 *   dS_t     += q do^T ;  dq = S_t do
 *   dk        = dS_t v ;  dv = dS_t^T k
 *   dalpha_i  = sum_j dS_t[i,j] S_{t-1}[i,j] ,  dg_i = alpha_i dalpha_i
 *   dS_{t-1}  = Diag(alpha) dS_t
 */
static void gla_token_bwd(double *dS, const double *Sp, const double *St,
                          const double *qt, const double *kt, const double *vt,
                          const double *dot, const double *gt, int dk, int dv,
                          double *dqt, double *dkt, double *dvt, double *dgt)
{
    for (int i = 0; i < dk; ++i) {
        double *dSi = dS + (size_t)i * dv;
        const double *Si = St + (size_t)i * dv;
        double acc = 0.0;
        for (int j = 0; j < dv; ++j) {
            dSi[j] += qt[i] * dot[j];
            acc += Si[j] * dot[j];
        }
        dqt[i] = acc;
    }
    for (int j = 0; j < dv; ++j) dvt[j] = 0.0;
    for (int i = 0; i < dk; ++i) {
        const double *dSi = dS + (size_t)i * dv;
        const double *Spi = Sp + (size_t)i * dv;
        double x = 0.0, frob = 0.0;
        for (int j = 0; j < dv; ++j) {
            x += dSi[j] * vt[j];
            frob += dSi[j] * Spi[j];
            dvt[j] += dSi[j] * kt[i];
        }
        dkt[i] = x;
        const double al = exp(gt[i]);
        dgt[i] = al * frob;
    }
    for (int i = 0; i < dk; ++i) {
        const double al = exp(gt[i]);
        double *dSi = dS + (size_t)i * dv;
        for (int j = 0; j < dv; ++j) dSi[j] *= al;
    }
}

int ref_gla_bwd(int B, int T, int H, int dk, int dv,
                const double *q, const double *k, const double *v,
                const double *g, const double *S_in, const double *dO,
                const double *dS_out, double *dq, double *dk_, double *dv_,
                double *dg, double *dS_in)
{
    if (B < 0 || T < 0 || H < 0 || dk <= 0 || dv <= 0) return -1;
    if (!q || !k || !v || !g || !dO) return -1;
    if (!dq || !dk_ || !dv_ || !dg || !dS_in) return -1;
    const size_t ns = (size_t)dk * dv;
    const int nck = T / CKPT + 1;
    int fail = 0;
#pragma omp parallel for schedule(dynamic, 1) num_threads(ref_get_max_threads()) reduction(|:fail)
    for (int bh = 0; bh < B * H; ++bh) {
        const int b = bh / H, h = bh % H;
        double *ck = (double *)malloc((size_t)nck * ns * sizeof(double));
        double *seg = (double *)malloc((size_t)(CKPT + 1) * ns * sizeof(double));
        double *dS = (double *)malloc(ns * sizeof(double));
        if (!ck || !seg || !dS) {
            free(ck); free(seg); free(dS);
            fail |= 1;
            continue;
        }
        double *S = seg;
        load_state(S, S_in, st(b, h, H, dk, dv), ns);
        for (int t = 0; t < T; ++t) {
            if (t % CKPT == 0) memcpy(ck + (size_t)(t / CKPT) * ns, S, ns * sizeof(double));
            gla_token_fwd(S, k + tok(b, t, h, T, H, dk), v + tok(b, t, h, T, H, dv),
                          g + tok(b, t, h, T, H, dk), dk, dv);
        }
        if (dS_out) memcpy(dS, dS_out + st(b, h, H, dk, dv), ns * sizeof(double));
        else memset(dS, 0, ns * sizeof(double));
        const int nseg = (T + CKPT - 1) / CKPT;
        for (int sgi = nseg - 1; sgi >= 0; --sgi) {
            const int t0 = sgi * CKPT;
            const int t1 = (t0 + CKPT < T) ? t0 + CKPT : T;
            memcpy(seg, ck + (size_t)sgi * ns, ns * sizeof(double));
            for (int t = t0; t < t1; ++t) {
                double *nx = seg + (size_t)(t - t0 + 1) * ns;
                memcpy(nx, seg + (size_t)(t - t0) * ns, ns * sizeof(double));
                gla_token_fwd(nx, k + tok(b, t, h, T, H, dk), v + tok(b, t, h, T, H, dv),
                              g + tok(b, t, h, T, H, dk), dk, dv);
            }
            for (int t = t1 - 1; t >= t0; --t) {
                gla_token_bwd(dS, seg + (size_t)(t - t0) * ns, seg + (size_t)(t - t0 + 1) * ns,
                              q + tok(b, t, h, T, H, dk), k + tok(b, t, h, T, H, dk),
                              v + tok(b, t, h, T, H, dv), dO + tok(b, t, h, T, H, dv),
                              g + tok(b, t, h, T, H, dk), dk, dv,
                              dq + tok(b, t, h, T, H, dk), dk_ + tok(b, t, h, T, H, dk),
                              dv_ + tok(b, t, h, T, H, dv), dg + tok(b, t, h, T, H, dk));
            }
        }
        memcpy(dS_in + st(b, h, H, dk, dv), dS, ns * sizeof(double));
        free(ck); free(seg); free(dS);
    }
    return fail ? -1 : 0;
}

/* ------------------------------------------------------------------------ */
/* Mamba-2 (scalar gate, no delta term)                                       */
/* ------------------------------------------------------------------------ */

/* S <- exp(g) S + k v^T  (one scalar decay for the whole state) */
static void m2_token_fwd(double *S, const double *kt, const double *vt,
                         double gt, int dk, int dv)
{
    const double al = exp(gt);
    for (int i = 0; i < dk; ++i)
        for (int j = 0; j < dv; ++j)
            S[(size_t)i * dv + j] = al * S[(size_t)i * dv + j] + kt[i] * vt[j];
}

int ref_m2_fwd(int B, int T, int H, int dk, int dv,
               const double *q, const double *k, const double *v,
               const double *g, const double *S_in, double *o, double *S_out)
{
    if (B < 0 || T < 0 || H < 0 || dk <= 0 || dv <= 0) return -1;
    if (!q || !k || !v || !g || !o) return -1;
    const size_t ns = (size_t)dk * dv;
    int fail = 0;
#pragma omp parallel for schedule(dynamic, 1) num_threads(ref_get_max_threads()) reduction(|:fail)
    for (int bh = 0; bh < B * H; ++bh) {
        const int b = bh / H, h = bh % H;
        double *S = (double *)malloc(ns * sizeof(double));
        if (!S) { fail |= 1; continue; }
        load_state(S, S_in, st(b, h, H, dk, dv), ns);
        for (int t = 0; t < T; ++t) {
            m2_token_fwd(S, k + tok(b, t, h, T, H, dk), v + tok(b, t, h, T, H, dv),
                         g[hd(b, t, h, T, H)], dk, dv);
            out_token(S, q + tok(b, t, h, T, H, dk), dk, dv, o + tok(b, t, h, T, H, dv));
        }
        if (S_out) memcpy(S_out + st(b, h, H, dk, dv), S, ns * sizeof(double));
        free(S);
    }
    return fail ? -1 : 0;
}

/*
 * Reverse-mode step for one token, S_t = alpha S_{t-1} + k v^T, o = S_t^T q:
 *   dS_t     += q do^T ;  dq = S_t do
 *   dk        = dS_t v ;  dv = dS_t^T k
 *   dalpha    = <dS_t, S_{t-1}>_F ,  dg = alpha dalpha
 *   dS_{t-1}  = alpha dS_t
 */
static void m2_token_bwd(double *dS, const double *Sp, const double *St,
                         const double *qt, const double *kt, const double *vt,
                         const double *dot, double gt, int dk, int dv,
                         double *dqt, double *dkt, double *dvt, double *dgt)
{
    const double al = exp(gt);
    for (int i = 0; i < dk; ++i) {
        double *dSi = dS + (size_t)i * dv;
        const double *Si = St + (size_t)i * dv;
        double acc = 0.0;
        for (int j = 0; j < dv; ++j) {
            dSi[j] += qt[i] * dot[j];
            acc += Si[j] * dot[j];
        }
        dqt[i] = acc;
    }
    /* dk_i = sum_j dS[i,j] v_j */
    for (int i = 0; i < dk; ++i) {
        double x = 0.0;
        for (int j = 0; j < dv; ++j) x += dS[(size_t)i * dv + j] * vt[j];
        dkt[i] = x;
    }
    /* dv_j = sum_i dS[i,j] k_i */
    for (int j = 0; j < dv; ++j) {
        double y = 0.0;
        for (int i = 0; i < dk; ++i) y += dS[(size_t)i * dv + j] * kt[i];
        dvt[j] = y;
    }
    /* dg = alpha <dS_t, S_{t-1}>_F */
    double frob = 0.0;
    for (size_t e = 0; e < (size_t)dk * dv; ++e) frob += dS[e] * Sp[e];
    *dgt = al * frob;
    for (size_t e = 0; e < (size_t)dk * dv; ++e) dS[e] *= al;
}

int ref_m2_bwd(int B, int T, int H, int dk, int dv,
               const double *q, const double *k, const double *v,
               const double *g, const double *S_in, const double *dO,
               const double *dS_out, double *dq, double *dk_, double *dv_,
               double *dg, double *dS_in)
{
    if (B < 0 || T < 0 || H < 0 || dk <= 0 || dv <= 0) return -1;
    if (!q || !k || !v || !g || !dO) return -1;
    if (!dq || !dk_ || !dv_ || !dg || !dS_in) return -1;
    const size_t ns = (size_t)dk * dv;
    const int nck = T / CKPT + 1;
    int fail = 0;
#pragma omp parallel for schedule(dynamic, 1) num_threads(ref_get_max_threads()) reduction(|:fail)
    for (int bh = 0; bh < B * H; ++bh) {
        const int b = bh / H, h = bh % H;
        double *ck = (double *)malloc((size_t)nck * ns * sizeof(double));
        double *seg = (double *)malloc((size_t)(CKPT + 1) * ns * sizeof(double));
        double *dS = (double *)malloc(ns * sizeof(double));
        if (!ck || !seg || !dS) {
            free(ck); free(seg); free(dS);
            fail |= 1;
            continue;
        }
        double *S = seg;
        load_state(S, S_in, st(b, h, H, dk, dv), ns);
        for (int t = 0; t < T; ++t) {
            if (t % CKPT == 0) memcpy(ck + (size_t)(t / CKPT) * ns, S, ns * sizeof(double));
            m2_token_fwd(S, k + tok(b, t, h, T, H, dk), v + tok(b, t, h, T, H, dv),
                         g[hd(b, t, h, T, H)], dk, dv);
        }
        if (dS_out) memcpy(dS, dS_out + st(b, h, H, dk, dv), ns * sizeof(double));
        else memset(dS, 0, ns * sizeof(double));
        const int nseg = (T + CKPT - 1) / CKPT;
        for (int sgi = nseg - 1; sgi >= 0; --sgi) {
            const int t0 = sgi * CKPT;
            const int t1 = (t0 + CKPT < T) ? t0 + CKPT : T;
            memcpy(seg, ck + (size_t)sgi * ns, ns * sizeof(double));
            for (int t = t0; t < t1; ++t) {
                double *nx = seg + (size_t)(t - t0 + 1) * ns;
                memcpy(nx, seg + (size_t)(t - t0) * ns, ns * sizeof(double));
                m2_token_fwd(nx, k + tok(b, t, h, T, H, dk), v + tok(b, t, h, T, H, dv),
                             g[hd(b, t, h, T, H)], dk, dv);
            }
            for (int t = t1 - 1; t >= t0; --t) {
                m2_token_bwd(dS, seg + (size_t)(t - t0) * ns, seg + (size_t)(t - t0 + 1) * ns,
                             q + tok(b, t, h, T, H, dk), k + tok(b, t, h, T, H, dk),
                             v + tok(b, t, h, T, H, dv), dO + tok(b, t, h, T, H, dv),
                             g[hd(b, t, h, T, H)], dk, dv,
                             dq + tok(b, t, h, T, H, dk), dk_ + tok(b, t, h, T, H, dk),
                             dv_ + tok(b, t, h, T, H, dv), dg + hd(b, t, h, T, H));
            }
        }
        memcpy(dS_in + st(b, h, H, dk, dv), dS, ns * sizeof(double));
        free(ck); free(seg); free(dS);
    }
    return fail ? -1 : 0;
}

/* ------------------------------------------------------------------------ */
/* KDA (per-channel decay, delta-rule erase and write)                        */
/* ------------------------------------------------------------------------ */

/*
 * One KDA token, in delta form with the decayed state S' = Diag(alpha) S:
 *   a     = S'^T k                (dv)
 *   delta = v - a                 (dv)
 *   S    <- S' + beta k delta^T
 * which equals (I - beta k k^T) Diag(alpha) S + beta k v^T.
 */
static void kda_token_fwd(double *S, const double *kt, const double *vt,
                          const double *gt, double beta, int dk, int dv,
                          double *a_out)
{
    for (int i = 0; i < dk; ++i) {
        const double al = exp(gt[i]);
        double *Si = S + (size_t)i * dv;
        for (int j = 0; j < dv; ++j) Si[j] *= al;
    }
    for (int j = 0; j < dv; ++j) a_out[j] = 0.0;
    for (int i = 0; i < dk; ++i)
        for (int j = 0; j < dv; ++j) a_out[j] += S[(size_t)i * dv + j] * kt[i];
    for (int i = 0; i < dk; ++i) {
        const double bk = beta * kt[i];
        double *Si = S + (size_t)i * dv;
        for (int j = 0; j < dv; ++j) Si[j] += bk * (vt[j] - a_out[j]);
    }
}

int ref_kda_fwd(int B, int T, int H, int dk, int dv,
                const double *q, const double *k, const double *v,
                const double *g, const double *beta, const double *S_in,
                double *o, double *S_out)
{
    if (B < 0 || T < 0 || H < 0 || dk <= 0 || dv <= 0) return -1;
    if (!q || !k || !v || !g || !beta || !o) return -1;
    const size_t ns = (size_t)dk * dv;
    int fail = 0;
#pragma omp parallel for schedule(dynamic, 1) num_threads(ref_get_max_threads()) reduction(|:fail)
    for (int bh = 0; bh < B * H; ++bh) {
        const int b = bh / H, h = bh % H;
        double *S = (double *)malloc(ns * sizeof(double));
        double *a = (double *)malloc((size_t)dv * sizeof(double));
        if (!S || !a) { free(S); free(a); fail |= 1; continue; }
        load_state(S, S_in, st(b, h, H, dk, dv), ns);
        for (int t = 0; t < T; ++t) {
            kda_token_fwd(S, k + tok(b, t, h, T, H, dk), v + tok(b, t, h, T, H, dv),
                          g + tok(b, t, h, T, H, dk), beta[hd(b, t, h, T, H)], dk, dv, a);
            out_token(S, q + tok(b, t, h, T, H, dk), dk, dv, o + tok(b, t, h, T, H, dv));
        }
        if (S_out) memcpy(S_out + st(b, h, H, dk, dv), S, ns * sizeof(double));
        free(S);
        free(a);
    }
    return fail ? -1 : 0;
}

/*
 * Reverse-mode step for one KDA token.  With S' = Diag(alpha) S_{t-1},
 * a = S'^T k, delta = v - a, S_t = S' + beta k delta^T, o = S_t^T q:
 *   dS_t      += q do^T ;  dq = S_t do
 *   dbeta      = k^T dS_t delta
 *   dk         = beta dS_t delta          (write term)
 *   ddelta     = beta dS_t^T k ;  dv = ddelta ;  da = -ddelta
 *   dS'        = dS_t + k da^T
 *   dk        += S' da                    (erase term)
 *   dalpha_i   = sum_j dS'[i,j] S_{t-1}[i,j],  dg_i = alpha_i dalpha_i
 *   dS_{t-1}   = Diag(alpha) dS'
 * Sp is S_{t-1}, St is S_t.
 */
static void kda_token_bwd(double *dS, const double *Sp, const double *St,
                          const double *qt, const double *kt, const double *vt,
                          const double *dot, const double *gt, double beta,
                          int dk, int dv, double *dqt, double *dkt,
                          double *dvt, double *dgt, double *dbt, double *wrk)
{
    double *Sd = wrk;             /* S' (dk x dv) */
    double *dl = wrk + (size_t)dk * dv;  /* delta, then ddelta (dv) */
    double *aa = dl + dv;                 /* a (dv) */
    for (int i = 0; i < dk; ++i) {
        const double al = exp(gt[i]);
        for (int j = 0; j < dv; ++j) Sd[(size_t)i * dv + j] = al * Sp[(size_t)i * dv + j];
    }
    for (int j = 0; j < dv; ++j) {
        double x = 0.0;
        for (int i = 0; i < dk; ++i) x += Sd[(size_t)i * dv + j] * kt[i];
        aa[j] = x;
        dl[j] = vt[j] - x;
    }
    /* output */
    for (int i = 0; i < dk; ++i) {
        double acc = 0.0;
        for (int j = 0; j < dv; ++j) {
            dS[(size_t)i * dv + j] += qt[i] * dot[j];
            acc += St[(size_t)i * dv + j] * dot[j];
        }
        dqt[i] = acc;
    }
    /* write term */
    double db = 0.0;
    for (int i = 0; i < dk; ++i) {
        double x = 0.0;
        for (int j = 0; j < dv; ++j) x += dS[(size_t)i * dv + j] * dl[j];
        dkt[i] = beta * x;
        db += kt[i] * x;
    }
    *dbt = db;
    /* ddelta = beta dS^T k, reusing dl */
    for (int j = 0; j < dv; ++j) {
        double y = 0.0;
        for (int i = 0; i < dk; ++i) y += kt[i] * dS[(size_t)i * dv + j];
        dl[j] = beta * y;
        dvt[j] = dl[j];
    }
    /* erase term: dS' = dS - k ddelta^T, dk -= S' ddelta */
    for (int i = 0; i < dk; ++i) {
        double x = 0.0;
        for (int j = 0; j < dv; ++j) {
            x += Sd[(size_t)i * dv + j] * dl[j];
            dS[(size_t)i * dv + j] -= kt[i] * dl[j];
        }
        dkt[i] -= x;
    }
    /* decay */
    for (int i = 0; i < dk; ++i) {
        const double al = exp(gt[i]);
        double frob = 0.0;
        for (int j = 0; j < dv; ++j) frob += dS[(size_t)i * dv + j] * Sp[(size_t)i * dv + j];
        dgt[i] = frob * al;
        for (int j = 0; j < dv; ++j) dS[(size_t)i * dv + j] *= al;
    }
}

int ref_kda_bwd(int B, int T, int H, int dk, int dv,
                const double *q, const double *k, const double *v,
                const double *g, const double *beta, const double *S_in,
                const double *dO, const double *dS_out, double *dq, double *dk_,
                double *dv_, double *dg, double *dbeta, double *dS_in)
{
    if (B < 0 || T < 0 || H < 0 || dk <= 0 || dv <= 0) return -1;
    if (!q || !k || !v || !g || !beta || !dO) return -1;
    if (!dq || !dk_ || !dv_ || !dg || !dbeta || !dS_in) return -1;
    const size_t ns = (size_t)dk * dv;
    const int nck = T / CKPT + 1;
    int fail = 0;
#pragma omp parallel for schedule(dynamic, 1) num_threads(ref_get_max_threads()) reduction(|:fail)
    for (int bh = 0; bh < B * H; ++bh) {
        const int b = bh / H, h = bh % H;
        double *ck = (double *)malloc((size_t)nck * ns * sizeof(double));
        double *seg = (double *)malloc((size_t)(CKPT + 1) * ns * sizeof(double));
        double *dS = (double *)malloc(ns * sizeof(double));
        double *wrk = (double *)malloc((ns + 2 * (size_t)dv) * sizeof(double));
        if (!ck || !seg || !dS || !wrk) {
            free(ck); free(seg); free(dS); free(wrk);
            fail |= 1;
            continue;
        }
        double *S = seg;
        load_state(S, S_in, st(b, h, H, dk, dv), ns);
        for (int t = 0; t < T; ++t) {
            if (t % CKPT == 0) memcpy(ck + (size_t)(t / CKPT) * ns, S, ns * sizeof(double));
            kda_token_fwd(S, k + tok(b, t, h, T, H, dk), v + tok(b, t, h, T, H, dv),
                          g + tok(b, t, h, T, H, dk), beta[hd(b, t, h, T, H)], dk, dv, wrk);
        }
        if (dS_out) memcpy(dS, dS_out + st(b, h, H, dk, dv), ns * sizeof(double));
        else memset(dS, 0, ns * sizeof(double));
        const int nseg = (T + CKPT - 1) / CKPT;
        for (int sgi = nseg - 1; sgi >= 0; --sgi) {
            const int t0 = sgi * CKPT;
            const int t1 = (t0 + CKPT < T) ? t0 + CKPT : T;
            memcpy(seg, ck + (size_t)sgi * ns, ns * sizeof(double));
            for (int t = t0; t < t1; ++t) {
                double *nx = seg + (size_t)(t - t0 + 1) * ns;
                memcpy(nx, seg + (size_t)(t - t0) * ns, ns * sizeof(double));
                kda_token_fwd(nx, k + tok(b, t, h, T, H, dk), v + tok(b, t, h, T, H, dv),
                              g + tok(b, t, h, T, H, dk), beta[hd(b, t, h, T, H)], dk, dv, wrk);
            }
            for (int t = t1 - 1; t >= t0; --t) {
                kda_token_bwd(dS, seg + (size_t)(t - t0) * ns, seg + (size_t)(t - t0 + 1) * ns,
                              q + tok(b, t, h, T, H, dk), k + tok(b, t, h, T, H, dk),
                              v + tok(b, t, h, T, H, dv), dO + tok(b, t, h, T, H, dv),
                              g + tok(b, t, h, T, H, dk), beta[hd(b, t, h, T, H)], dk, dv,
                              dq + tok(b, t, h, T, H, dk), dk_ + tok(b, t, h, T, H, dk),
                              dv_ + tok(b, t, h, T, H, dv), dg + tok(b, t, h, T, H, dk),
                              dbeta + hd(b, t, h, T, H), wrk);
            }
        }
        memcpy(dS_in + st(b, h, H, dk, dv), dS, ns * sizeof(double));
        free(ck); free(seg); free(dS); free(wrk);
    }
    return fail ? -1 : 0;
}
