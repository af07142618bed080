/*
 * conv_oracle.c -- fp64 CPU oracle for the causal short convolution with a
 * boundary state.
 *
 * TEST INFRASTRUCTURE ONLY (see clr_oracle.c): loaded by the tests, the smoke
 * check and the benchmark's CPU-baseline leg, never by the product library.
 *
 * What it computes.  The StateFlow paper (Sec. 1 and Sec. 3.3) requires the
 * local-convolution modules of a linear-recurrence layer to hand their
 * boundary state from one sequence chunk to the next, like the recurrent
 * state.  The pages do not define the convolution itself; the reading taken is
 * the depthwise causal convolution of width W used in front of such layers:
 * per batch b, channel c and token t of a chunk of T tokens,
 *     xe = [state_in ; x]          (W-1 carried rows, then the chunk's rows)
 *     z_t = bias_c + sum_{j=0}^{W-1} w[c][j] * xe[t + j]     (xe index from 0)
 *     y_t = act(z_t),  act = identity or SiLU (z * sigmoid(z))
 *     state_out = the last W-1 rows of xe
 * so the chunks of a split sequence reproduce the unsplit run exactly.
 * Gradients are those of L = sum <dy, y> + <dstate_out, state_out>:
 *     dz_t = dy_t * act'(z_t)
 *     dxe[s] = dstate_out part + sum_j w[c][j] dz_{s-j}  (over 0 <= s-j < T)
 *     dw[c][j] = sum_{b,t} dz_t xe[t + j],   dbias_c = sum_{b,t} dz_t
 *     dx = dxe[W-1 ..],  dstate_in = dxe[0 .. W-2].
 *
 * Layouts (contiguous, row-major, fp64): x, y, dy, dx [B, T, C];
 * state_in, state_out, dstate_out, dstate_in [B, W-1, C]; w, dw [C, W];
 * bias, dbias [C].  state_in / dstate_out / bias may be NULL (zero);
 * state_out may be NULL.  Returns 0, or -1 on bad arguments.
 */
#include <math.h>
#include <stdlib.h>
#include <string.h>

static double act_f(double z, int act)
{
    return act ? z / (1.0 + exp(-z)) : z;
}

/* derivative of act at z */
static double act_d(double z, int act)
{
    if (!act) return 1.0;
    const double s = 1.0 / (1.0 + exp(-z));
    return s * (1.0 + z * (1.0 - s));
}

/* xe[b][r][c] for r in [0, T + W - 1): state rows, then x rows */
static double xe_at(const double *x, const double *state_in, int b, int r, int c,
                    int T, int C, int W)
{
    if (r < W - 1)
        return state_in ? state_in[((size_t)b * (W - 1) + r) * C + c] : 0.0;
    return x[((size_t)b * T + (r - (W - 1))) * C + c];
}

int ref_conv_fwd(int B, int T, int C, int W, int act,
                 const double *x, const double *w, const double *bias,
                 const double *state_in, double *y, double *state_out)
{
    if (B < 0 || T < 0 || C <= 0 || W < 1 || !x || !w || !y) return -1;
    for (int b = 0; b < B; ++b)
        for (int t = 0; t < T; ++t)
            for (int c = 0; c < C; ++c) {
                double z = bias ? bias[c] : 0.0;
                for (int j = 0; j < W; ++j)
                    z += w[(size_t)c * W + j] * xe_at(x, state_in, b, t + j, c, T, C, W);
                y[((size_t)b * T + t) * C + c] = act_f(z, act);
            }
    if (state_out)
        for (int b = 0; b < B; ++b)
            for (int i = 0; i < W - 1; ++i)
                for (int c = 0; c < C; ++c)
                    state_out[((size_t)b * (W - 1) + i) * C + c] =
                        xe_at(x, state_in, b, T + i, c, T, C, W);
    return 0;
}

int ref_conv_bwd(int B, int T, int C, int W, int act,
                 const double *x, const double *w, const double *bias,
                 const double *state_in, const double *dy, const double *dstate_out,
                 double *dx, double *dw, double *dbias, double *dstate_in)
{
    if (B < 0 || T < 0 || C <= 0 || W < 1 || !x || !w || !dy || !dx || !dw || !dbias)
        return -1;
    if (W > 1 && !dstate_in) return -1;
    const int R = T + W - 1; /* rows of xe */
    double *dz = (double *)malloc((size_t)(T > 0 ? T : 1) * sizeof(double));
    double *dxe = (double *)malloc((size_t)(R > 0 ? R : 1) * sizeof(double));
    if (!dz || !dxe) { free(dz); free(dxe); return -1; }
    memset(dw, 0, (size_t)C * W * sizeof(double));
    memset(dbias, 0, (size_t)C * sizeof(double));
    for (int b = 0; b < B; ++b)
        for (int c = 0; c < C; ++c) {
            for (int t = 0; t < T; ++t) {
                double z = bias ? bias[c] : 0.0;
                for (int j = 0; j < W; ++j)
                    z += w[(size_t)c * W + j] * xe_at(x, state_in, b, t + j, c, T, C, W);
                dz[t] = dy[((size_t)b * T + t) * C + c] * act_d(z, act);
            }
            /* Row r of xe feeds z_t for t = r - j.  The sum starts from the
             * upstream gradient of state_out (rows T .. T + W - 2 of xe) and
             * takes the taps from the latest token back (j ascending).  In
             * this order a chunk's dstate_in, added first into the previous
             * chunk's last rows, continues the same left fold, so chunked and
             * unchunked runs give the same bits. */
            for (int r = 0; r < R; ++r) {
                double acc = (dstate_out && r >= T) ? dstate_out[((size_t)b * (W - 1) + (r - T)) * C + c] : 0.0;
                for (int j = 0; j < W; ++j) {
                    const int t = r - j;
                    if (t >= 0 && t < T) acc += w[(size_t)c * W + j] * dz[t];
                }
                dxe[r] = acc;
            }
            for (int t = 0; t < T; ++t) {
                for (int j = 0; j < W; ++j)
                    dw[(size_t)c * W + j] += dz[t] * xe_at(x, state_in, b, t + j, c, T, C, W);
                dbias[c] += dz[t];
            }
            for (int t = 0; t < T; ++t) dx[((size_t)b * T + t) * C + c] = dxe[W - 1 + t];
            for (int i = 0; i < W - 1; ++i) dstate_in[((size_t)b * (W - 1) + i) * C + c] = dxe[i];
        }
    free(dz);
    free(dxe);
    return 0;
}
