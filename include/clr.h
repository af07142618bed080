/*
 * clr.h -- C ABI of the chunked gated linear recurrence layer for AMD MI355X
 * (gfx950).  Hand-written HIP kernels; plain pointers and sizes only.
 *
 * The operations
 * --------------
 * A sequence chunk of T tokens is processed with an incoming boundary state
 * and produces the outgoing one, as in the chunk forward / backward of the
 * StateFlow paper ("StateFlow: Sequence Pipeline Parallelism for Long-Context
 * Modeling with Linear Recurrence", Sec. 3.1, "Forward Computation" and
 * "Backward Computation"):
 *     fwd:  (o, S_out)            = Fwd(q, k, v, g, beta; S_in)
 *     bwd:  (dq, dk, dv, dg, dbeta, dS_in)
 *                                 = Bwd(q, k, v, g, beta, S_in; dO, dS_out)
 * so that feeding S_out of chunk i as S_in of chunk i+1, and dS_in of chunk
 * i+1 as dS_out of chunk i, reproduces the unchunked sequence (the boundary
 * chains S_{i+1}^in = S_i^out and dS_i^out = dS_{i+1}^in of the same paper).
 *
 * The recurrence is the matrix-state family of that paper's Sec. 2.1 (Eq. 1)
 * with its Gated DeltaNet and Gated Linear Attention transitions, written with
 * a key-major state S in R^{dk x dv} per (batch, head):
 *     GDN:  S_t = alpha_t (I - beta_t k_t k_t^T) S_{t-1} + beta_t k_t v_t^T
 *     GLA:  S_t = Diag(alpha_t) S_{t-1} + k_t v_t^T      (alpha_t in R^dk)
 *     both: o_t = S_t^T q_t,   alpha_t = exp(g_t),  g = log alpha (<= 0).
 * No query scaling is applied.  The gradients are those of
 *     L = sum_t <dO_t, o_t> + <dS_out, S_out>_F
 * with respect to q, k, v, g, beta and S_in.
 *
 * Layouts (all tensors contiguous, row-major, device memory)
 * ----------------------------------------------------------
 *     q, k, dq, dk      [B, T, H, dk]      element type = shape.dtype
 *     v, o, dO, dv      [B, T, H, dv]      element type = shape.dtype
 *     g, dg             GDN, Mamba-2: [B, T, H]   GLA: [B, T, H, dk]   (shape.dtype)
 *     beta, dbeta       GDN: [B, T, H]     GLA: must be NULL     (shape.dtype)
 *     S_in, S_out, dS_out, dS_in   [B, H, dk, dv]  always float32
 * Supported head sizes: GDN (dk, dv) in {(32,32), (64,64), (128,128)};
 * GLA additionally (128, 256).  The float32 backward supports (32, 32) and
 * (64, 64).
 * Others, among them GDN and KDA at dk = dv = 256 (the block kernels' LDS
 * tiles and the scans' per-block operands would not fit a CU at that size),
 * return CLR_ENOTSUP.  Any T >= 0 (a ragged last 64-token block is
 * handled by treating the missing tokens as identity steps; with T == 0 the
 * per-token tensors are empty and may be NULL, and the state passes through:
 * S_out = S_in, dS_in = dS_out).
 *
 * Ownership and execution
 * -----------------------
 * The caller allocates every buffer, including the workspace `ws` of at least
 * clr_workspace_bytes() bytes (256-byte aligned).  The library allocates no
 * device memory (its one static device array, the scratch of gdn_fwd_noalloc,
 * is part of its code object) and is re-entrant; calls are enqueued asynchronously on
 * `stream` (a hipStream_t of the current device; NULL = the default stream).
 * Inputs are never modified; outputs are overwritten.  Calls that share a
 * workspace must be ordered on one stream.  The only state kept between calls
 * is the split setting below and, per device, one auxiliary stream with four
 * events that the split forward creates on first use (kept until exit); work
 * put on it is joined back into `stream` before the call's last operation, so
 * ordering on `stream` alone remains sufficient for the caller.
 * Nullable: S_in (zero state), dS_out (zero), S_out (not wanted), o (not
 * wanted; GDN/GLA fwd).
 *
 * Errors
 * ------
 * Every argument is validated on the host before anything is enqueued; on a
 * non-zero status nothing has been launched and no output was touched:
 *     CLR_EINVAL      null required pointer, bad sizes, misaligned pointer
 *                     (tensors need 16-byte alignment), or an output that
 *                     overlaps an input / another output
 *     CLR_ENOTSUP     unsupported dtype or head size
 *     CLR_EWORKSPACE  ws is NULL or smaller than clr_workspace_bytes()
 *     CLR_EHIP        a HIP launch error (reported after enqueueing)
 *     CLR_ESCRATCH    gdn_fwd_noalloc only: the call needs more workspace
 *                     than the library's static scratch holds
 *     CLR_ERANGE      clr_range_status only: the gates of the last GLA, KDA
 *                     or Mamba-2 call left the diagonal tiles' bound
 * No exception or abort crosses the ABI.  Loading the library needs no GPU.
 */
#ifndef CLR_H
#define CLR_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    CLR_OK = 0,
    CLR_EINVAL = 1,
    CLR_ENOTSUP = 2,
    CLR_EWORKSPACE = 3,
    CLR_EHIP = 4,
    CLR_ESCRATCH = 5,
    CLR_ERANGE = 6
} clr_status_t;

typedef enum { CLR_F32 = 0, CLR_BF16 = 1 } clr_dtype_t;

typedef enum {
    CLR_OP_GDN_FWD = 0,
    CLR_OP_GDN_BWD = 1,
    CLR_OP_GLA_FWD = 2,
    CLR_OP_GLA_BWD = 3,
    CLR_OP_M2_FWD = 4,
    CLR_OP_M2_BWD = 5,
    CLR_OP_KDA_FWD = 6,
    CLR_OP_KDA_BWD = 7
} clr_op_t;

/* Shape of a call.  `chunk` is the kernel-level block of the chunkwise form
 * (the "kernel-level chunks" of the StateFlow paper, Sec. 3.1), in tokens:
 * 0 or 64, the only block size the kernels are built for (any other value
 * returns CLR_ENOTSUP).  Being last, it is 0 when an initialiser omits it. */
typedef struct {
    int32_t B, T, H, dk, dv;
    int32_t dtype; /* clr_dtype_t */
    int32_t chunk; /* 0 or 64 */
} clr_shape_t;

/* Workspace bytes needed by `op` (clr_op_t) at `shape`; 0 on invalid input. */
size_t clr_workspace_bytes(const clr_shape_t* shape, int op);

/* Gated DeltaNet chunk forward (see the header comment for the definition). */
int gdn_fwd(const clr_shape_t* shape, const void* q, const void* k, const void* v,
            const void* g, const void* beta, const float* S_in, void* o, float* S_out,
            void* ws, size_t ws_bytes, void* stream);

/* Gated DeltaNet chunk backward.  Recomputes the forward from (q, k, v, g,
 * beta, S_in); dS_out may be NULL (zero).  All gradient outputs required. */
int gdn_bwd(const clr_shape_t* shape, const void* q, const void* k, const void* v,
            const void* g, const void* beta, const float* S_in, const void* dO,
            const float* dS_out, void* dq, void* dk, void* dv, void* dg, void* dbeta,
            float* dS_in, void* ws, size_t ws_bytes, void* stream);

/* Gated DeltaNet forward and backward with saved activations.  The backward
 * needs the state entering every 64-token block and the block's U (the
 * delta-rule values, U = T Diag(beta) (V - Diag(Gam) K S)).  gdn_bwd
 * recomputes them from S_in; the pair below keeps them instead, as the
 * StateFlow paper's chunk backward may (Sec. 3.1, "Backward Computation":
 * the chunk's intermediate activations are either kept from the forward or
 * recomputed from its boundary state).
 *   clr_saved_bytes(shape): bytes of one chunk call's saved activations, for
 *     the shapes gdn_bwd supports (0 otherwise, and 0 when T == 0): per
 *     64-token block dk x dv states and 64 x dv values, in shape.dtype.
 *   gdn_fwd_save: gdn_fwd (same results, bit for bit) that also writes them
 *     into `saved` (device memory of at least clr_saved_bytes, 256-byte
 *     aligned, owned by the caller; its layout is the library's).  Its
 *     workspace is CLR_OP_GDN_FWD's.
 *   gdn_bwd_saved: the operation of gdn_bwd, reading `saved`, as the
 *     gdn_fwd_save of the same chunk (same shape and inputs) left it, in
 *     place of recomputing the forward; S_in is not read (it may be NULL).
 *     Its results equal gdn_bwd's bit for bit where gdn_bwd's recompute
 *     runs one wave per state slice (float32, and d = 32) and to rounding
 *     otherwise (bf16 at d >= 64, where that recompute sums each block's
 *     products over two halves of the key dimension: the states it gets
 *     differ from the forward's in their last bits).  Its workspace is
 *     CLR_OP_GDN_BWD's.
 * Both return CLR_EWORKSPACE for a missing, small or misaligned `saved`, and
 * CLR_EINVAL when it overlaps another buffer (an output, for gdn_fwd_save). */
size_t clr_saved_bytes(const clr_shape_t* shape);
int gdn_fwd_save(const clr_shape_t* shape, const void* q, const void* k, const void* v,
                 const void* g, const void* beta, const float* S_in, void* o, float* S_out,
                 void* saved, size_t saved_bytes, void* ws, size_t ws_bytes, void* stream);
int gdn_bwd_saved(const clr_shape_t* shape, const void* q, const void* k, const void* v,
                  const void* g, const void* beta, const float* S_in, const void* dO,
                  const float* dS_out, const void* saved, size_t saved_bytes, void* dq, void* dk,
                  void* dv, void* dg, void* dbeta, float* dS_in, void* ws, size_t ws_bytes,
                  void* stream);

/* Allocation-free Gated DeltaNet forward, for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, harnesses
 * that forbid allocation).  Same operation, arguments, layouts and results as
 * gdn_fwd (bit for bit), without the workspace: the library keeps one static
 * device array of CLR_NOALLOC_SCRATCH_BYTES per GPU for it (taken when the
 * library's code is loaded on that GPU, held until the process ends) and
 * allocates nothing per call.  Calls whose workspace, clr_workspace_bytes(
 * shape, CLR_OP_GDN_FWD), exceeds CLR_NOALLOC_SCRATCH_BYTES return
 * CLR_ESCRATCH before launching anything (at dk = dv = 128, bf16, the limit
 * is about 570 64-token blocks x heads, e.g. 16 heads x 2240 tokens).  All
 * calls on one GPU share its array and each call leaves it dirty: calls on
 * one GPU must be ordered (one stream, or synchronised); calls that overlap
 * on one GPU race.  The split-and-overlap schedule (clr_set_fwd_split) is
 * never used here. */
#define CLR_NOALLOC_SCRATCH_BYTES (64u << 20)
int gdn_fwd_noalloc(const clr_shape_t* shape, const void* q, const void* k, const void* v,
                    const void* g, const void* beta, const float* S_in, void* o, float* S_out,
                    void* stream);

/* GLA chunk forward; `beta` must be NULL (no delta term, no write scale).
 * Exact within the decay bound that clr_range_status reports on. */
int gla_fwd(const clr_shape_t* shape, const void* q, const void* k, const void* v,
            const void* g, const void* beta, const float* S_in, void* o, float* S_out,
            void* ws, size_t ws_bytes, void* stream);

/* GLA chunk backward; `beta` and `dbeta` must be NULL. */
int gla_bwd(const clr_shape_t* shape, const void* q, const void* k, const void* v,
            const void* g, const void* beta, const float* S_in, const void* dO,
            const float* dS_out, void* dq, void* dk, void* dv, void* dg, void* dbeta,
            float* dS_in, void* ws, size_t ws_bytes, void* stream);

/* Mamba-2 member of the family (StateFlow paper, Sec. 2.1, Eq. 1: the
 * transition F_t is a scalar times the identity), key-major:
 *     S_t = alpha_t S_{t-1} + k_t v_t^T,   o_t = S_t^T q_t,   alpha_t = exp(g_t)
 * with one scalar gate per (token, head).  A Mamba-2 SSD layer maps onto it
 * as q = C, k = B, v = dt * x, g = dt * A (the D skip term and the
 * discretisation stay with the caller).  Same arguments and layouts as
 * gla_fwd / gla_bwd except g and dg, which are [B, T, H] (shape.dtype);
 * beta and dbeta must be NULL.  Head sizes as for GLA.  Runs on the GLA
 * kernels with the gate broadcast over the key channels; dg is the channel
 * sum of the per-channel gate gradient.  Workspace: CLR_OP_M2_FWD /
 * CLR_OP_M2_BWD.  Decay bound as for GLA (clr_range_status). */
int mamba2_fwd(const clr_shape_t* shape, const void* q, const void* k, const void* v,
               const void* g, const void* beta, const float* S_in, void* o, float* S_out,
               void* ws, size_t ws_bytes, void* stream);
int mamba2_bwd(const clr_shape_t* shape, const void* q, const void* k, const void* v,
               const void* g, const void* beta, const float* S_in, const void* dO,
               const float* dS_out, void* dq, void* dk, void* dv, void* dg, void* dbeta,
               float* dS_in, void* ws, size_t ws_bytes, void* stream);

/* GLA, Mamba-2 and KDA forward and backward with saved activations (StateFlow
 * paper, Sec. 3.1, "Backward Computation": a chunk's intermediate activations
 * kept from its forward instead of recomputed from its boundary state).  The
 * backward needs the state entering every 64-token block; gla_bwd and
 * mamba2_bwd recompute it from S_in, the pairs below keep it.
 *   clr_saved_bytes_op(shape, op): bytes of one chunk call's saved
 *     activations for the member that op names (CLR_OP_GDN_*, CLR_OP_GLA_*,
 *     CLR_OP_M2_*, CLR_OP_KDA_*; the forward and backward of a member give
 *     the same figure), for the shapes that member's backward supports; 0
 *     otherwise and when T == 0.  GLA and Mamba-2: per 64-token block one
 *     dk x dv state in shape.dtype.  KDA: the states and the delta-rule
 *     values U, the same size as clr_saved_bytes.  With the Gated DeltaNet
 *     ops it equals clr_saved_bytes.
 *   gla_fwd_save / mamba2_fwd_save: gla_fwd / mamba2_fwd (same results, bit
 *     for bit) that also write the states into `saved` (device memory of at
 *     least clr_saved_bytes_op, 256-byte aligned, owned by the caller; its
 *     layout is the library's).  Workspace: CLR_OP_GLA_FWD / CLR_OP_M2_FWD.
 *   gla_bwd_saved / mamba2_bwd_saved: the operation of gla_bwd / mamba2_bwd,
 *     reading `saved` as the forward of the same chunk (same shape and
 *     inputs, same member) left it, in place of the recompute; S_in is not
 *     read (it may be NULL).  The saved states are those the recompute
 *     forms, bit for bit, so the results equal gla_bwd's / mamba2_bwd's bit
 *     for bit.  Workspace: CLR_OP_GLA_BWD / CLR_OP_M2_BWD.
 *   kda_fwd_save / kda_bwd_saved: the same for the KDA member (states and
 *     U kept; the results equal kda_fwd's / kda_bwd's bit for bit).
 *     Workspace: CLR_OP_KDA_FWD / CLR_OP_KDA_BWD.
 * Errors as for the Gated DeltaNet pair: CLR_EWORKSPACE for a missing, small
 * or misaligned `saved`, CLR_EINVAL when it overlaps another buffer. */
size_t clr_saved_bytes_op(const clr_shape_t* shape, int op);
int gla_fwd_save(const clr_shape_t* shape, const void* q, const void* k, const void* v,
                 const void* g, const void* beta, const float* S_in, void* o, float* S_out,
                 void* saved, size_t saved_bytes, void* ws, size_t ws_bytes, void* stream);
int gla_bwd_saved(const clr_shape_t* shape, const void* q, const void* k, const void* v,
                  const void* g, const void* beta, const float* S_in, const void* dO,
                  const float* dS_out, const void* saved, size_t saved_bytes, void* dq, void* dk,
                  void* dv, void* dg, void* dbeta, float* dS_in, void* ws, size_t ws_bytes,
                  void* stream);
int mamba2_fwd_save(const clr_shape_t* shape, const void* q, const void* k, const void* v,
                    const void* g, const void* beta, const float* S_in, void* o, float* S_out,
                    void* saved, size_t saved_bytes, void* ws, size_t ws_bytes, void* stream);
int mamba2_bwd_saved(const clr_shape_t* shape, const void* q, const void* k, const void* v,
                     const void* g, const void* beta, const float* S_in, const void* dO,
                     const float* dS_out, const void* saved, size_t saved_bytes, void* dq, void* dk,
                     void* dv, void* dg, void* dbeta, float* dS_in, void* ws, size_t ws_bytes,
                     void* stream);
int kda_fwd_save(const clr_shape_t* shape, const void* q, const void* k, const void* v,
                 const void* g, const void* beta, const float* S_in, void* o, float* S_out,
                 void* saved, size_t saved_bytes, void* ws, size_t ws_bytes, void* stream);
int kda_bwd_saved(const clr_shape_t* shape, const void* q, const void* k, const void* v,
                  const void* g, const void* beta, const float* S_in, const void* dO,
                  const float* dS_out, const void* saved, size_t saved_bytes, void* dq, void* dk,
                  void* dv, void* dg, void* dbeta, float* dS_in, void* ws, size_t ws_bytes,
                  void* stream);

/* KDA member of the family (StateFlow paper, Sec. 2.1, Eq. 1: F_t
 * diagonal-plus-low-rank), key-major:
 *     S_t = (I - beta_t k_t k_t^T) Diag(alpha_t) S_{t-1} + beta_t k_t v_t^T,
 *     o_t = S_t^T q_t,   alpha_t = exp(g_t) in R^dk (per key channel).
 * Same arguments as gdn_fwd / gdn_bwd except g and dg, which are
 * [B, T, H, dk] as for GLA; beta and dbeta are required.  Head sizes as for
 * GDN (fp32: d <= 64; CLR_ENOTSUP otherwise).
 * Workspace: CLR_OP_KDA_FWD / CLR_OP_KDA_BWD.  The backward recomputes the
 * forward from S_in (as gdn_bwd does); dS_out may be NULL (zero).  The
 * per-block decays use 16-token sub-tiles with the same e^80 bound as the GLA
 * path (see clr_range_status). */
int kda_fwd(const clr_shape_t* shape, const void* q, const void* k, const void* v,
            const void* g, const void* beta, const float* S_in, void* o, float* S_out,
            void* ws, size_t ws_bytes, void* stream);
int kda_bwd(const clr_shape_t* shape, const void* q, const void* k, const void* v,
            const void* g, const void* beta, const float* S_in, const void* dO,
            const float* dS_out, void* dq, void* dk, void* dv, void* dg, void* dbeta,
            float* dS_in, void* ws, size_t ws_bytes, void* stream);

/* Range check of the per-channel and scalar-gate members (GLA, KDA, Mamba-2).
 * Their kernels apply the decay between two tokens of one 16-token diagonal
 * sub-tile as a factor on each operand, both taken relative to the sub-tile's
 * 8th token (StateFlow paper, Sec. 2.1, Eq. 1: the products of the gates
 * between two steps); each factor is clamped at e^80 so that it stays finite
 * in float32 and bfloat16.  The results are exact while, for every key
 * channel, the summed -g from a sub-tile's first token to its 8th, and from
 * its 8th to its last, stays within 80 (for example -g <= 10 on every token);
 * beyond it the affected within-sub-tile terms are too small, but every
 * output stays finite.  Every GLA, KDA and Mamba-2 forward and backward
 * records, per 64-token block, in its workspace whether that bound held (no
 * extra launch).  clr_range_status waits for `stream`, reads those records
 * from `ws` as the last such call of `op` at `shape` left them, and returns
 * CLR_OK if the bound held in every block and CLR_ERANGE if not.  Call it
 * after that call, on the same stream, before `ws` is used again.  For the
 * Gated DeltaNet ops it returns CLR_OK without reading `ws` (the scalar gate
 * enters through exact exponentials of non-positive arguments).  Errors:
 * CLR_EINVAL / CLR_ENOTSUP for a bad shape or op, CLR_EWORKSPACE for a NULL
 * or misaligned ws, CLR_EHIP if the copy fails. */
int clr_range_status(const clr_shape_t* shape, int op, const void* ws, void* stream);

/* Causal short convolution with a boundary state.
 * The StateFlow paper (Sec. 1 and Sec. 3.3) hands the boundary state of a
 * layer's local-convolution modules from one sequence chunk to the next,
 * next to the recurrent state.  Here that convolution is the depthwise causal
 * one of width W applied in front of such layers (the pages leave it
 * unspecified; this is the plainest reading):
 *     xe = [state_in ; x]                       (W - 1 carried rows first)
 *     z_t = bias_c + sum_{j<W} w[c][j] xe[t + j],   y_t = act(z_t)
 *     state_out = the last W - 1 rows of xe
 * act: 0 = identity, 1 = SiLU (z * sigmoid(z)).  Chaining state_out ->
 * state_in over sequence chunks reproduces the unchunked y, and chaining
 * dstate_in -> dstate_out backward reproduces the unchunked dx, bit for bit;
 * dw and dbias are sums over tokens (accumulate them over chunks with
 * `accumulate` = 1).
 * Layouts (contiguous, row-major, device memory):
 *     x, y, dy, dx                    [B, T, C]    element type = dtype
 *     state_in, state_out             [B, W-1, C]  element type = dtype
 *                                                  (copies of input rows)
 *     dstate_out, dstate_in           [B, W-1, C]  float32 (partial sums)
 *     w, dw [C, W] and bias, dbias [C]             float32
 * C must be a multiple of 8 and 1 <= W <= 4.  Nullable: bias (zero),
 * state_in (zero), state_out (not wanted), dstate_out (zero), dbias (not
 * wanted), dstate_in when W == 1.  All pointers 16-byte aligned.
 * The backward needs a workspace of clr_shortconv_workspace_bytes() bytes.
 * Errors as for the layer entry points (validated before any launch). */
typedef struct {
    int32_t B, T, C, W;
    int32_t dtype; /* clr_dtype_t of x, y, the states and their gradients */
    int32_t act;   /* 0 = identity, 1 = SiLU */
} clr_conv_shape_t;

size_t clr_shortconv_workspace_bytes(const clr_conv_shape_t* shape);
int shortconv_fwd(const clr_conv_shape_t* shape, const void* x, const float* w, const float* bias,
                  const void* state_in, void* y, void* state_out, void* stream);
/* dw and dbias are overwritten (accumulate = 0) or added to (accumulate = 1). */
int shortconv_bwd(const clr_conv_shape_t* shape, const void* x, const float* w, const float* bias,
                  const void* state_in, const void* dy, const float* dstate_out, void* dx, float* dw,
                  float* dbias, float* dstate_in, int accumulate, void* ws, size_t ws_bytes,
                  void* stream);

/* Split-and-overlap forward (StateFlow paper, Sec. 3.4.2, "Split and
 * Overlap", forward wavefront).  gdn_fwd with o != NULL and at least 16
 * 64-token blocks splits its blocks into two parts at `permille`/1000 of the
 * blocks (each part keeps at least 8) and runs
 *     Pre(1) -> (ST(1) || Pre(2)) -> (ST(2) || Out(1)) -> Out(2)
 * with the bracketed pairs on `stream` and the auxiliary stream.  The results
 * are bit-identical to the unsplit schedule.  permille = 0 disables the split
 * and is the default: on MI355X each wait between the two streams costs
 * 10-20 us, more than the overlap hides at the supported sizes (opt in to
 * measure it).  Process-global.  Returns CLR_EINVAL unless
 * 0 <= permille < 1000.  clr_get_fwd_split returns the current value. */
int clr_set_fwd_split(int permille);
int clr_get_fwd_split(void);

/* Value-tile width B_V of the Gated DeltaNet forward state scan (StateFlow
 * paper, Sec. 3.4.1: the ST kernel's grid is B x heads x dv / B_V, and B_V is
 * chosen by profiling).  16 (the default): one work-group per 16 value
 * columns of a head, one consumer wave.  32: one work-group per 32 columns,
 * two consumer waves sharing the stream of the block operands W and K^T
 * (half the work-groups, each slot 40 instead of 36 KB, three slots instead
 * of four).  The results are bit-identical.  Process-global; returns
 * CLR_EINVAL for any other value.  clr_get_scan_bv returns the current
 * value. */
int clr_set_scan_bv(int bv);
int clr_get_scan_bv(void);

/* Human-readable text of a status code (static storage). */
const char* clr_status_string(int status);

/* Library ABI version (major * 100 + minor). */
int clr_version(void);

/* Profiling aid.  While enabled, every kernel the library launches is
 * bracketed by a start/stop event pair (hipExtLaunchKernelGGL) on the stream
 * it runs on.  clr_timing_report waits for the recorded events, writes one
 * entry per kernel name (launch count and summed duration, in launch order of
 * first appearance) into out[0..max_entries), clears the record and returns
 * the number of entries (or -CLR_EHIP).  Process-global; meant for
 * single-threaded benchmarking, not for concurrent use. */
typedef struct {
    char name[48];
    int launches;
    double total_ms;
} clr_kernel_time_t;
int clr_timing_enable(int on);
int clr_timing_report(clr_kernel_time_t* out, int max_entries);

/* Self-check of the matrix-core fragment layout used by every kernel:
 * C[16][16] = A[16][32] * Bt[16][32]^T for device buffers of `dtype`
 * (A, Bt row-major; C float32).  For tests. */
int clr_probe_mma(int dtype, const void* A, const void* Bt, float* C, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* CLR_H */
