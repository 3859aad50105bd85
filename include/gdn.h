/*
 * gdn.h - C ABI of the MI355X (gfx950) gated delta rule library, libgdn.so.
 *
 * What is computed. Per batch b and head h the library carries an fp32 state
 * h in R^{dk x dv} through the gated delta rule
 *
 *     alpha_t = exp(g_t * A),  A = -exp(A_log[h])
 *     h_t     = alpha_t (h_{t-1} - beta_t k_t (k_t^T h_{t-1})) + beta_t k_t v_t^T
 *     o_t     = h_t^T q_t
 *
 * The recurrence is the one of "GDN & MLA Mechanism Deep-Dive" (Intuition and
 * Math derivation, Step 4: per-head decay alpha_t = exp(g_t A) in (0,1), A kept
 * in log space as A_log, read o_t after the write) and of "HyMo-434M
 * documentation portal" (FIG. A0 probe and 01 GDN RECURRENCE: the delta rule
 * with gate beta_t), whose erase term is read with the key k_t. With
 * GDN_FLAG_ADDITIVE the erase term is off and the write/read pair of Step 4
 * remains: h_t = alpha_t h_{t-1} + beta_t k_t v_t^T. The forward runs the
 * chunked algorithm of Step 5 (chunk of 64 tokens solved in closed form with
 * 64 x 64 matrices, state carried serially between chunks); results equal the
 * serial definition above up to floating-point rounding.
 *
 * Layouts (all contiguous, row-major, no padding in memory):
 *   q, k, dq, dk        [B, T, H, dk]   dtype of the call (fp32 or bf16)
 *   v, o, do, dv        [B, T, H, dv]   dtype of the call
 *   g, beta, dg, dbeta  [B, T, H]       fp32; g and beta are the values the
 *                                       recurrence uses (post-sigmoid gate,
 *                                       no sigmoid is applied here)
 *   A_log, dA_log       [H]             fp32
 *   h0, hT, dhT, dh0    [B, H, dk, dv]  fp32 (row i = key index)
 *   decode (gdn_step):  q,k [N,H,dk], v,o [N,H,dv], g,beta [N,H],
 *                       states [N,H,dk,dv]; gdn_step_tokens: [N,S,H,*]
 *   D, dD               [H]             fp32 (skip term, optional)
 * bf16 outputs are rounded to nearest even. The library applies no scaling
 * to q; k is used as given unless GDN_FLAG_L2NORM_K asks for its per-token
 * normalisation.
 *
 * Layer edges. Two steps that sit on either side of the recurrence in the
 * GDN layer are fused into the kernels when asked for: the per-token L2
 * normalisation of the keys (GDN_FLAG_L2NORM_K) and the per-head skip term
 * o_t += D[h] v_t (a non-NULL D argument; "HyMo-434M documentation portal",
 * Architecture: the recurrence carries A_log, dt_bias and D). Both default
 * to off, which gives the recurrence above unchanged.
 *
 * Ownership. The caller allocates every buffer, including the workspaces
 * sized by the *_workspace_size queries; the library never allocates, frees
 * or synchronises. All device pointers are HIP device memory; `stream` is a
 * hipStream_t (NULL = the default stream). Work is enqueued on that stream and
 * the call returns without waiting for it.
 *
 * Errors. Argument checks run before anything is enqueued; a failing call
 * writes nothing and returns GDN_EINVAL / GDN_EUNSUPPORTED / GDN_EWORKSPACE.
 * A failed launch returns GDN_EHIP. Faults inside kernels surface at the
 * caller's next synchronisation. gdn_last_error_detail() gives a text for the
 * last non-OK status of the calling thread. NaN/Inf inputs propagate.
 * Results are bitwise reproducible for a given build, shape and device.
 *
 * Supported sizes: T >= 0 (a last chunk shorter than 64 is handled on chip),
 * 1 <= dk, dv <= 128 for bf16 and <= 64 for fp32, chunk 0 or 64, base
 * pointers 16-byte aligned, B*H < 2^31, tensors below 2^31 elements.
 *
 * Empty sequences (T = 0) run no step: gdn_fwd sets hT = h0 (zeros when h0
 * is NULL); gdn_bwd sets dh0 = dhT (zeros when dhT is NULL), dA_log = 0,
 * dD = 0 when given and, when asked, hT = h0. Pointers to arrays with a factor T in their extent may
 * then be NULL, and no workspace or context is used.
 */
#ifndef GDN_H
#define GDN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    GDN_OK = 0,
    GDN_EINVAL = 1,       /* bad argument (size, null pointer, alignment, aliasing) */
    GDN_EUNSUPPORTED = 2, /* valid request the library does not implement */
    GDN_EWORKSPACE = 3,   /* workspace pointer NULL or smaller than required */
    GDN_EHIP = 4          /* a HIP runtime call or kernel launch failed */
} gdn_status_t;

typedef enum { GDN_F32 = 0, GDN_BF16 = 1 } gdn_dtype_t;

/* Erase term off: h_t = alpha_t h_{t-1} + beta_t k_t v_t^T ("GDN & MLA
 * Mechanism Deep-Dive", Step 4 write line, write key b_t = beta_t k_t). */
#define GDN_FLAG_ADDITIVE 1u

/* g and beta are given as logits: the library applies the logistic sigmoid
 * on load (g = sigmoid(dt_proj(x)) in "GDN & MLA Mechanism Deep-Dive", Step 4;
 * the write gate beta likewise), and gdn_bwd returns dg and dbeta with
 * respect to the logits. dA_log is unchanged (it is taken through the gate
 * values). Without the flag g and beta are the gate values themselves. */
#define GDN_FLAG_GATE_LOGITS 2u

/* Keys are L2-normalised per token where the kernels load them: the
 * recurrence runs on k_hat = k / sqrt(sum_j k_j^2 + 1e-6), the unit-length
 * erase/write key of "GDN & MLA Mechanism Deep-Dive", Step 3 and Step 4 (the
 * epsilon under the root keeps a zero key finite). gdn_bwd then returns dk
 * with respect to the raw keys, dk = (dk_hat - k_hat (k_hat . dk_hat)) /
 * sqrt(sum_j k_j^2 + 1e-6). The raw keys are what the caller passes and
 * keeps; nothing normalised is written back. */
#define GDN_FLAG_L2NORM_K 4u

typedef struct {
    int32_t B, T, H; /* batch, tokens, heads */
    int32_t dk, dv;  /* key and value head dimensions */
    int32_t dtype;   /* gdn_dtype_t of q, k, v, o, do, dq, dk, dv */
    int32_t chunk;   /* 0 or 64 */
    uint32_t flags;  /* GDN_FLAG_ADDITIVE | GDN_FLAG_GATE_LOGITS | GDN_FLAG_L2NORM_K, or 0 */
} gdn_shape_t;

/* Bytes of device workspace gdn_fwd / gdn_bwd need for this shape. Return 0
 * for an invalid shape; the call itself then reports the error. */
size_t gdn_fwd_workspace_size(const gdn_shape_t *s);
size_t gdn_bwd_workspace_size(const gdn_shape_t *s);

/* Bytes of the optional forward context: what gdn_fwd can save for gdn_bwd
 * so that the backward skips recomputing the forward. It holds, in the
 * call's dtype, the state at the start of every 64-token chunk and the
 * chunk's -Tm diag(beta e^gam) K, Tm diag(beta) V and Tm = (I + L)^{-1}
 * blocks. Its layout is private to the library. */
size_t gdn_fwd_context_size(const gdn_shape_t *s);

/* Forward pass over a whole sequence ("GDN & MLA Mechanism Deep-Dive",
 * Step 4 and Step 5).
 *   q, k, v, g, beta, A_log  inputs (layouts above)
 *   D             [H] skip weights (o_t += D[h] v_t) or NULL (no skip term)
 *   h0            initial state or NULL (zero state)
 *   o             output [B,T,H,dv], or NULL: a state-only pass (e.g. the
 *                 prefill of a decode state), which writes hT and/or ctx
 *                 and skips the outputs
 *   hT            final state or NULL (not written)
 *   ctx           NULL, or gdn_fwd_context_size() bytes (256-byte aligned)
 *                 that receive the forward context for gdn_bwd
 *   ws, ws_bytes  workspace of gdn_fwd_workspace_size() bytes, 256-byte
 *                 aligned; its contents are scratch */
gdn_status_t gdn_fwd(const gdn_shape_t *s, const void *q, const void *k, const void *v,
                     const float *g, const float *beta, const float *A_log, const float *D,
                     const float *h0, void *o, float *hT, void *ctx, void *ws, size_t ws_bytes,
                     void *stream);

/* Bytes of the static device scratch gdn_fwd_noalloc uses as its workspace
 * (64 MiB per GPU, held until the process ends). */
#define GDN_NOALLOC_SCRATCH_BYTES (64u << 20)

/* gdn_fwd without a workspace argument and without any device allocation,
 * for callers that cannot allocate (code under HIP graph capture, tight
 * serving loops, harnesses that forbid allocation). Same computation,
 * arguments and results as gdn_fwd (bit for bit), with every launch on
 * `stream`. The workspace is a static device array of
 * GDN_NOALLOC_SCRATCH_BYTES in the library, one per GPU, shared by every
 * call on that GPU: calls that overlap in time on one GPU race and must be
 * ordered by the caller (e.g. issued on one stream). Shapes whose
 * gdn_fwd_workspace_size() exceeds GDN_NOALLOC_SCRATCH_BYTES are rejected
 * with GDN_EWORKSPACE before anything is enqueued (at d = 56 in bf16 the
 * scratch holds about 290,000 token-heads, e.g. B*T = 18,000 at H = 16). */
gdn_status_t gdn_fwd_noalloc(const gdn_shape_t *s, const void *q, const void *k, const void *v,
                             const float *g, const float *beta, const float *A_log, const float *D,
                             const float *h0, void *o, float *hT, void *ctx, void *stream);

/* Backward pass: gradients of sum(do * o) + sum(dhT * hT) with respect to q,
 * k, v, g, beta, A_log, D and h0, by the reverse-chunk derivative of the
 * chunked forward. Inputs are those of the gdn_fwd call (same flags, same D);
 * do is the upstream gradient of o, dhT that of the final state (NULL = zero).
 *   ctx           NULL (the forward is recomputed in the workspace) or the
 *                 context gdn_fwd saved for the same inputs
 *   dq, dk, dv    [B,T,H,*] in the call's dtype
 *   dg, dbeta     [B,T,H] fp32
 *   dA_log        [H] fp32, overwritten (sum over the batch)
 *   dD            [H] fp32 or NULL: overwritten with the sum over batch,
 *                 tokens and value columns of do * v, the gradient of the
 *                 skip weights (also when D is NULL: the gradient at D = 0)
 *   dh0           [B,H,dk,dv] fp32 or NULL
 *   hT            NULL, or receives the recomputed final state; only allowed
 *                 when ctx is NULL
 *   ws, ws_bytes  workspace of gdn_bwd_workspace_size() bytes, 256-byte
 *                 aligned
 * Supported head dimensions: those of gdn_fwd (bf16 up to 128, fp32 up to
 * 64). The local gradients of heads wider than 64 (bf16) or 16 (fp32) run in
 * a kernel that keeps its intermediates in the workspace; the workspace size
 * query includes that scratch. */
gdn_status_t gdn_bwd(const gdn_shape_t *s, const void *q, const void *k, const void *v,
                     const float *g, const float *beta, const float *A_log, const float *D,
                     const float *h0, const void *ctx, const void *dout, const float *dhT,
                     void *dq, void *dk, void *dv, float *dg, float *dbeta, float *dA_log,
                     float *dD, float *dh0, float *hT, void *ws, size_t ws_bytes, void *stream);

/* One decode token for each of N independent sequences: one step of the
 * recurrence from a carried state (the O(1)-state read/write of "GDN & MLA
 * Mechanism Deep-Dive", Intuition). h_in may be NULL (zero state) and may
 * equal h_out (in-place update); no other aliasing is allowed. `dtype` is the
 * gdn_dtype_t of q, k, v and o; `flags` is any of GDN_FLAG_ADDITIVE,
 * GDN_FLAG_GATE_LOGITS and GDN_FLAG_L2NORM_K, or 0; D is the [H] skip
 * weights or NULL, as in gdn_fwd. */
gdn_status_t gdn_step(int32_t N, int32_t H, int32_t dk, int32_t dv, int32_t dtype, uint32_t flags,
                      const void *q, const void *k, const void *v, const float *g,
                      const float *beta, const float *A_log, const float *D, const float *h_in,
                      float *h_out, void *o, void *stream);

/* S consecutive decode tokens for each of N independent sequences from a
 * carried state: the recurrence applied token after token (the serial
 * definition of "GDN & MLA Mechanism Deep-Dive", Step 4), as when the draft
 * tokens of a multi-token prediction are verified ("HyMo-434M documentation
 * portal", 04 MTP SPECULATION: a depth-2 draft, three tokens accepted per
 * step). q, k are
 * [N,S,H,dk], v, o [N,S,H,dv], g, beta [N,S,H] (the forward's layouts with
 * B = N, T = S); the states are [N,H,dk,dv]. The state is read once and
 * written once per call (heads up to 64 wide keep it on chip between the
 * tokens). For draft verification, call out of place: h_in then stays the
 * state to roll back to, and if only the first j tokens are accepted, a call
 * over those j tokens from h_in gives the state to keep.
 * h_in may be NULL (zero state) or equal h_out. S = 0 carries the
 * state over unchanged (h_out = h_in, zeros when h_in is NULL; the token
 * arrays may be NULL); N = 0 does nothing. gdn_step is this call with S = 1
 * and the [N,H,*] layouts. */
gdn_status_t gdn_step_tokens(int32_t N, int32_t S, int32_t H, int32_t dk, int32_t dv, int32_t dtype,
                             uint32_t flags, const void *q, const void *k, const void *v,
                             const float *g, const float *beta, const float *A_log, const float *D,
                             const float *h_in, float *h_out, void *o, void *stream);

/* Timing aid for benchmarks (no effect on results). While `events` is
 * non-NULL, every kernel the library launches from this thread is bracketed
 * by hipEventRecord calls on the launch's stream: events[2i] before launch i
 * and events[2i+1] after it, for the first n/2 launches counted from this
 * call (later launches are not bracketed). `events` points to n hipEvent_t
 * handles owned by the caller; NULL switches the aid off. Returns the number
 * of launches bracketed since the previous call. */
int32_t gdn_time_launches(void *const *events, int32_t n);

/* Which kernel the i-th bracketed launch of the current (or, once switched
 * off, the last) bracketing period was: 0 forward prep, 1 forward serial
 * pass, 2 backward serial pass, 3 backward local gradients, 4 dA_log (or
 * dD) reduction, 5 decode step, 6 forward scan over chunk ranges, 7 backward
 * scan; -1 when i is out of range. A forward call may launch its two kernels
 * several times each, over consecutive chunk ranges (prep of the next range
 * runs on a second stream while the serial pass works on the current one),
 * and a serial pass run as a parallel scan launches twice (the ranges' maps,
 * then every range from its start). */
int32_t gdn_launch_kind(int32_t i);

const char *gdn_status_string(gdn_status_t st);
const char *gdn_last_error_detail(void);

#ifdef __cplusplus
}
#endif

#endif /* GDN_H */
