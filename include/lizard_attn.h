/*
 * lizard_attn.h -- C ABI of the MI355X (gfx950) hybrid attention library.
 *
 * The layer is the hybrid attention of "Lizard: An Efficient Linearization
 * Framework for Large Language Models" as described on the gist.science
 * explainer pages (English page, section 2.A "Hybrid Attention Architecture"
 * and section 2.C "Hardware-Aware Algorithm"):
 *
 *   GLA branch     S_t = diag(exp g_t) S_{t-1} + k_t^T v_t,  o^gla_t = q_t S_t
 *                  (gate Gamma_t = diag(exp g_t), given in log space, one
 *                  value per key dimension; zero initial state)
 *   anchor window  o^swa_t = softmax over { scale*q_t.mk_m : m < M } and
 *                  { scale*q_t.k_s : t-W < s <= t } applied to [mv ; v]
 *                  (meta keys are sinks; meta values are zero when meta_v is
 *                  NULL, the pages' reading that meta tokens add no value)
 *   output         o_t = o^gla_t + mix * o^swa_t    (section 2.A, "Final Output")
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * - Every tensor pointer is a DEVICE pointer owned by the caller.  The
 *   library never allocates or frees device memory, never synchronises the
 *   stream and keeps no global mutable state: calls are re-entrant and
 *   thread-safe; calls that overlap on the same output buffers race.
 * - All tensors are dense row-major ("contiguous") in the shapes given:
 *     q, k, o, dq, dk, dO : [B,H,L,d_k]      v, dv : [B,H,L,d_v]
 *     g, dg               : [B,H,L,d_k] fp32 (log-gates, g <= 0)
 *     meta_k              : [H,M,d_k]        meta_v: [H,M,d_v] or NULL
 *     lse                 : [B,H,L] fp32     o_swa : [B,H,L,d_v]
 *     chunk_states        : [B,H,ceil(L/chunk),d_k,d_v]  (state entering each chunk)
 *     state, state_out    : [B,H,d_k,d_v] fp32
 *     ring_k, ring_v      : [B,H,W,d_k] / [B,H,W,d_v]    pos : [B] int32
 *   "dtype" tensors (q, k, v, o, meta_k, meta_v, dO, dq, dk, dv, o_swa,
 *   chunk_states, ring_k, ring_v) are fp32 or bf16 as lizard_attn_shape_t
 *   says; gates, lse, dg, dmeta_* and the decode state are always fp32.
 * - Every pointer must be 16-byte aligned.
 * - Validation runs on the host before any launch.  On any error nothing is
 *   launched and no output is written; the return value says why.  A launch
 *   failure returns LIZARD_EHIP.  Faults inside kernels surface, as usual
 *   for HIP, at the caller's next synchronisation.
 * - Supported: d_k = d_v in {64, 128}, bf16 or fp32.  lizard_attn_fwd and
 *   lizard_attn_bwd take chunk in {16, 32, 64, 128} (0 selects 64): chunk 64 in
 *   bf16, or in fp32 at d = 64, runs on the fast (matrix-core) kernels; every
 *   other chunk, and fp32 at d = 128, on the general path -- the same chunkwise
 *   algorithm (states passed and stored at the chunk boundaries in the operand
 *   dtype) with fp32 arithmetic on the vector units, exact for every gate and
 *   many times slower.  The continuation, the log-feature entry points, the
 *   Hedgehog map and the stage-1 loss take chunk 64 and, in fp32, d = 64 only;
 *   decode has no chunk and takes either dtype at d in {64, 128}.
 *   Forward/backward: any W >= 1 (W >= L sees the whole causal prefix);
 *   continued segments and decode keep the window in a ring: 1 <= W <= 8192.
 *   0 <= M <= 16; B, H >= 1; 0 <= L <= 2^30 (L = 0 writes only the zero state /
 *   zero meta gradients).  Anything else returns LIZARD_EUNSUPPORTED.
 * - Numerical domain: every finite log-gate g <= 0, per token and key
 *   dimension (English page §2.C: the gate handled in log space keeps gated
 *   attention exact in low precision).  Inside a chunk the gate is folded into
 *   q and k relative to the chunk start while every key dimension's chunk
 *   total stays at or above -64; a chunk with a stronger gate (the pages' own
 *   sigmoid gate, g = log sigmoid(z), sums to about -50 .. -200 per 64 tokens)
 *   is computed by 16-token blocks with the gate folded relative to each
 *   block's end, and a block that itself decays by more than that range is
 *   formed exactly pair by pair.  The state sweep decides per chunk on the
 *   device; no host scan, no synchronisation.
 */
#ifndef LIZARD_ATTN_H
#define LIZARD_ATTN_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  LIZARD_OK = 0,
  LIZARD_EINVAL = 1,        /* null pointer, negative size, meta_v/dmeta_v mismatch */
  LIZARD_EUNSUPPORTED = 2,  /* a size or dtype outside the supported set above */
  LIZARD_EALIGN = 3,        /* a pointer not 16-byte aligned */
  LIZARD_EWORKSPACE = 4,    /* workspace missing or smaller than required */
  LIZARD_EHIP = 5           /* a HIP launch or runtime call failed */
} lizard_status_t;

typedef enum { LIZARD_FP32 = 0, LIZARD_BF16 = 1 } lizard_dtype_t;

/* Gate granularity.  PER_DIM: one log-gate per key dimension, g and dg
 * [B,H,L,d_k] (decode g [B,H,d_k]).  SCALAR: one log-gate per head and token,
 * g and dg [B,H,L] (decode g [B,H]): Gamma_t = exp(g_t) I, the lightweight
 * gate the Chinese page's ablation section prefers over richer gate
 * structures; it cuts the gate traffic from 4*d_k to 4 bytes per head-token. */
typedef enum { LIZARD_GATE_PER_DIM = 0, LIZARD_GATE_SCALAR = 1 } lizard_gate_t;

typedef struct {
  int32_t B, H, L;          /* batch, heads, sequence length (L unused by decode) */
  int32_t d_k, d_v;         /* head dims; must be equal */
  int32_t W;                /* window length, counting the current token */
  int32_t M;                /* meta-memory tokens */
  int32_t chunk;            /* chunk length of the chunkwise form; 0 -> 64 */
  float scale;              /* softmax logit scale, normally 1/sqrt(d_k) */
  float mix;                /* alpha in o = o_gla + alpha * o_swa */
  int32_t dtype;            /* lizard_dtype_t */
  int32_t gate;             /* lizard_gate_t (0, the zero-initialised default, is per key dimension) */
} lizard_attn_shape_t;

enum { LIZARD_OP_FWD = 0, LIZARD_OP_BWD = 1, LIZARD_OP_DECODE = 2, LIZARD_OP_FWD_CONTINUE = 3,
       LIZARD_OP_DISTILL = 4, LIZARD_OP_FEATURE_BWD = 5,
       LIZARD_OP_BWD_RECOMPUTE = 6 /* the backward without its saved forward tensors */ };

/* Bytes of device workspace that `op` needs for shape `s` (0 when none, or
 * when `s` is invalid).  Pass at least this many bytes to the call. */
size_t lizard_attn_workspace_bytes(const lizard_attn_shape_t* s, int op);

/* Forward pass (training or prefill): GLA branch in the chunkwise form with
 * log-space gate handling (English page §2.C: the cumulative gate is folded
 * into q and k so the core is a plain matrix product) plus the anchor window
 * (English page §2.A).
 *   o                 [B,H,L,d_v] output (written)
 *   lse          opt  [B,H,L] fp32, log-sum-exp of each window softmax row
 *   o_swa        opt  [B,H,L,d_v] window branch before mixing
 *   chunk_states opt  [B,H,ceil(L/chunk),d_k,d_v] dtype: the state entering every
 *                     chunk (needed by lizard_attn_bwd with the same chunk)
 *   state_out    opt  [B,H,d_k,d_v] fp32 state after the last token (decode hand-off)
 *   workspace         caller-owned device memory, clobbered: when chunk_states
 *                     is NULL at least lizard_attn_workspace_bytes(s, LIZARD_OP_FWD)
 *                     bytes (the chunk states go there); when chunk_states is
 *                     given, that figure less B*H*ceil(L/chunk)*d_k*d_v*esz
 *                     bytes (esz = 2 for bf16, 4 for fp32): the per-chunk
 *                     strong-gate masks and dispatch list (about 24 bytes per
 *                     (b, h, chunk)) and, when B*H is small enough for the state
 *                     sweep to run in sequence segments, its segment buffers
 *                     (general path: the gates' 16-token block sums, B*H*L*d*4
 *                     + B*H*ceil(L/16)*d*4 bytes); may be NULL only for L = 0
 * NULL optional outputs are not written.  Launches on `stream`: the state
 * sweep over chunks (when B*H*(d/64)^2 < 512 and L spans at least 32
 * chunks, in segments of the sequence: a reduce pass per segment, a scan
 * over segments, then the sweep of every segment from its entering state),
 * then one workgroup per (batch, head, chunk), then a persistent launch that
 * computes the chunks the sweep flagged as strong-gated (it ends at once when
 * there are none). */
lizard_status_t lizard_attn_fwd(const lizard_attn_shape_t* s,
                                const void* q, const void* k, const void* v, const float* g,
                                const void* meta_k, const void* meta_v,
                                void* o, float* lse, void* o_swa, void* chunk_states,
                                float* state_out,
                                void* workspace, size_t workspace_bytes, hipStream_t stream);

/* Backward pass: exact gradients of sum(dO * o) (the pages give no backward;
 * the formulas are the derivative of the forward above).
 *   lse, o_swa, chunk_states   optional: as written by lizard_attn_fwd on the
 *                              same inputs; when any of them is NULL, the forward
 *                              kernels recompute all three into the workspace
 *                              first (o is not written), which trades the memory
 *                              of keeping them between the passes (about
 *                              B*H*L*(4 + 2*d) + B*H*ceil(L/chunk)*d*d*2 bytes in
 *                              bf16) for a forward's time
 *   dq, dk, dv                 written (dtype)
 *   dg                         written, fp32 [B,H,L,d_k]
 *   dmeta_k                    written, fp32 [H,M,d_k] (summed over batch)
 *   dmeta_v                    fp32 [H,M,d_v]; must be NULL iff meta_v is NULL
 *   workspace                  lizard_attn_workspace_bytes(s, LIZARD_OP_BWD) bytes,
 *                              or (LIZARD_OP_BWD_RECOMPUTE) bytes when any saved
 *                              tensor is NULL; caller-owned device memory,
 *                              clobbered by the call
 *   stage_events          opt  profiling hook: NULL, or LIZARD_BWD_STAGES + 1
 *                              caller-created events that are recorded on
 *                              `stream` before the first, between consecutive
 *                              and after the last of the backward's kernels
 *                              (state-gradient sweep with the window row
 *                              dots, preceded by the recomputed forward when a
 *                              saved tensor is NULL; chunk gradients; meta
 *                              reduction; a stage
 *                              with nothing to do still gets its event).  For
 *                              L = 0, and on the general path, they are not
 *                              recorded. */
#define LIZARD_BWD_STAGES 3
lizard_status_t lizard_attn_bwd(const lizard_attn_shape_t* s,
                                const void* q, const void* k, const void* v, const float* g,
                                const void* meta_k, const void* meta_v, const void* dO,
                                const float* lse, const void* o_swa, const void* chunk_states,
                                void* dq, void* dk, void* dv, float* dg,
                                float* dmeta_k, float* dmeta_v,
                                void* workspace, size_t workspace_bytes, hipStream_t stream,
                                hipEvent_t* stage_events);

/* Forward and backward with a feature map on the GLA branch.  The branch keeps
 * its state from feature-mapped keys, S_t = Gamma_t S_{t-1} + phi(k_t) v_t^T,
 * read by phi(q_t) (English page §2.A, state update), and the pages absorb the
 * cumulative gate into the query and key projections in log space, which the
 * feature map's non-negativity allows (Chinese page §2.3; English page §2.C).
 * These calls take the logarithms of the features and form
 *   q~ = exp(lq + b),  k^ = exp(lk - b)   (b: chunk-local gate prefix)
 * directly, so no feature, however small, is rounded before the gate meets it.
 * The anchor window keeps the raw q and k; v is shared.
 *   lq, lk   [B,H,L,d_k] fp32: log phi(q), log phi(k) (e.g. from a Hedgehog map)
 *   dlq, dlk [B,H,L,d_k] fp32, written: gradients of lq and lk
 *   dq, dk   written: the window branch's gradients of q and k only
 * Everything else is as for lizard_attn_fwd / lizard_attn_bwd; per-dimension
 * gates only (LIZARD_GATE_SCALAR returns LIZARD_EUNSUPPORTED); the chunked-prefill
 * and decode forms follow below. */
lizard_status_t lizard_attn_fwd_feat(const lizard_attn_shape_t* s,
                                     const void* q, const void* k, const void* v,
                                     const float* lq, const float* lk, const float* g,
                                     const void* meta_k, const void* meta_v,
                                     void* o, float* lse, void* o_swa, void* chunk_states,
                                     float* state_out,
                                     void* workspace, size_t workspace_bytes, hipStream_t stream);
lizard_status_t lizard_attn_bwd_feat(const lizard_attn_shape_t* s,
                                     const void* q, const void* k, const void* v,
                                     const float* lq, const float* lk, const float* g,
                                     const void* meta_k, const void* meta_v, const void* dO,
                                     const float* lse, const void* o_swa, const void* chunk_states,
                                     void* dq, void* dk, void* dv, float* dlq, float* dlk, float* dg,
                                     float* dmeta_k, float* dmeta_v,
                                     void* workspace, size_t workspace_bytes, hipStream_t stream,
                                     hipEvent_t* stage_events);

/* Chunked prefill and decode with log features: as lizard_attn_fwd_continue and
 * lizard_attn_decode_step, with the GLA state updated by exp(lk) and read by
 * exp(lq) (lq, lk [B,H,L,d_k] or, for decode, [B,H,d_k], fp32) and the window
 * on the raw q, k.  The carry (state, ring of raw keys and values, pos) is
 * the same as for the plain calls, so a log-feature prefill
 * (lizard_attn_fwd_feat with state_out) hands over to these. */
lizard_status_t lizard_attn_fwd_continue_feat(const lizard_attn_shape_t* s,
                                              const void* q, const void* k, const void* v,
                                              const float* lq, const float* lk, const float* g,
                                              const void* meta_k, const void* meta_v,
                                              float* state, void* ring_k, void* ring_v, int32_t* pos,
                                              void* o, void* workspace, size_t workspace_bytes,
                                              hipStream_t stream);
lizard_status_t lizard_attn_decode_step_feat(const lizard_attn_shape_t* s,
                                             const void* q, const void* k, const void* v,
                                             const float* lq, const float* lk, const float* g,
                                             const void* meta_k, const void* meta_v,
                                             float* state, void* ring_k, void* ring_v, int32_t* pos,
                                             void* o, void* workspace, size_t workspace_bytes,
                                             hipStream_t stream);

/* Hedgehog feature map in log space, the input of the *_feat calls above.  The
 * pages name the GLA branch's feature map a Hedgehog map and rely on its
 * non-negativity (Chinese page §2.3); they do not print it.  This is its
 * two-sided softmax form, per head h:
 *
 *   log phi(x) = [ z - lse(z),  -z - lse(-z) ],  z = x W_h  (d/2 features each half)
 *
 *   s      validated as for lizard_attn_fwd; uses B, H, L, d_k and dtype
 *   x      [B,H,L,d_k] dtype (q or k of the layer)
 *   w      [H,d_k,d_k/2] dtype, row-major per head
 *   lphi   written, [B,H,L,d_k] fp32
 * Backward, from dl = dL/dlog phi ([B,H,L,d_k] fp32):
 *   dx     written, [B,H,L,d_k] dtype (the feature map's part only)
 *   dw     written, [H,d_k,d_k/2] fp32, summed over batch and tokens in a fixed order
 *   workspace  lizard_attn_workspace_bytes(s, LIZARD_OP_FEATURE_BWD) bytes of
 *          caller-owned device memory (per-group partial sums of dw)
 * L = 0: the forward writes nothing, the backward writes dw = 0. */
lizard_status_t lizard_hedgehog_fwd(const lizard_attn_shape_t* s, const void* x, const void* w, float* lphi,
                                    hipStream_t stream);
lizard_status_t lizard_hedgehog_bwd(const lizard_attn_shape_t* s, const void* x, const void* w, const float* dl,
                                    void* dx, float* dw, void* workspace, size_t workspace_bytes,
                                    hipStream_t stream);

/* Chunked prefill: the forward of the next L tokens of every sequence, resuming
 * from the carry that earlier segments or decode steps left.  The state update
 * of the GLA branch (English page section 2.A, "Gated Linear Attention (GLA)
 * with Learnable Gating") is continued from the carried state instead of zero,
 * and the anchor window of
 * the segment's first tokens reaches back into the carried ring; the result is
 * the forward of the whole sequence restricted to the new tokens (French page
 * section 2.A: inference in O(1) memory through an incremental state; English
 * page section 4, "Efficiency": constant memory at any length).  A segment with
 * pos = 0 and a zero state is the plain prefill that also writes the hand-off.
 *   q, k [B,H,L,d_k], v [B,H,L,d_v] (dtype), g [B,H,L,d_k] fp32: the segment
 *   state   in/out [B,H,d_k,d_v] fp32: state after the pos[b] earlier tokens;
 *           on return the state after the segment
 *   ring_k, ring_v in/out [B,H,W,d] (dtype): keys / values of the last
 *           min(pos[b], W) earlier tokens, token t in slot t mod W (the decode
 *           layout); on return the segment's last tokens are stored likewise
 *   pos     in/out, device int32 [B]: tokens before the segment, per sequence
 *           (sequences of one batch may differ); pos[b] + L < 2^31; incremented by L
 *   o       [B,H,L,d_v] written
 *   workspace  lizard_attn_workspace_bytes(s, LIZARD_OP_FWD_CONTINUE) bytes of
 *           caller-owned device memory (clobbered): the chunk states
 * Same size limits as lizard_attn_fwd.  L = 0 launches nothing.  Four launches
 * on `stream`: state sweep, output kernel, ring update, pos update. */
lizard_status_t lizard_attn_fwd_continue(const lizard_attn_shape_t* s,
                                         const void* q, const void* k, const void* v, const float* g,
                                         const void* meta_k, const void* meta_v,
                                         float* state, void* ring_k, void* ring_v, int32_t* pos,
                                         void* o, void* workspace, size_t workspace_bytes,
                                         hipStream_t stream);

/* One constant-memory decode step for every sequence (English page §4,
 * "Efficiency": constant memory at any length; French page §2.A: O(1)
 * inference by updating an incremental hidden state).
 *   q, k [B,H,d_k], v [B,H,d_v] (dtype), g [B,H,d_k] fp32: the new token
 *   state  in/out: S <- diag(exp g) S + k^T v (fp32)
 *   ring_k, ring_v in/out: the new key/value is stored in slot pos[b] mod W
 *   pos    in/out, device int32 [B]: tokens already consumed, 0 <= pos[b] <
 *          2^31 - 1 (not checked: it lives on the device); incremented
 *   o      [B,H,d_v] written: q S + mix * softmax over M meta keys and the
 *          min(pos+1, W) filled ring slots.
 *   workspace  none is needed: lizard_attn_workspace_bytes(s, LIZARD_OP_DECODE)
 *          is 0 and the argument may be NULL (kept for the signature)
 * Two launches on `stream`: the step (d/64 workgroups per head, each owning
 * 64 value columns of the state, the output and the ring), then the advance
 * of pos.
 * Uses s->B, H, d_k, d_v, W, M, scale, mix, dtype; s->L and s->chunk are ignored. */
lizard_status_t lizard_attn_decode_step(const lizard_attn_shape_t* s,
                                        const void* q, const void* k, const void* v,
                                        const float* g, const void* meta_k, const void* meta_v,
                                        float* state, void* ring_k, void* ring_v, int32_t* pos,
                                        void* o,
                                        void* workspace, size_t workspace_bytes,
                                        hipStream_t stream);

/* lizard_attn_decode_step for callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid allocation): the same step with the same
 * arguments, minus the workspace.  The step needs no device memory beyond its arguments, so this
 * call allocates nothing and keeps nothing between calls; it validates like
 * lizard_attn_decode_step and launches the same kernels. */
lizard_status_t lizard_attn_decode_step_noalloc(const lizard_attn_shape_t* s,
                                                const void* q, const void* k, const void* v,
                                                const float* g, const void* meta_k, const void* meta_v,
                                                float* state, void* ring_k, void* ring_v, int32_t* pos,
                                                void* o, hipStream_t stream);

/* Stage-1 attention-approximation loss (English page §2, "Stage 1: Attention
 * Approximation"; French page "Étape 1"): the layer is trained to reproduce
 * the teacher's softmax attention output under a mean squared error.
 *
 *   o_T  = causal softmax attention: o_T[t] = sum_{s<=t} softmax_s(scale q_t.k_s) v_s
 *   loss = sum over every element of (o_S - o_T)^2 / N,  N = B*H*L*d_v
 *   dO   = 2 (o_S - o_T) / N
 *
 *   s        validated as for lizard_attn_fwd (bf16 d in {64, 128}, fp32 d = 64);
 *            B, H, L, d_k, d_v, scale and dtype define the call, W, M, chunk,
 *            mix and gate do not affect it
 *   q_t, k_t, v_t  the teacher's queries, keys and values, [B,H,L,d] dtype
 *            (they may alias the layer's q, k, v)
 *   o_s      the layer's output for the same tokens, [B,H,L,d_v] dtype
 *   dO       written, [B,H,L,d_v] dtype: the gradient to pass to lizard_attn_bwd
 *   loss     written, device fp32 scalar (0 when L = 0)
 *   workspace  lizard_attn_workspace_bytes(s, LIZARD_OP_DISTILL) bytes of
 *            caller-owned device memory (one partial sum per workgroup)
 * o_T is never written: the loss is applied in the attention kernel's
 * epilogue, and the partial sums are added in a fixed order (deterministic).
 * A stage-1 step is lizard_attn_fwd -> lizard_distill_mse -> lizard_attn_bwd. */
lizard_status_t lizard_distill_mse(const lizard_attn_shape_t* s, const void* q_t, const void* k_t,
                                   const void* v_t, const void* o_s, void* dO, float* loss, void* workspace,
                                   size_t workspace_bytes, hipStream_t stream);

/* Gate projection: the learnable gating module Gamma_t = sigmoid(W x_t)
 * (English page §2.A "Adaptive Memory Control"; Chinese page §2.1), produced
 * in log space for the layer (English page §2.C):
 *
 *   g = log sigmoid(x W^T) / tau
 *
 *   s        uses B, H, L, d_k, dtype and gate; the number of gate rows is
 *            Ng = H*d_k (LIZARD_GATE_PER_DIM) or Ng = H (LIZARD_GATE_SCALAR)
 *   d_model  width of x and W: a multiple of 32 in [32, 65536]
 *   tau      temperature, finite and > 0 (1 is the pages' gate; larger values
 *            slow the decay)
 *   x        [B,L,d_model] dtype, the layer input
 *   w        [Ng,d_model] dtype; row h*d_k + i gives gate dimension i of head h
 *            (row h for the scalar gate)
 *   g        written: fp32 in the layer's gate layout, [B,H,L,d_k] or [B,H,L]
 * One launch: an MFMA matrix product whose epilogue applies the log-sigmoid
 * and the temperature and writes the gate layout directly.  Sizes beyond the
 * supported set (d_k in {64, 128}, B*L*max(Ng, d_model) below 2^31 elements)
 * return LIZARD_EUNSUPPORTED; L = 0 writes nothing. */
lizard_status_t lizard_gate_proj_fwd(const lizard_attn_shape_t* s, int32_t d_model, float tau,
                                     const void* x, const void* w, float* g, hipStream_t stream);

/* Device workspace bytes that lizard_gate_proj_bwd needs (0 for an invalid shape). */
size_t lizard_gate_proj_workspace_bytes(const lizard_attn_shape_t* s, int32_t d_model);

/* Backward of the gate projection (the exact derivative; the pages give none):
 * with dz = dg * (1 - sigmoid(z)) / tau = -dg * expm1(tau*g) / tau,
 *   dx = dz W   written, [B,L,d_model] dtype (not accumulated)
 *   dw = dz^T x written, [Ng,d_model] fp32, summed over batch and tokens in a
 *               fixed order (deterministic)
 *   g           the forward's output for the same x and w; dg its gradient,
 *               both fp32 in the gate layout
 *   workspace   lizard_gate_proj_workspace_bytes(s, d_model) bytes of
 *               caller-owned device memory, clobbered (dz in the operand dtype,
 *               then partial sums of dw)
 * Launches: the dz pass, the dx product, the dw product (split over tokens
 * when Ng*d_model alone gives too few tiles) and, when split, the sum of the
 * splits.  L = 0 writes dw = 0. */
lizard_status_t lizard_gate_proj_bwd(const lizard_attn_shape_t* s, int32_t d_model, float tau,
                                     const void* x, const void* w, const float* g, const float* dg,
                                     void* dx, float* dw, void* workspace, size_t workspace_bytes,
                                     hipStream_t stream);

/* Static description of a status code. */
const char* lizard_attn_status_string(lizard_status_t st);

#ifdef __cplusplus
}
#endif

#endif /* LIZARD_ATTN_H */
