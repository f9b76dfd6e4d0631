// lz_api.cpp -- C ABI of the hybrid attention library: validation and launch.
//
// Host code only.  Every entry point validates its arguments completely
// before the first HIP call, so an invalid call launches nothing and writes
// nothing; kernels are then enqueued on the caller's stream without any
// synchronisation or allocation.
#include <math.h>
#include <stdint.h>
#include <string.h>

#include "../../include/lizard_attn.h"
#include "lz_kernels.hpp"

namespace {

constexpr int kChunk = 64;
constexpr int kMaxMeta = 16;
constexpr int kMaxDecodeWindow = 8192;
constexpr int32_t kMaxL = 1 << 30;

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Checks common to all ops.  `need_L` is false for decode.
lizard_status_t check_shape(const lizard_attn_shape_t* s, int op) {
  if (s == nullptr) return LIZARD_EINVAL;
  if (s->B < 1 || s->H < 1 || s->d_k < 1 || s->d_v < 1 || s->W < 1 || s->M < 0) return LIZARD_EINVAL;
  if (op != LIZARD_OP_DECODE && s->L < 0) return LIZARD_EINVAL;
  // token indices (and a chunk's end, t0 + 64) stay far inside int32 in every kernel
  if (op != LIZARD_OP_DECODE && s->L > kMaxL) return LIZARD_EUNSUPPORTED;
  if (!isfinite(s->scale) || !isfinite(s->mix)) return LIZARD_EINVAL;
  if (s->dtype != LIZARD_FP32 && s->dtype != LIZARD_BF16) return LIZARD_EUNSUPPORTED;
  if (s->gate != LIZARD_GATE_PER_DIM && s->gate != LIZARD_GATE_SCALAR) return LIZARD_EUNSUPPORTED;
  if (s->d_k != s->d_v) return LIZARD_EUNSUPPORTED;
  const int d = s->d_k;
  if (d != 64 && d != 128) return LIZARD_EUNSUPPORTED;
  if (s->M > kMaxMeta) return LIZARD_EUNSUPPORTED;
  // a continued segment and a decode step keep the window's keys in a ring of W slots
  if ((op == LIZARD_OP_DECODE || op == LIZARD_OP_FWD_CONTINUE) && s->W > kMaxDecodeWindow)
    return LIZARD_EUNSUPPORTED;
  if (op != LIZARD_OP_DECODE) {
    const int C = s->chunk == 0 ? kChunk : s->chunk;
    if (C != 16 && C != 32 && C != 64 && C != 128) return LIZARD_EUNSUPPORTED;
    // a continued segment runs on the fast kernels only: chunk 64, fp32 at d = 64
    if (op == LIZARD_OP_FWD_CONTINUE && (C != kChunk || (s->dtype == LIZARD_FP32 && d != 64)))
      return LIZARD_EUNSUPPORTED;
  }
  // every tensor of the call must be addressable with 64-bit offsets and
  // the grid must fit one launch
  const double elems = (double)s->B * s->H * (op == LIZARD_OP_DECODE ? s->W : (s->L > 0 ? s->L : 1)) * d;
  if (elems > 9.0e15) return LIZARD_EUNSUPPORTED;
  if ((double)s->B * s->H * (d / 16) > 2.0e9) return LIZARD_EUNSUPPORTED;
  if (op != LIZARD_OP_DECODE && (double)s->B * s->H * ((s->L + 15) / 16) > 2.0e9)
    return LIZARD_EUNSUPPORTED;   // one workgroup per (batch, head, chunk or 16-token block)
  return LIZARD_OK;
}

// The chunk size of a call (0 selects 64).
int chunk_of(const lizard_attn_shape_t* s) { return s->chunk == 0 ? kChunk : s->chunk; }

// Calls the fast kernels are not laid out for run on the general path: a chunk other than 64, or
// fp32 operands at d = 128 (forward and backward of the plain layer only).
bool general_path(const lizard_attn_shape_t* s) {
  return chunk_of(s) != kChunk || (s->dtype == LIZARD_FP32 && s->d_k != 64);
}

// Window length a whole sequence uses: keys in (t - W, t] that exist, so any W >= L sees the
// full causal prefix and is the same as W = L (this also keeps t - W + 1 far from overflow).
int32_t window_in(const lizard_attn_shape_t* s) { return s->W < s->L ? s->W : (s->L > 0 ? s->L : 1); }

lizard_status_t check_ptrs(std::initializer_list<const void*> required,
                           std::initializer_list<const void*> optional) {
  for (const void* p : required)
    if (p == nullptr) return LIZARD_EINVAL;
  for (const void* p : required)
    if (!aligned16(p)) return LIZARD_EALIGN;
  for (const void* p : optional)
    if (p != nullptr && !aligned16(p)) return LIZARD_EALIGN;
  return LIZARD_OK;
}

// Shape checks of the gate projection (B, H, L, d_k, dtype, gate and d_model only).
lizard_status_t check_gate_shape(const lizard_attn_shape_t* s, int32_t d_model, float tau) {
  if (s == nullptr) return LIZARD_EINVAL;
  if (s->B < 1 || s->H < 1 || s->L < 0 || s->d_k < 1 || d_model < 1) return LIZARD_EINVAL;
  if (!isfinite(tau) || !(tau > 0.f)) return LIZARD_EINVAL;
  if (s->dtype != LIZARD_FP32 && s->dtype != LIZARD_BF16) return LIZARD_EUNSUPPORTED;
  if (s->gate != LIZARD_GATE_PER_DIM && s->gate != LIZARD_GATE_SCALAR) return LIZARD_EUNSUPPORTED;
  if (s->d_k != 64 && s->d_k != 128) return LIZARD_EUNSUPPORTED;
  if (d_model % 32 != 0 || d_model > 65536) return LIZARD_EUNSUPPORTED;
  const double ng = s->gate == LIZARD_GATE_SCALAR ? (double)s->H : (double)s->H * s->d_k;
  const double tokens = (double)s->B * s->L;
  if (tokens * (ng > d_model ? ng : d_model) >= 2147483648.0) return LIZARD_EUNSUPPORTED;
  if (ng * d_model >= 2147483648.0) return LIZARD_EUNSUPPORTED;
  return LIZARD_OK;
}

lizard_status_t fwd_impl(const lizard_attn_shape_t* s,
                         const void* q, const void* k, const void* v, const float* lq, const float* lk,
                         const float* g, const void* meta_k, const void* meta_v,
                         void* o, float* lse, void* o_swa, void* chunk_states, float* state_out,
                         void* workspace, size_t workspace_bytes, hipStream_t stream) {
  lizard_status_t st = check_shape(s, LIZARD_OP_FWD);
  if (st != LIZARD_OK) return st;
  if (s->M > 0 && meta_k == nullptr) return LIZARD_EINVAL;
  // L = 0: the sequence tensors are empty (possibly NULL); only state_out is written (zero)
  if (s->L > 0)
    st = check_ptrs({q, k, v, g, o}, {meta_k, meta_v, lse, o_swa, chunk_states, state_out, workspace, lq, lk});
  else
    st = check_ptrs({}, {q, k, v, g, o, meta_k, meta_v, lse, o_swa, chunk_states, state_out, workspace, lq, lk});
  if (st != LIZARD_OK) return st;
  const bool gen = general_path(s);
  if (gen && lq != nullptr) return LIZARD_EUNSUPPORTED;   // log features: chunk 64, fast kernels only
  // the workspace holds the sweep's segment buffers (general path: the gates' block sums), and the
  // chunk states unless chunk_states is given
  const size_t need = s->L == 0 ? 0
                      : gen ? lz::fwd_general_workspace_bytes(s->B, s->H, s->L, s->d_k, chunk_of(s), s->dtype,
                                                              chunk_states != nullptr)
                      : chunk_states != nullptr ? lz::fwd_aux_bytes(s->B, s->H, s->L, s->d_k)
                                                : lz::fwd_workspace_bytes(s->B, s->H, s->L, s->d_k, s->dtype);
  if (need > 0 && (workspace == nullptr || workspace_bytes < need)) return LIZARD_EWORKSPACE;
  if (s->L == 0 && state_out == nullptr) return LIZARD_OK;
  lz::FwdArgs a{q, k, v, g, meta_k, s->M > 0 ? meta_v : nullptr, o, lse, o_swa, chunk_states, state_out,
                workspace, nullptr, nullptr, nullptr, nullptr, s->B, s->H, s->L, window_in(s), s->M, s->scale, s->mix,
                s->gate, s->L > 0 ? lq : nullptr, s->L > 0 ? lk : nullptr};
  const hipError_t e = gen ? lz::launch_fwd_general(a, s->dtype, s->d_k, chunk_of(s), stream)
                           : lz::launch_fwd(a, s->dtype, s->d_k, stream);
  return e == hipSuccess ? LIZARD_OK : LIZARD_EHIP;
}

lizard_status_t bwd_impl(const lizard_attn_shape_t* s,
                         const void* q, const void* k, const void* v, const float* lq, const float* lk,
                         const float* g, const void* meta_k, const void* meta_v, const void* dO,
                         const float* lse, const void* o_swa, const void* chunk_states,
                         void* dq, void* dk, void* dv, float* dlq, float* dlk, float* dg,
                         float* dmeta_k, float* dmeta_v,
                         void* workspace, size_t workspace_bytes, hipStream_t stream,
                         hipEvent_t* stage_events) {
  lizard_status_t st = check_shape(s, LIZARD_OP_BWD);
  if (st != LIZARD_OK) return st;
  if ((meta_v == nullptr) != (dmeta_v == nullptr)) return LIZARD_EINVAL;
  if (s->M > 0 && (meta_k == nullptr || dmeta_k == nullptr)) return LIZARD_EINVAL;
  if (s->L > 0)
    st = check_ptrs({q, k, v, g, dO, dq, dk, dv, dg},
                    {lse, o_swa, chunk_states, meta_k, meta_v, dmeta_k, dmeta_v, workspace, lq, lk, dlq, dlk});
  else   // L = 0: only the meta gradients (zero) are written
    st = check_ptrs({}, {q, k, v, g, dO, lse, o_swa, chunk_states, dq, dk, dv, dg,
                         meta_k, meta_v, dmeta_k, dmeta_v, workspace, lq, lk, dlq, dlk});
  if (st != LIZARD_OK) return st;
  const bool gen = general_path(s);
  if (gen && lq != nullptr) return LIZARD_EUNSUPPORTED;   // log features: chunk 64, fast kernels only
  // without the saved forward tensors the workspace also holds their recomputation
  const bool recompute = s->L > 0 && (lse == nullptr || o_swa == nullptr || chunk_states == nullptr);
  const size_t need =
      gen ? lz::bwd_general_workspace_bytes(s->B, s->H, s->L, s->M, s->d_k, chunk_of(s), s->dtype, recompute)
      : recompute ? lz::bwd_recompute_workspace_bytes(s->B, s->H, s->L, s->M, s->d_k, s->dtype)
                  : lz::bwd_workspace_bytes(s->B, s->H, s->L, s->M, s->d_k, s->dtype);
  if (need > 0 && (workspace == nullptr || workspace_bytes < need)) return LIZARD_EWORKSPACE;
  lz::BwdArgs a{};
  a.q = q; a.k = k; a.v = v; a.g = g;
  a.meta_k = meta_k; a.meta_v = s->M > 0 ? meta_v : nullptr; a.dO = dO;
  a.lse = lse; a.o_swa = o_swa; a.chunk_states = chunk_states;
  a.dq = dq; a.dk = dk; a.dv = dv; a.dg = dg;
  a.dmeta_k = s->M > 0 ? dmeta_k : nullptr;
  a.dmeta_v = s->M > 0 ? dmeta_v : nullptr;
  a.B = s->B; a.H = s->H; a.L = s->L; a.W = window_in(s); a.M = s->M;
  a.scale = s->scale; a.mix = s->mix; a.gate = s->gate;
  a.workspace = workspace;
  a.stage_events = stage_events;
  if (s->L > 0 && lq != nullptr) { a.lq = lq; a.lk = lk; a.dlq = dlq; a.dlk = dlk; }
  const hipError_t e = gen ? lz::launch_bwd_general(a, s->dtype, s->d_k, chunk_of(s), stream)
                           : lz::launch_bwd(a, s->dtype, s->d_k, stream);
  return e == hipSuccess ? LIZARD_OK : LIZARD_EHIP;
}

lizard_status_t continue_impl(const lizard_attn_shape_t* s, const void* q, const void* k, const void* v,
                              const float* lq, const float* lk, const float* g, const void* meta_k,
                              const void* meta_v, float* state, void* ring_k, void* ring_v, int32_t* pos, void* o,
                              void* workspace, size_t workspace_bytes, hipStream_t stream) {
  lizard_status_t st = check_shape(s, LIZARD_OP_FWD_CONTINUE);
  if (st != LIZARD_OK) return st;
  if (s->M > 0 && meta_k == nullptr) return LIZARD_EINVAL;
  if (s->L > 0)
    st = check_ptrs({q, k, v, g, state, ring_k, ring_v, pos, o}, {meta_k, meta_v, workspace, lq, lk});
  else   // L = 0: nothing to do; the carry is left as it is
    st = check_ptrs({}, {q, k, v, g, state, ring_k, ring_v, pos, o, meta_k, meta_v, workspace, lq, lk});
  if (st != LIZARD_OK) return st;
  if (s->L == 0) return LIZARD_OK;
  if (workspace == nullptr || workspace_bytes < lz::fwd_workspace_bytes(s->B, s->H, s->L, s->d_k, s->dtype))
    return LIZARD_EWORKSPACE;
  lz::FwdArgs a{q, k, v, g, meta_k, s->M > 0 ? meta_v : nullptr, o, nullptr, nullptr, nullptr, state,
                workspace, state, pos, ring_k, ring_v, s->B, s->H, s->L, s->W, s->M, s->scale, s->mix, s->gate,
                lq, lk};
  return lz::launch_fwd_continue(a, s->dtype, s->d_k, stream) == hipSuccess ? LIZARD_OK : LIZARD_EHIP;
}


lizard_status_t decode_impl(const lizard_attn_shape_t* s, const void* q, const void* k, const void* v,
                            const float* lq, const float* lk, const float* g, const void* meta_k, const void* meta_v,
                            float* state, void* ring_k, void* ring_v, int32_t* pos, void* o, void* workspace,
                            size_t /*workspace_bytes*/, hipStream_t stream) {
  lizard_status_t st = check_shape(s, LIZARD_OP_DECODE);
  if (st != LIZARD_OK) return st;
  if (s->M > 0 && meta_k == nullptr) return LIZARD_EINVAL;
  // the step needs no workspace (lizard_attn_workspace_bytes gives 0): the argument may be NULL
  st = check_ptrs({q, k, v, g, state, ring_k, ring_v, pos, o}, {meta_k, meta_v, workspace, lq, lk});
  if (st != LIZARD_OK) return st;
  lz::DecodeArgs a{q, k, v, g, meta_k, s->M > 0 ? meta_v : nullptr, state, ring_k, ring_v, pos, o,
                   s->B, s->H, s->W, s->M, s->scale, s->mix, s->gate, lq, lk};
  return lz::launch_decode(a, s->dtype, s->d_k, stream) == hipSuccess ? LIZARD_OK : LIZARD_EHIP;
}

}  // namespace

extern "C" {

const char* lizard_attn_status_string(lizard_status_t st) {
  // a C caller may pass any int: read it as one (an out-of-range enum value is undefined in C++)
  static_assert(sizeof(lizard_status_t) == sizeof(int), "status codes travel as int");
  int code;
  memcpy(&code, &st, sizeof(code));
  switch (code) {
    case LIZARD_OK: return "ok";
    case LIZARD_EINVAL: return "invalid argument (null pointer, bad size or inconsistent optional pair)";
    case LIZARD_EUNSUPPORTED: return "unsupported size, dtype or parameter";
    case LIZARD_EALIGN: return "pointer not 16-byte aligned";
    case LIZARD_EWORKSPACE: return "workspace missing or too small";
    case LIZARD_EHIP: return "HIP launch or runtime error";
  }
  return "unknown status";
}

size_t lizard_attn_workspace_bytes(const lizard_attn_shape_t* s, int op) {
  if (op != LIZARD_OP_FWD && op != LIZARD_OP_BWD && op != LIZARD_OP_DECODE && op != LIZARD_OP_FWD_CONTINUE &&
      op != LIZARD_OP_DISTILL && op != LIZARD_OP_FEATURE_BWD && op != LIZARD_OP_BWD_RECOMPUTE)
    return 0;
  const bool seq_op = op == LIZARD_OP_DISTILL || op == LIZARD_OP_FEATURE_BWD || op == LIZARD_OP_BWD_RECOMPUTE;
  if (check_shape(s, seq_op ? LIZARD_OP_FWD : op) != LIZARD_OK) return 0;
  if (op == LIZARD_OP_DISTILL) return lz::distill_workspace_bytes(s->B, s->H, s->L);
  if (op == LIZARD_OP_FEATURE_BWD) return s->L > 0 ? lz::feature_workspace_bytes(s->B, s->H, s->L, s->d_k) : 0;
  if (general_path(s) && (op == LIZARD_OP_FWD || op == LIZARD_OP_BWD || op == LIZARD_OP_BWD_RECOMPUTE)) {
    if (op == LIZARD_OP_FWD)
      return lz::fwd_general_workspace_bytes(s->B, s->H, s->L, s->d_k, chunk_of(s), s->dtype, false);
    return lz::bwd_general_workspace_bytes(s->B, s->H, s->L, s->M, s->d_k, chunk_of(s), s->dtype,
                                           op == LIZARD_OP_BWD_RECOMPUTE);
  }
  if (op == LIZARD_OP_BWD) return lz::bwd_workspace_bytes(s->B, s->H, s->L, s->M, s->d_k, s->dtype);
  if (op == LIZARD_OP_BWD_RECOMPUTE)
    return lz::bwd_recompute_workspace_bytes(s->B, s->H, s->L, s->M, s->d_k, s->dtype);
  if (op == LIZARD_OP_FWD || op == LIZARD_OP_FWD_CONTINUE)
    return lz::fwd_workspace_bytes(s->B, s->H, s->L, s->d_k, s->dtype);
  return 0;   // the decode step keeps nothing between its launches but pos
}

lizard_status_t lizard_attn_fwd(const lizard_attn_shape_t* s,
                                const void* q, const void* k, const void* v, const float* g,
                                const void* meta_k, const void* meta_v,
                                void* o, float* lse, void* o_swa, void* chunk_states,
                                float* state_out,
                                void* workspace, size_t workspace_bytes, hipStream_t stream) {
  return fwd_impl(s, q, k, v, nullptr, nullptr, g, meta_k, meta_v, o, lse, o_swa, chunk_states, state_out,
                  workspace, workspace_bytes, stream);
}

lizard_status_t lizard_attn_fwd_feat(const lizard_attn_shape_t* s,
                                     const void* q, const void* k, const void* v,
                                     const float* lq, const float* lk, const float* g,
                                     const void* meta_k, const void* meta_v,
                                     void* o, float* lse, void* o_swa, void* chunk_states,
                                     float* state_out,
                                     void* workspace, size_t workspace_bytes, hipStream_t stream) {
  if (s != nullptr && s->gate != LIZARD_GATE_PER_DIM) return LIZARD_EUNSUPPORTED;
  if (s != nullptr && s->L > 0 && (lq == nullptr || lk == nullptr)) return LIZARD_EINVAL;
  return fwd_impl(s, q, k, v, lq, lk, g, meta_k, meta_v, o, lse, o_swa, chunk_states, state_out, workspace,
                  workspace_bytes, stream);
}

lizard_status_t lizard_attn_fwd_continue(const lizard_attn_shape_t* s,
                                         const void* q, const void* k, const void* v, const float* g,
                                         const void* meta_k, const void* meta_v,
                                         float* state, void* ring_k, void* ring_v, int32_t* pos,
                                         void* o, void* workspace, size_t workspace_bytes,
                                         hipStream_t stream) {
  return continue_impl(s, q, k, v, nullptr, nullptr, g, meta_k, meta_v, state, ring_k, ring_v, pos, o, workspace,
                       workspace_bytes, stream);
}

lizard_status_t lizard_attn_fwd_continue_feat(const lizard_attn_shape_t* s,
                                              const void* q, const void* k, const void* v,
                                              const float* lq, const float* lk, const float* g,
                                              const void* meta_k, const void* meta_v,
                                              float* state, void* ring_k, void* ring_v, int32_t* pos,
                                              void* o, void* workspace, size_t workspace_bytes,
                                              hipStream_t stream) {
  if (s != nullptr && s->gate != LIZARD_GATE_PER_DIM) return LIZARD_EUNSUPPORTED;
  if (s != nullptr && s->L > 0 && (lq == nullptr || lk == nullptr)) return LIZARD_EINVAL;
  return continue_impl(s, q, k, v, lq, lk, g, meta_k, meta_v, state, ring_k, ring_v, pos, o, workspace,
                       workspace_bytes, stream);
}

lizard_status_t lizard_attn_bwd(const lizard_attn_shape_t* s,
                                const void* q, const void* k, const void* v, const float* g,
                                const void* meta_k, const void* meta_v, const void* dO,
                                const float* lse, const void* o_swa, const void* chunk_states,
                                void* dq, void* dk, void* dv, float* dg,
                                float* dmeta_k, float* dmeta_v,
                                void* workspace, size_t workspace_bytes, hipStream_t stream,
                                hipEvent_t* stage_events) {
  return bwd_impl(s, q, k, v, nullptr, nullptr, g, meta_k, meta_v, dO, lse, o_swa, chunk_states, dq, dk, dv,
                  nullptr, nullptr, dg, dmeta_k, dmeta_v, workspace, workspace_bytes, stream, stage_events);
}

lizard_status_t lizard_attn_bwd_feat(const lizard_attn_shape_t* s,
                                     const void* q, const void* k, const void* v,
                                     const float* lq, const float* lk, const float* g,
                                     const void* meta_k, const void* meta_v, const void* dO,
                                     const float* lse, const void* o_swa, const void* chunk_states,
                                     void* dq, void* dk, void* dv, float* dlq, float* dlk, float* dg,
                                     float* dmeta_k, float* dmeta_v,
                                     void* workspace, size_t workspace_bytes, hipStream_t stream,
                                     hipEvent_t* stage_events) {
  if (s != nullptr && s->gate != LIZARD_GATE_PER_DIM) return LIZARD_EUNSUPPORTED;
  if (s != nullptr && s->L > 0 && (lq == nullptr || lk == nullptr || dlq == nullptr || dlk == nullptr))
    return LIZARD_EINVAL;
  return bwd_impl(s, q, k, v, lq, lk, g, meta_k, meta_v, dO, lse, o_swa, chunk_states, dq, dk, dv, dlq, dlk, dg,
                  dmeta_k, dmeta_v, workspace, workspace_bytes, stream, stage_events);
}

lizard_status_t lizard_attn_decode_step(const lizard_attn_shape_t* s,
                                        const void* q, const void* k, const void* v,
                                        const float* g, const void* meta_k, const void* meta_v,
                                        float* state, void* ring_k, void* ring_v, int32_t* pos,
                                        void* o, void* workspace, size_t workspace_bytes,
                                        hipStream_t stream) {
  return decode_impl(s, q, k, v, nullptr, nullptr, g, meta_k, meta_v, state, ring_k, ring_v, pos, o, workspace,
                     workspace_bytes, stream);
}

lizard_status_t lizard_attn_decode_step_noalloc(const lizard_attn_shape_t* s,
                                                const void* q, const void* k, const void* v,
                                                const float* g, const void* meta_k, const void* meta_v,
                                                float* state, void* ring_k, void* ring_v, int32_t* pos,
                                                void* o, hipStream_t stream) {
  // the step keeps nothing in device memory of its own: the plain step without a workspace
  return decode_impl(s, q, k, v, nullptr, nullptr, g, meta_k, meta_v, state, ring_k, ring_v, pos, o, nullptr, 0,
                     stream);
}

lizard_status_t lizard_attn_decode_step_feat(const lizard_attn_shape_t* s,
                                             const void* q, const void* k, const void* v,
                                             const float* lq, const float* lk, const float* g,
                                             const void* meta_k, const void* meta_v,
                                             float* state, void* ring_k, void* ring_v, int32_t* pos,
                                             void* o, void* workspace, size_t workspace_bytes,
                                             hipStream_t stream) {
  if (s != nullptr && s->gate != LIZARD_GATE_PER_DIM) return LIZARD_EUNSUPPORTED;
  if (lq == nullptr || lk == nullptr) return LIZARD_EINVAL;
  return decode_impl(s, q, k, v, lq, lk, g, meta_k, meta_v, state, ring_k, ring_v, pos, o, workspace,
                     workspace_bytes, stream);
}

lizard_status_t lizard_hedgehog_fwd(const lizard_attn_shape_t* s, const void* x, const void* w, float* lphi,
                                    hipStream_t stream) {
  lizard_status_t st = check_shape(s, LIZARD_OP_FWD);
  if (st != LIZARD_OK) return st;
  if (s->dtype == LIZARD_FP32 && s->d_k != 64) return LIZARD_EUNSUPPORTED;   // fp32 kernels: d = 64
  st = s->L > 0 ? check_ptrs({x, w, lphi}, {}) : check_ptrs({}, {x, w, lphi});
  if (st != LIZARD_OK) return st;
  if (s->L == 0) return LIZARD_OK;
  lz::FeatArgs a{x, w, lphi, nullptr, nullptr, nullptr, nullptr, nullptr, s->B, s->H, s->L, 0};
  return lz::launch_feature_fwd(a, s->dtype, s->d_k, stream) == hipSuccess ? LIZARD_OK : LIZARD_EHIP;
}

lizard_status_t lizard_hedgehog_bwd(const lizard_attn_shape_t* s, const void* x, const void* w, const float* dl,
                                    void* dx, float* dw, void* workspace, size_t workspace_bytes,
                                    hipStream_t stream) {
  lizard_status_t st = check_shape(s, LIZARD_OP_FWD);
  if (st != LIZARD_OK) return st;
  if (s->dtype == LIZARD_FP32 && s->d_k != 64) return LIZARD_EUNSUPPORTED;   // fp32 kernels: d = 64
  st = s->L > 0 ? check_ptrs({x, w, dl, dx, dw, workspace}, {}) : check_ptrs({w, dw}, {x, dl, dx, workspace});
  if (st != LIZARD_OK) return st;
  if (s->L > 0 && workspace_bytes < lz::feature_workspace_bytes(s->B, s->H, s->L, s->d_k)) return LIZARD_EWORKSPACE;
  lz::FeatArgs a{x, w, nullptr, dl, dx, dw, workspace, nullptr, s->B, s->H, s->L, 0};
  return lz::launch_feature_bwd(a, s->dtype, s->d_k, stream) == hipSuccess ? LIZARD_OK : LIZARD_EHIP;
}

lizard_status_t lizard_distill_mse(const lizard_attn_shape_t* s, const void* q_t, const void* k_t,
                                   const void* v_t, const void* o_s, void* dO, float* loss, void* workspace,
                                   size_t workspace_bytes, hipStream_t stream) {
  lizard_status_t st = check_shape(s, LIZARD_OP_FWD);
  if (st != LIZARD_OK) return st;
  if (s->dtype == LIZARD_FP32 && s->d_k != 64) return LIZARD_EUNSUPPORTED;   // fp32 kernels: d = 64
  st = s->L > 0 ? check_ptrs({q_t, k_t, v_t, o_s, dO, loss, workspace}, {})
                : check_ptrs({loss}, {q_t, k_t, v_t, o_s, dO, workspace});
  if (st != LIZARD_OK) return st;
  if (s->L > 0 && workspace_bytes < lz::distill_workspace_bytes(s->B, s->H, s->L)) return LIZARD_EWORKSPACE;
  const double n = (double)s->B * s->H * s->L * s->d_v;
  lz::DistillArgs a{q_t, k_t, v_t, o_s, dO, loss, reinterpret_cast<float*>(workspace), s->B, s->H, s->L, s->scale,
                    n > 0 ? (float)(1.0 / n) : 0.f};
  return lz::launch_distill(a, s->dtype, s->d_k, stream) == hipSuccess ? LIZARD_OK : LIZARD_EHIP;
}

lizard_status_t lizard_gate_proj_fwd(const lizard_attn_shape_t* s, int32_t d_model, float tau,
                                     const void* x, const void* w, float* g, hipStream_t stream) {
  lizard_status_t st = check_gate_shape(s, d_model, tau);
  if (st != LIZARD_OK) return st;
  st = s->L > 0 ? check_ptrs({x, w, g}, {}) : check_ptrs({w}, {x, g});
  if (st != LIZARD_OK) return st;
  if (s->L == 0) return LIZARD_OK;
  lz::GateArgs a{x, w, g, nullptr, nullptr, nullptr, nullptr, s->B, s->H, s->L, s->d_k,
                 s->gate == LIZARD_GATE_SCALAR ? 1 : 0, d_model, tau};
  return lz::launch_gate_fwd(a, s->dtype, stream) == hipSuccess ? LIZARD_OK : LIZARD_EHIP;
}

size_t lizard_gate_proj_workspace_bytes(const lizard_attn_shape_t* s, int32_t d_model) {
  if (check_gate_shape(s, d_model, 1.f) != LIZARD_OK || s->L == 0) return 0;
  return lz::gate_bwd_workspace_bytes(s->B, s->H, s->L, s->d_k, s->gate == LIZARD_GATE_SCALAR ? 1 : 0, d_model,
                                      s->dtype);
}

lizard_status_t lizard_gate_proj_bwd(const lizard_attn_shape_t* s, int32_t d_model, float tau,
                                     const void* x, const void* w, const float* g, const float* dg,
                                     void* dx, float* dw, void* workspace, size_t workspace_bytes,
                                     hipStream_t stream) {
  lizard_status_t st = check_gate_shape(s, d_model, tau);
  if (st != LIZARD_OK) return st;
  st = s->L > 0 ? check_ptrs({x, w, g, dg, dx, dw}, {workspace}) : check_ptrs({w, dw}, {x, g, dg, dx, workspace});
  if (st != LIZARD_OK) return st;
  const size_t need = lizard_gate_proj_workspace_bytes(s, d_model);
  if (need > 0 && (workspace == nullptr || workspace_bytes < need)) return LIZARD_EWORKSPACE;
  lz::GateArgs a{x, w, const_cast<float*>(g), dg, dx, dw, workspace, s->B, s->H, s->L, s->d_k,
                 s->gate == LIZARD_GATE_SCALAR ? 1 : 0, d_model, tau};
  return lz::launch_gate_bwd(a, s->dtype, stream) == hipSuccess ? LIZARD_OK : LIZARD_EHIP;
}

}  // extern "C"
