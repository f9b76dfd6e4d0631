// lz_kernels.hpp -- internal launch interface between the C ABI layer and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace lz {

struct FwdArgs {
  const void* q; const void* k; const void* v; const float* g;
  const void* meta_k; const void* meta_v;
  void* o; float* lse; void* o_swa; void* chunk_states; float* state_out;
  void* workspace;      // chunk-state buffer (fwd_workspace_bytes) used when chunk_states is NULL
  // continuation from a carried state (all NULL for a forward from the start of the sequences):
  // state_in [B,H,d,d] fp32 enters the first chunk; pos [B] counts the tokens before the segment;
  // ring_k / ring_v [B,H,W,d] hold the keys / values of the last min(pos, W) of them in slots t mod W
  const float* state_in; int32_t* pos; void* ring_k; void* ring_v;
  int B, H, L, W, M;
  float scale, mix;
  int gate;             // 0: g [B,H,L,d] per key dimension; 1: g [B,H,L] one per head and token
  // optional fp32 log features [B,H,L,d] of phi(q), phi(k) for the GLA branch (both or neither;
  // per-dimension gates, no continuation); the window branch reads q and k
  const float* lq; const float* lk;
  // set by the launcher (strong-gate dispatch, see StrongDispatch)
  uint16_t* strong; int32_t* list; int32_t* list_count;
};

// Strong-gate dispatch.  The gate is folded into q and k relative to the chunk start only while
// every column's chunk total Gamma stays at or above -kStrongGate; a chunk with any column below
// takes the sub-block path instead.  The state sweep writes, per (b*h, chunk), D/16 masks of 16
// bits (bit e of mask m: column 16m + e has Gamma < -kStrongGate) and zeroes list_count; the
// chunk-parallel kernel of the fast path appends every chunk with a nonzero mask to `list`
// (index b*h*NC + c) and leaves it, and a second launch of the sub-block variant works through
// the list.  Workspace: dispatch_bytes().
constexpr float kStrongGate = 64.f;
size_t dispatch_bytes(int B, int H, int L, int D);
struct StrongDispatch {
  uint16_t* mask; int32_t* list; int32_t* count;
};
StrongDispatch dispatch_layout(void* base, int B, int H, int L, int D);

struct BwdArgs {
  const void* q; const void* k; const void* v; const float* g;
  const void* meta_k; const void* meta_v; const void* dO;
  const float* lse; const void* o_swa; const void* chunk_states;
  void* dq; void* dk; void* dv; float* dg; float* dmeta_k; float* dmeta_v;
  void* workspace;      // bwd_workspace_bytes() bytes, carved up by launch_bwd
  float* ws_delta;      // set by launch_bwd: [B,H,L] fp32, D_t = mix * dO_t . o_swa_t
  float* ws_dmeta;      // set by launch_bwd: [B*NC, H, M, 2*d] fp32 meta partials per (b, chunk)
  hipEvent_t* stage_events;   // optional: 4 events recorded around the 3 stages
  int B, H, L, W, M;
  float scale, mix;
  int gate;             // as in FwdArgs; dg has the shape of g
  // optional log features as in FwdArgs, with their gradients dlq, dlk [B,H,L,d] fp32 written;
  // dq, dk then hold the window branch's part only
  const float* lq; const float* lk; float* dlq; float* dlk;
  // set by the launcher (strong-gate dispatch)
  uint16_t* strong; int32_t* list; int32_t* list_count;
};

// One sequential sweep over chunks (lz_sweep.hip).  Forward: a_src = k,
// b_src = v, out = chunk states [B,H,NC,d,d] (state entering each chunk),
// state_out = final state (fp32, optional), state_in = state entering the
// first chunk (fp32, optional; may alias state_out).  Backward: a_src = q, b_src = dO,
// states = the forward's chunk states, out = dS' transposed [B,H,NC,d,d],
// bnd = boundary rowsums [B,H,NC,d/64,d].
//
// Sequence segments: with NS > 1 the chunks are cut into NS segments of SC chunks
// that sweep in parallel.  A reduce pass carries every segment but the one swept
// first (the last forward, the first backward) from zero and writes its final state
// (state gradient) to seg_fin [B*H][NS][d][d] and its gate total to seg_gtot
// [B*H][NS][d]; a scan over segments writes what enters each segment to seg_in
// [B*H][NS][d][d] (forward: state_in or zero first; backward: zero last); the sweep
// pass then starts segment s from seg_in[s].  NS = 1: one segment, the fields below
// it are unused.
struct SweepArgs {
  const void* a_src; const void* b_src; const float* g;
  const void* states; void* out; float* bnd; float* state_out; const float* state_in;
  int B, H, L;
  int NS, SC;
  float* seg_in; float* seg_fin; float* seg_gtot;
  int gate;             // as in FwdArgs
  int feat;             // a_src is fp32 log features (per-dimension gates only)
  // backward: with delta set, the row blocks of each head also form the window row dots
  // delta_t = mix * dO_t . o_swa_t [B,H,L] fp32 from the dO rows they stream (each block a
  // share of the token rows)
  const void* o_swa; float* delta; float mix;
  // strong-gate masks [B*H][NC][D/16] written by the sweep pass (NULL: none), and the
  // dispatch list counter it zeroes (NULL: none).  Backward: the state gradient is stored
  // decayed (dS' = e^Gamma dS) in the columns whose mask bit is clear and undecayed (dS) in
  // the columns whose bit is set, where e^Gamma may underflow.
  uint16_t* strong; int32_t* list_count;
};

struct DecodeArgs {
  const void* q; const void* k; const void* v; const float* g;
  const void* meta_k; const void* meta_v;
  float* state; void* ring_k; void* ring_v; int32_t* pos; void* o;
  int B, H, W, M;
  float scale, mix;
  int gate;             // 0: g [B,H,d]; 1: g [B,H]
  // optional fp32 log features [B,H,d] of phi(q), phi(k) for the state (both or neither)
  const float* lq; const float* lk;
};

// Gate projection (lz_gate.hip).  Forward: g (output) = log sigmoid(x W^T) / tau in the gate
// layout.  Backward: g is the forward's output (input), dg its gradient; writes dx and dw.
struct GateArgs {
  const void* x; const void* w;   // x [B*L][d_model], w [Ng][d_model]; Ng = H*dk, or H when sg
  float* g; const float* dg;
  void* dx; float* dw;
  void* workspace;                // backward: gate_bwd_workspace_bytes()
  int B, H, L, dk, sg, d_model;
  float tau;
};

// Stage-1 distillation loss (lz_distill.hip): teacher causal attention of (q, k, v), MSE against
// the student output o_s, dO = 2 (o_s - o_T) / N; partial: distill_workspace_bytes() bytes.
struct DistillArgs {
  const void* q; const void* k; const void* v; const void* o_s;
  void* dO; float* loss; float* partial;
  int B, H, L;
  float scale, inv_n;
};

// Hedgehog feature map in log space (lz_feature.hip).  Forward: lphi [B,H,L,d] fp32 from
// x [B,H,L,d] and w [H,d,d/2].  Backward: dx [B,H,L,d] (dtype) and dw [H,d,d/2] fp32 from dl.
struct FeatArgs {
  const void* x; const void* w;
  float* lphi; const float* dl;
  void* dx; float* dw;
  void* workspace;      // backward: feature_workspace_bytes() bytes
  float* dw_part;       // set by the launcher
  int B, H, L;
  int cpg;              // set by the launcher: (batch, chunk) slots per backward workgroup
};

// Each returns hipSuccess or the launch error.  dtype: 0 fp32, 1 bf16.
hipError_t launch_fwd(const FwdArgs& a, int dtype, int D, hipStream_t st);
hipError_t launch_bwd(const BwdArgs& a, int dtype, int D, hipStream_t st);
hipError_t launch_decode(const DecodeArgs& a, int dtype, int D, hipStream_t st);
// Segment forward resuming from (state_in, ring, pos): launch_fwd, then the ring and pos advance.
hipError_t launch_fwd_continue(const FwdArgs& a, int dtype, int D, hipStream_t st);
hipError_t launch_sweep(const SweepArgs& a, int dtype, int D, bool reverse, hipStream_t st);
hipError_t launch_distill(const DistillArgs& a, int dtype, int D, hipStream_t st);
hipError_t launch_feature_fwd(const FeatArgs& a, int dtype, int D, hipStream_t st);
hipError_t launch_feature_bwd(const FeatArgs& a, int dtype, int D, hipStream_t st);   // L = 0: dw = 0
hipError_t launch_gate_fwd(const GateArgs& a, int dtype, hipStream_t st);
hipError_t launch_gate_bwd(const GateArgs& a, int dtype, hipStream_t st);   // L = 0: dw = 0

// General path (lz_general.hip): the chunkwise forward / backward at any chunk C in {16, 32, 64, 128}
// for fp32 or bf16 operands at d in {64, 128}, fp32 arithmetic on the vector units.  Same arguments
// as launch_fwd / launch_bwd (no continuation, no log features); chunk_states are [B,H,ceil(L/C),d,d].
hipError_t launch_fwd_general(const FwdArgs& a, int dtype, int D, int C, hipStream_t st);
hipError_t launch_bwd_general(const BwdArgs& a, int dtype, int D, int C, hipStream_t st);
size_t fwd_general_workspace_bytes(int B, int H, int L, int D, int C, int dtype, bool states_given);
size_t bwd_general_workspace_bytes(int B, int H, int L, int M, int D, int C, int dtype, bool recompute);

// Segments of the forward sweep for this shape (sequence parallelism when B*H is small).
int sweep_segments(int B, int H, int L, int D);
// Workspace bytes of the forward: the segment buffers (first), the strong-gate dispatch
// (fwd_aux_bytes covers both), then the chunk states (used when no chunk-state output is given).
size_t fwd_segment_bytes(int B, int H, int L, int D);
size_t fwd_aux_bytes(int B, int H, int L, int D);
size_t fwd_workspace_bytes(int B, int H, int L, int D, int dtype);
// Workspace bytes needed by launch_gate_bwd: dz [B*L][Ng rounded up to 16 bytes] in the operand
// dtype, then the fp32 partial sums of dW when its contraction over tokens is split.
size_t gate_bwd_workspace_bytes(int B, int H, int L, int dk, int sg, int d_model, int dtype);
// Workspace bytes needed by launch_feature_bwd: per-group partial sums of dw.
size_t feature_workspace_bytes(int B, int H, int L, int D);
// Workspace bytes needed by launch_distill: one fp32 partial per workgroup.
size_t distill_workspace_bytes(int B, int H, int L);
// Workspace bytes needed by launch_bwd when lse, o_swa and chunk_states are given, and when
// any of them is NULL (the forward kernels then recompute all three into the workspace).
size_t bwd_workspace_bytes(int B, int H, int L, int M, int D, int dtype);
size_t bwd_recompute_workspace_bytes(int B, int H, int L, int M, int D, int dtype);

}  // namespace lz
