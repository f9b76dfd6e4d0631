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
  int B, H, L, W, M;
  float scale, mix;
};

struct BwdArgs {
  const void* q; const void* k; const void* v; const float* g;
  const void* meta_k; const void* meta_v; const void* dO;
  const float* lse; const void* o_swa; const void* chunk_states;
  void* dq; void* dk; void* dv; float* dg; float* dmeta_k; float* dmeta_v;
  void* workspace;      // bwd_workspace_bytes() bytes, carved up by launch_bwd
  float* ws_delta;      // set by launch_bwd: [B,H,L] fp32, D_t = mix * dO_t . o_swa_t
  float* ws_dmeta;      // set by launch_bwd: [B*NC, H, M, 2*d] fp32 meta partials per (b, chunk)
  hipEvent_t* stage_events;   // optional: 5 events recorded around the 4 kernels
  int B, H, L, W, M;
  float scale, mix;
};

struct DecodeArgs {
  const void* q; const void* k; const void* v; const float* g;
  const void* meta_k; const void* meta_v;
  float* state; void* ring_k; void* ring_v; int32_t* pos; void* o;
  int B, H, W, M;
  float scale, mix;
};

// Each returns hipSuccess or the launch error.  dtype: 0 fp32, 1 bf16.
hipError_t launch_fwd(const FwdArgs& a, int dtype, int D, hipStream_t st);
hipError_t launch_bwd(const BwdArgs& a, int dtype, int D, hipStream_t st);
hipError_t launch_decode(const DecodeArgs& a, int dtype, int D, hipStream_t st);

// Workspace bytes needed by launch_bwd.
size_t bwd_workspace_bytes(int B, int H, int L, int M, int D, int dtype);

}  // namespace lz
