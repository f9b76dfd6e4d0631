// lz_decode.hip -- constant-memory decode step of the Lizard hybrid attention layer.
//
// Whole decode state (gist.science explainer of "Lizard: An Efficient
// Linearization Framework for Large Language Models": English page §4
// "Efficiency", constant memory at any length; French page §2.A, O(1)
// inference through an incrementally updated hidden state):
//   S     [B,H,d_k,d_v] fp32   GLA state
//   ring  [B,H,W,d]            last W keys / values, token n in slot n mod W
//   pos   [B] int32            tokens consumed so far
//
// Two launches per step:
//   decode_state_kernel   one workgroup per (b, h, 32 state rows): streams the
//                         fp32 state, S <- diag(exp g) S + k^T v, and writes the
//                         rows' partial q . S to the workspace;
//   decode_window_kernel  one workgroup per (b, h): softmax over the meta keys
//                         and the filled ring slots (the new token's slot taken
//                         from the inputs, never from the ring), values, sum of
//                         the partials, o = o_gla + mix * o_swa, the ring write
//                         and the advance of pos.  Every load it needs is issued
//                         up front (one 128-key block of the key and value rings).
// Splitting keeps the state stream (two thirds of the step's bytes) in small,
// register-light workgroups that fill the chip.
//
// pos is shared by the H heads of a sequence: every window workgroup reads it
// first; when done, it adds 1 << 24 to it, and the workgroup that brings that
// arrival count to H stores pos + 1 (clearing the count).  Between calls the
// top byte of pos is zero; pos must stay below 2^24 and H below 256.
#include "lz_common.hpp"
#include "lz_kernels.hpp"

namespace lz {
namespace {

constexpr int NTHR = 256;
constexpr int KB = 128;          // ring keys per register block

constexpr int RB = 32;           // state rows per workgroup of the state kernel

template <typename T, int D>
__global__ __launch_bounds__(NTHR) void decode_state_kernel(DecodeArgs a) {
  constexpr int F4R = D / 4;                  // float4 per state row
  constexpr int RPT = RB * F4R / NTHR;        // rows per thread
  constexpr int RS = NTHR / F4R;              // row stride between a thread's rows
  static_assert(NTHR % F4R == 0 && RPT * RS == RB, "state thread map");
  __shared__ float sred[NTHR / 64][D];

  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int bh = blockIdx.x / (D / RB), rb = blockIdx.x % (D / RB);
  const int c4 = tid % F4R, r0 = tid / F4R;
  const size_t vo = (size_t)bh * D;
  float* S = a.state + ((size_t)bh * D + rb * RB) * D;
  f32x4 st[RPT];
#pragma unroll
  for (int u = 0; u < RPT; ++u) st[u] = *reinterpret_cast<const f32x4*>(S + (size_t)(r0 + u * RS) * D + 4 * c4);
  const T* vg = reinterpret_cast<const T*>(a.v) + vo;
  f32x4 vv;
#pragma unroll
  for (int e = 0; e < 4; ++e) vv[e] = Tr<T>::to_f(vg[4 * c4 + e]);
  float qi[RPT], ki[RPT], ai[RPT];
#pragma unroll
  for (int u = 0; u < RPT; ++u) {
    const int i = rb * RB + r0 + u * RS;
    qi[u] = Tr<T>::to_f(reinterpret_cast<const T*>(a.q)[vo + i]);
    ki[u] = Tr<T>::to_f(reinterpret_cast<const T*>(a.k)[vo + i]);
    ai[u] = __expf(a.gate ? a.g[bh] : a.g[vo + i]);   // scalar gate: one per head
  }
  f32x4 part = f32x4{0, 0, 0, 0};
#pragma unroll
  for (int u = 0; u < RPT; ++u) {
    const f32x4 x = ai[u] * st[u] + ki[u] * vv;
    *reinterpret_cast<f32x4*>(S + (size_t)(r0 + u * RS) * D + 4 * c4) = x;
    part += qi[u] * x;
  }
  // threads sharing c4 differ in the lane bits above log2(F4R), then across waves
#pragma unroll
  for (int m = F4R; m < 64; m <<= 1)
#pragma unroll
    for (int e = 0; e < 4; ++e) part[e] = xor_sum(part[e], m);
  if (lane < F4R)
#pragma unroll
    for (int e = 0; e < 4; ++e) sred[wv][4 * lane + e] = part[e];
  __syncthreads();
  for (int j = tid; j < D; j += NTHR) {
    float acc = 0.f;
#pragma unroll
    for (int w2 = 0; w2 < NTHR / 64; ++w2) acc += sred[w2][j];
    a.o_part[((size_t)bh * (D / RB) + rb) * D + j] = acc;
  }
}

template <typename T, int D>
__global__ __launch_bounds__(NTHR) void decode_window_kernel(DecodeArgs a) {
  constexpr int VEC = Tr<T>::VEC;
  constexpr int VPR = D / VEC;                // 16-byte vectors per ring row
  constexpr int RPP = NTHR / VPR;             // ring rows per pass
  constexpr int NR = KB / RPP;                // ring vectors per thread per block
  static_assert(NTHR % VPR == 0 && KB % RPP == 0, "thread maps");

  extern __shared__ __align__(16) float slog[];   // [M + W] logits, then probabilities
  __shared__ float sq[D], sk[D], sv[D], sgla[D];
  __shared__ float sstat[2][NTHR / 64];

  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int bh = blockIdx.x;
  const int b = bh / a.H, h = bh % a.H;
  const int W = a.W, M = a.M;
  unsigned int* posu = reinterpret_cast<unsigned int*>(a.pos);
  const int pos = (int)(*reinterpret_cast<volatile unsigned int*>(posu + b) & 0x00FFFFFFu);
  const int slot = pos % W;
  const int n = min(pos + 1, W);
  const size_t vo = (size_t)bh * D;
  const T* qg = reinterpret_cast<const T*>(a.q) + vo;
  const T* kg = reinterpret_cast<const T*>(a.k) + vo;
  const T* vg = reinterpret_cast<const T*>(a.v) + vo;
  const T* rk = reinterpret_cast<const T*>(a.ring_k) + (size_t)bh * W * D;
  const T* rv = reinterpret_cast<const T*>(a.ring_v) + (size_t)bh * W * D;

  // ---- issue every load of the step
  const int cv = tid % VPR, s0 = tid / VPR;
  V16 kr[NR], vr[NR];
#pragma unroll
  for (int u = 0; u < NR; ++u) {
    const int s = s0 + u * RPP;
    const bool ok = s < n && s != slot;
    kr[u] = ok ? ldg16(rk + (size_t)s * D + cv * VEC) : zero16();
    vr[u] = ok ? ldg16(rv + (size_t)s * D + cv * VEC) : zero16();
  }
  // meta keys: rows m = s0 + p * RPP of the ring thread map (M <= 16)
  constexpr int NMP = (16 + RPP - 1) / RPP;
  const T* mk = reinterpret_cast<const T*>(a.meta_k) + (size_t)h * M * D;
  V16 mkr[NMP];
#pragma unroll
  for (int p = 0; p < NMP; ++p) {
    const int m = s0 + p * RPP;
    mkr[p] = m < M ? ldg16(mk + (size_t)m * D + cv * VEC) : zero16();
  }
  for (int i = tid; i < D; i += NTHR) {
    sq[i] = Tr<T>::to_f(qg[i]);
    sk[i] = Tr<T>::to_f(kg[i]);
    sv[i] = Tr<T>::to_f(vg[i]);
    float og = 0.f;
#pragma unroll
    for (int p = 0; p < D / RB; ++p) og += a.o_part[((size_t)bh * (D / RB) + p) * D + i];
    sgla[i] = og;
  }
  __syncthreads();

  // ---- window logits (log2 units): meta keys, then ring slots (new token from the inputs)
  const float sl2 = a.scale * LOG2E;
  float lmax = -INFINITY;
#pragma unroll
  for (int p = 0; p < NMP; ++p) {
    const int m = s0 + p * RPP;
    float acc = 0.f;
#pragma unroll
    for (int e = 0; e < VEC; ++e) acc += sq[cv * VEC + e] * v16_get(mkr[p], e, (T*)nullptr);
    acc = group_sum<VPR>(acc);
    if (m < M) {
      if (cv == 0) slog[m] = acc * sl2;
      lmax = fmaxf(lmax, acc * sl2);
    }
  }
  for (int blk = 0; blk < n; blk += KB) {
    if (blk > 0) {   // windows longer than one register block: load the next block
#pragma unroll
      for (int u = 0; u < NR; ++u) {
        const int s = blk + s0 + u * RPP;
        kr[u] = (s < n && s != slot) ? ldg16(rk + (size_t)s * D + cv * VEC) : zero16();
      }
    }
#pragma unroll
    for (int u = 0; u < NR; ++u) {
      const int s = blk + s0 + u * RPP;
      float acc = 0.f;
      if (s == slot) {
#pragma unroll
        for (int e = 0; e < VEC; ++e) acc += sq[cv * VEC + e] * sk[cv * VEC + e];
      } else {
#pragma unroll
        for (int e = 0; e < VEC; ++e) acc += sq[cv * VEC + e] * v16_get(kr[u], e, (T*)nullptr);
      }
      acc = group_sum<VPR>(acc);
      if (s < n) {
        if (cv == 0) slog[M + s] = acc * sl2;
        lmax = fmaxf(lmax, acc * sl2);
      }
    }
  }
#pragma unroll
  for (int m = 1; m < 64; m <<= 1) lmax = xor_max(lmax, m);
  if (lane == 0) sstat[0][wv] = lmax;
  __syncthreads();
  float gmax = sstat[0][0];
#pragma unroll
  for (int i = 1; i < NTHR / 64; ++i) gmax = fmaxf(gmax, sstat[0][i]);
  float lsum = 0.f;
  for (int e = tid; e < M + n; e += NTHR) {
    const float p = fast_exp2(slog[e] - gmax);
    slog[e] = p;
    lsum += p;
  }
#pragma unroll
  for (int m = 1; m < 64; m <<= 1) lsum = xor_sum(lsum, m);
  if (lane == 0) sstat[1][wv] = lsum;
  __syncthreads();
  float l = 0.f;
#pragma unroll
  for (int i = 0; i < NTHR / 64; ++i) l += sstat[1][i];

  // ---- o_swa: thread sums p_s v_s over its ring rows for its VEC columns
  float ow[VEC];
#pragma unroll
  for (int e = 0; e < VEC; ++e) ow[e] = 0.f;
  for (int blk = 0; blk < n; blk += KB) {
    if (blk > 0) {
#pragma unroll
      for (int u = 0; u < NR; ++u) {
        const int s = blk + s0 + u * RPP;
        vr[u] = (s < n && s != slot) ? ldg16(rv + (size_t)s * D + cv * VEC) : zero16();
      }
    }
#pragma unroll
    for (int u = 0; u < NR; ++u) {
      const int s = blk + s0 + u * RPP;
      if (s < n) {
        const float p = slog[M + s];
        if (s == slot) {
#pragma unroll
          for (int e = 0; e < VEC; ++e) ow[e] += p * sv[cv * VEC + e];
        } else {
#pragma unroll
          for (int e = 0; e < VEC; ++e) ow[e] += p * v16_get(vr[u], e, (T*)nullptr);
        }
      }
    }
  }
  if (a.meta_v != nullptr) {
    for (int m = s0; m < M; m += RPP) {
      const V16 x = ldg16(reinterpret_cast<const T*>(a.meta_v) + ((size_t)h * M + m) * D + cv * VEC);
      const float p = slog[m];
#pragma unroll
      for (int e = 0; e < VEC; ++e) ow[e] += p * v16_get(x, e, (T*)nullptr);
    }
  }
  // threads sharing cv differ in the lane bits above log2(VPR), then across waves
#pragma unroll
  for (int m = VPR; m < 64; m <<= 1)
#pragma unroll
    for (int e = 0; e < VEC; ++e) ow[e] = xor_sum(ow[e], m);
  __shared__ float swin[NTHR / 64][D];
  if (lane < VPR)
#pragma unroll
    for (int e = 0; e < VEC; ++e) swin[wv][lane * VEC + e] = ow[e];
  __syncthreads();
  for (int j = tid; j < D; j += NTHR) {
    float osw = 0.f;
#pragma unroll
    for (int w2 = 0; w2 < NTHR / 64; ++w2) osw += swin[w2][j];
    reinterpret_cast<T*>(a.o)[vo + j] = Tr<T>::from_f(sgla[j] + a.mix * osw / l);
  }
  // ---- ring: the new key and value into slot pos mod W
  {
    T* rkw = reinterpret_cast<T*>(a.ring_k) + ((size_t)bh * W + slot) * D;
    T* rvw = reinterpret_cast<T*>(a.ring_v) + ((size_t)bh * W + slot) * D;
    for (int d = tid; d < D; d += NTHR) {   // exact: the LDS copies came from these values
      put_elem(rkw + d, sk[d]);
      put_elem(rvw + d, sv[d]);
    }
  }
  // ---- pos: the last of the H workgroups of sequence b advances it
  // (no fence: nothing this step writes is read by another workgroup of the step;
  // the next step is a later launch)
  if (tid == 0) {
    const unsigned int old = atomicAdd(posu + b, 1u << 24);
    if ((old >> 24) == (unsigned int)(a.H - 1)) atomicExch(posu + b, (old & 0x00FFFFFFu) + 1u);
  }
}

template <typename T, int D>
hipError_t launch_decode_t(const DecodeArgs& a, hipStream_t st) {
  hipLaunchKernelGGL((decode_state_kernel<T, D>), dim3(a.B * a.H * (D / RB)), dim3(NTHR), 0, st, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const size_t lds = sizeof(float) * (size_t)(a.M + a.W);
  hipLaunchKernelGGL((decode_window_kernel<T, D>), dim3(a.B * a.H), dim3(NTHR), lds, st, a);
  return hipGetLastError();
}

}  // namespace

size_t decode_workspace_bytes(int B, int H, int D) { return sizeof(float) * (size_t)B * H * (D / RB) * D; }

hipError_t launch_decode(const DecodeArgs& a, int dtype, int D, hipStream_t st) {
  if (dtype == 1) {
    if (D == 128) return launch_decode_t<bf16_t, 128>(a, st);
    if (D == 64) return launch_decode_t<bf16_t, 64>(a, st);
  } else if (dtype == 0) {
    if (D == 64) return launch_decode_t<float, 64>(a, st);
    if (D == 128) return launch_decode_t<float, 128>(a, st);
  }
  return hipErrorInvalidValue;
}

}  // namespace lz
