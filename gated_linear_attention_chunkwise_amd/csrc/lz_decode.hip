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
// One launch per step, NP = d/32 workgroups per (b, h).  Part j of a head
//   - streams state rows 32j .. 32j+31: S <- diag(exp g) S + k^T v, and forms
//     the rows' partial q . S;
//   - covers ring slots [j*WS, (j+1)*WS) (WS = ceil(W / NP); part 0 also the M
//     meta keys): partial softmax statistics of its logits (max m_j and sum
//     l_j, log2 units) and the unnormalised partial sum o_j of its values; the
//     new token's slot is taken from the inputs, never from the ring, and the
//     part owning it writes the new key and value there;
//   - writes both partials to the workspace.
// Every workgroup moves the same share of the step's bytes (state rows and ring
// slots alike), so the state stream and the window read fill the chip together.
// A second, small launch (one workgroup per (b, h)) combines the partials,
//   o = sum_j gla_j + mix * sum_j e^{m_j - m} o_j / sum_j e^{m_j - m} l_j  (m = max_j m_j),
// and advances pos: the kernel boundary orders the partials' writes and reads, and
// orders every read of pos (first launch) before its update (second launch).
#include <atomic>
#include <mutex>

#include "lz_common.hpp"
#include "lz_kernels.hpp"

namespace lz {

// The decode step's partials for callers that cannot allocate (lizard_attn_decode_step_noalloc):
// one array per device, resident until the process ends.  Host code never passes its name to a
// kernel (on the host it is only a stand-in for the symbol); it passes the device address that
// hipGetSymbolAddress returns for the current device.
static __device__ __align__(256) unsigned char scratch[kDecodeScratchBytes];

namespace {

constexpr int NTHR = 256;
constexpr int RB = 32;           // state rows (and the share of ring slots) per workgroup
constexpr int KBP = 32;          // ring slots per register block

// workspace: per (b, h, part) [D] partial q.S, [D] unnormalised window sum, (max, sum)
template <int D>
struct DecWs {
  static constexpr int NP = D / RB;
  static constexpr int PS = 2 * D + 4;       // floats per part (16-byte aligned)
  static size_t bytes(int B, int H) { return (size_t)B * H * NP * PS * sizeof(float); }
};

// FEAT: the state update and readout use phi(k), phi(q) given as fp32 log features lk, lq
// [B,H,d] (S <- diag(exp g) S + exp(lk)^T v, o_gla = exp(lq) S); the window keeps q and k.
template <typename T, int D, bool FEAT>
__global__ __launch_bounds__(NTHR) void decode_kernel(DecodeArgs a) {
  using WS_ = DecWs<D>;
  constexpr int NP = WS_::NP, PS = WS_::PS;
  constexpr int F4R = D / 4;                  // float4 per state row
  constexpr int RPT = RB * F4R / NTHR;        // state rows per thread
  constexpr int RS = NTHR / F4R;              // row stride between a thread's rows
  constexpr int VEC = Tr<T>::VEC;
  constexpr int VPR = D / VEC;                // 16-byte vectors per ring row
  constexpr int RPP = NTHR / VPR;             // ring rows per pass
  constexpr int NR = (KBP + RPP - 1) / RPP;   // ring vectors per thread per block
  constexpr int NMP = (16 + RPP - 1) / RPP;   // meta-key passes (M <= 16)
  static_assert(NTHR % F4R == 0 && RPT * RS == RB && NTHR % VPR == 0, "thread maps");

  extern __shared__ __align__(16) float slog[];   // [WS + 16] logits of the part, then probabilities
  __shared__ float sred[NTHR / 64][D];
  __shared__ float sq[D], sk[D], sv[D];
  __shared__ float sstat[2][NTHR / 64];

  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int bh = blockIdx.x / NP, part = blockIdx.x % NP;
  const int b = bh / a.H, h = bh % a.H;
  const int W = a.W, M = a.M;
  const int WSL = (W + NP - 1) / NP;          // ring slots per part
  const int lo = part * WSL, hi = min(W, lo + WSL);
  const size_t vo = (size_t)bh * D;
  float* wsp = a.o_part + ((size_t)bh * NP) * PS;
  const unsigned int* posu = reinterpret_cast<const unsigned int*>(a.pos);
  const T* rk = reinterpret_cast<const T*>(a.ring_k) + (size_t)bh * W * D;
  const T* rv = reinterpret_cast<const T*>(a.ring_v) + (size_t)bh * W * D;

  // ---- issue the step's loads: state rows, the first ring block (slots clamped, masked when
  // used: no load waits for pos), pos, meta keys, inputs
  const int c4 = tid % F4R, r0 = tid / F4R;
  float* S = a.state + ((size_t)bh * D + part * RB) * D;
  f32x4 st[RPT];
#pragma unroll
  for (int u = 0; u < RPT; ++u) st[u] = *reinterpret_cast<const f32x4*>(S + (size_t)(r0 + u * RS) * D + 4 * c4);
  const int cv = tid % VPR, s0 = tid / VPR;
  V16 kr[NR], vr[NR];
  auto load_block = [&](int blk) {
#pragma unroll
    for (int u = 0; u < NR; ++u) {
      const int sl = min(blk + s0 + u * RPP, hi - 1);
      kr[u] = ldg16(rk + (size_t)sl * D + cv * VEC);
      vr[u] = ldg16(rv + (size_t)sl * D + cv * VEC);
    }
  };
  load_block(lo);
  const int pos = (int)posu[b];
  const T* mk = reinterpret_cast<const T*>(a.meta_k) + (size_t)h * M * D;
  V16 mkr[NMP];
#pragma unroll
  for (int p = 0; p < NMP; ++p) {
    const int m = s0 + p * RPP;
    mkr[p] = (part == 0 && m < M) ? ldg16(mk + (size_t)m * D + cv * VEC) : zero16();
  }
  const T* qg = reinterpret_cast<const T*>(a.q) + vo;
  const T* kg = reinterpret_cast<const T*>(a.k) + vo;
  const T* vg = reinterpret_cast<const T*>(a.v) + vo;
  f32x4 vv;
#pragma unroll
  for (int e = 0; e < 4; ++e) vv[e] = Tr<T>::to_f(vg[4 * c4 + e]);
  float qi[RPT], ki[RPT], ai[RPT];
#pragma unroll
  for (int u = 0; u < RPT; ++u) {
    const int i = part * RB + r0 + u * RS;
    if constexpr (FEAT) {
      qi[u] = __expf(a.lq[vo + i]);
      ki[u] = __expf(a.lk[vo + i]);
    } else {
      qi[u] = Tr<T>::to_f(qg[i]);
      ki[u] = Tr<T>::to_f(kg[i]);
    }
    ai[u] = __expf(a.gate ? a.g[bh] : a.g[vo + i]);   // scalar gate: one per head
  }
  for (int i = tid; i < D; i += NTHR) {
    sq[i] = Tr<T>::to_f(qg[i]);
    sk[i] = Tr<T>::to_f(kg[i]);
    sv[i] = Tr<T>::to_f(vg[i]);
  }

  // ---- state rows: decay + rank-1 update, partial q . S of the rows
  {
    f32x4 pq = f32x4{0, 0, 0, 0};
#pragma unroll
    for (int u = 0; u < RPT; ++u) {
      const f32x4 x = ai[u] * st[u] + ki[u] * vv;
      *reinterpret_cast<f32x4*>(S + (size_t)(r0 + u * RS) * D + 4 * c4) = x;
      pq += qi[u] * x;
    }
    // threads sharing c4 differ in the lane bits above log2(F4R), then across waves
#pragma unroll
    for (int m = F4R; m < 64; m <<= 1)
#pragma unroll
      for (int e = 0; e < 4; ++e) pq[e] = xor_sum(pq[e], m);
    if (lane < F4R)
#pragma unroll
      for (int e = 0; e < 4; ++e) sred[wv][4 * lane + e] = pq[e];
  }
  __syncthreads();
  for (int j = tid; j < D; j += NTHR) {
    float acc = 0.f;
#pragma unroll
    for (int w2 = 0; w2 < NTHR / 64; ++w2) acc += sred[w2][j];
    wsp[part * PS + j] = acc;
  }

  // ---- window logits (log2 units) of this part's slots that hold a token, then its meta keys
  const int slot = pos % W;
  const int n = min(pos + 1, W);              // filled slots, the new token's included
  const float sl2 = a.scale * LOG2E;
  const int nhold = max(0, min(hi, n) - lo);  // this part's filled slots: lo .. lo+nhold-1
  float lmax = -INFINITY;
  for (int blk = lo; blk < lo + nhold; blk += KBP) {
    if (blk > lo) load_block(blk);
#pragma unroll
    for (int u = 0; u < NR; ++u) {
      const int sl = blk + s0 + u * RPP;
      float acc = 0.f;
      if (sl == slot) {
#pragma unroll
        for (int e = 0; e < VEC; ++e) acc += sq[cv * VEC + e] * sk[cv * VEC + e];
      } else {
#pragma unroll
        for (int e = 0; e < VEC; ++e) acc += sq[cv * VEC + e] * v16_get(kr[u], e, (T*)nullptr);
      }
      acc = group_sum<VPR>(acc);
      if (sl < lo + nhold && u * RPP < KBP) {
        if (cv == 0) slog[sl - lo] = acc * sl2;
        lmax = fmaxf(lmax, acc * sl2);
      }
    }
  }
  if (part == 0) {
#pragma unroll
    for (int p = 0; p < NMP; ++p) {
      const int m = s0 + p * RPP;
      float acc = 0.f;
#pragma unroll
      for (int e = 0; e < VEC; ++e) acc += sq[cv * VEC + e] * v16_get(mkr[p], e, (T*)nullptr);
      acc = group_sum<VPR>(acc);
      if (m < M) {
        if (cv == 0) slog[WSL + m] = acc * sl2;
        lmax = fmaxf(lmax, acc * sl2);
      }
    }
  }
  lmax = wave_max(lmax);
  if (lane == 0) sstat[0][wv] = lmax;
  __syncthreads();
  float pmax = sstat[0][0];
#pragma unroll
  for (int i = 1; i < NTHR / 64; ++i) pmax = fmaxf(pmax, sstat[0][i]);
  const int nmeta = part == 0 ? M : 0;
  float lsum = 0.f;
  if (pmax > -INFINITY) {
    for (int e = tid; e < nhold; e += NTHR) {
      const float p = fast_exp2(slog[e] - pmax);
      slog[e] = p;
      lsum += p;
    }
    for (int e = tid; e < nmeta; e += NTHR) {
      const float p = fast_exp2(slog[WSL + e] - pmax);
      slog[WSL + e] = p;
      lsum += p;
    }
  }
  lsum = wave_sum(lsum);
  __syncthreads();   // probabilities visible; sstat[0] read by every thread
  if (lane == 0) sstat[1][wv] = lsum;

  // ---- unnormalised value sum of the part
  float ow[VEC];
#pragma unroll
  for (int e = 0; e < VEC; ++e) ow[e] = 0.f;
  for (int blk = lo; blk < lo + nhold; blk += KBP) {
    if (blk > lo || nhold > KBP) load_block(blk);   // the first block is still held unless reloaded
#pragma unroll
    for (int u = 0; u < NR; ++u) {
      const int sl = blk + s0 + u * RPP;
      if (sl < lo + nhold && u * RPP < KBP) {
        const float p = slog[sl - lo];
        if (sl == slot) {
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
    for (int m = s0; m < nmeta; m += RPP) {
      const V16 x = ldg16(reinterpret_cast<const T*>(a.meta_v) + ((size_t)h * M + m) * D + cv * VEC);
      const float p = slog[WSL + m];
#pragma unroll
      for (int e = 0; e < VEC; ++e) ow[e] += p * v16_get(x, e, (T*)nullptr);
    }
  }
  // threads sharing cv differ in the lane bits above log2(VPR), then across waves
#pragma unroll
  for (int m = VPR; m < 64; m <<= 1)
#pragma unroll
    for (int e = 0; e < VEC; ++e) ow[e] = xor_sum(ow[e], m);
  if (lane < VPR)
#pragma unroll
    for (int e = 0; e < VEC; ++e) sred[wv][lane * VEC + e] = ow[e];
  __syncthreads();
  for (int j = tid; j < D; j += NTHR) {
    float osw = 0.f;
#pragma unroll
    for (int w2 = 0; w2 < NTHR / 64; ++w2) osw += sred[w2][j];
    wsp[part * PS + D + j] = osw;
  }
  if (tid == 0) {
    float l = 0.f;
#pragma unroll
    for (int i = 0; i < NTHR / 64; ++i) l += sstat[1][i];
    wsp[part * PS + 2 * D] = pmax;
    wsp[part * PS + 2 * D + 1] = l;
  }
  // ---- ring: the new key and value into slot pos mod W, by the part that owns it
  if (slot >= lo && slot < hi) {
    T* rkw = reinterpret_cast<T*>(a.ring_k) + ((size_t)bh * W + slot) * D;
    T* rvw = reinterpret_cast<T*>(a.ring_v) + ((size_t)bh * W + slot) * D;
    for (int d = tid; d < D; d += NTHR) {   // exact: the LDS copies came from these values
      put_elem(rkw + d, sk[d]);
      put_elem(rvw + d, sv[d]);
    }
  }

}

// One workgroup per (b, h), one thread per output column: combine the NP partials of the
// head, store o, and advance pos (the last of the H heads of a sequence).
template <typename T, int D>
__global__ __launch_bounds__(D) void decode_combine_kernel(DecodeArgs a) {
  using WS_ = DecWs<D>;
  constexpr int NP = WS_::NP, PS = WS_::PS;
  const int bh = blockIdx.x, d = threadIdx.x, b = bh / a.H;
  const float* wsp = a.o_part + ((size_t)bh * NP) * PS;
  float mj[NP], gmax = -INFINITY;
#pragma unroll
  for (int j = 0; j < NP; ++j) {
    mj[j] = wsp[j * PS + 2 * D];
    gmax = fmaxf(gmax, mj[j]);
  }
  float og = 0.f, osw = 0.f, l = 0.f;
#pragma unroll
  for (int j = 0; j < NP; ++j) {
    const float wj = mj[j] > -INFINITY ? fast_exp2(mj[j] - gmax) : 0.f;
    l += wj * wsp[j * PS + 2 * D + 1];
    og += wsp[j * PS + d];
    osw += wj * wsp[j * PS + D + d];
  }
  reinterpret_cast<T*>(a.o)[(size_t)bh * D + d] = Tr<T>::from_f(og + a.mix * osw / l);
  // pos: nothing in this launch reads it, so head 0's workgroup advances it alone
  if (d == 0 && bh % a.H == 0) a.pos[b] = a.pos[b] + 1;
}

template <typename T, int D>
hipError_t launch_decode_t(const DecodeArgs& a, hipStream_t st) {
  constexpr int NP = D / RB;
  const size_t lds = sizeof(float) * (size_t)((a.W + NP - 1) / NP + 16);
  if (a.lq != nullptr)
    hipLaunchKernelGGL((decode_kernel<T, D, true>), dim3(a.B * a.H * NP), dim3(NTHR), lds, st, a);
  else
    hipLaunchKernelGGL((decode_kernel<T, D, false>), dim3(a.B * a.H * NP), dim3(NTHR), lds, st, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((decode_combine_kernel<T, D>), dim3(a.B * a.H), dim3(D), 0, st, a);
  return hipGetLastError();
}

}  // namespace

size_t decode_workspace_bytes(int B, int H, int D) {
  return D == 128 ? DecWs<128>::bytes(B, H) : DecWs<64>::bytes(B, H);
}

namespace {
constexpr int kMaxDevices = 64;
std::atomic<void*> g_scratch[kMaxDevices];
std::mutex g_scratch_mu;

// Device address of `scratch` on the current device, looked up once per device.
hipError_t scratch_address(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  void* p = g_scratch[dev].load(std::memory_order_acquire);
  if (p == nullptr) {
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    p = g_scratch[dev].load(std::memory_order_relaxed);
    if (p == nullptr) {
      e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
      if (e != hipSuccess) return e;
      if (p == nullptr) return hipErrorInvalidSymbol;
      g_scratch[dev].store(p, std::memory_order_release);
    }
  }
  *out = p;
  return hipSuccess;
}
}  // namespace

hipError_t launch_decode_noalloc(const DecodeArgs& args, int dtype, int D, hipStream_t st) {
  if (decode_workspace_bytes(args.B, args.H, D) > kDecodeScratchBytes) return hipErrorInvalidValue;
  void* p = nullptr;
  const hipError_t e = scratch_address(&p);
  if (e != hipSuccess) return e;
  DecodeArgs a = args;
  a.o_part = reinterpret_cast<float*>(p);   // every partial is written by the step before it is read
  return launch_decode(a, dtype, D, st);
}

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
