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
// NP = d/64 workgroups per (b, h).  Part j of a head owns the value columns 64j .. 64j+63:
//   - streams those columns of every state row: S <- diag(exp g) S + k^T v, and forms
//     o_gla = q S for its columns (a sum over rows, inside the workgroup);
//   - forms the logits of all filled ring slots and the M meta keys (whole key rows; the
//     NP parts of a head read the same key rows, placed on one XCD so that the shared L2
//     serves them) and the softmax over them, then the value sum of its columns; the new
//     token's slot is taken from the inputs, never from the ring;
//   - writes o for its columns, o = o_gla + mix * o_swa, and its columns of the new key and
//     value into slot pos mod W.
// No partial leaves a workgroup: the step needs no workspace and no combine.  pos, read by
// every workgroup of a sequence, advances in a second, one-workgroup launch (the kernel
// boundary orders every read before the update).  Passing pos between the workgroups of one
// launch instead costs more than that launch on this chip: device-scope atomics on a
// sequence's word contend across the XCDs, and a device-scope fence writes back an XCD's L2.
#include "lz_common.hpp"
#include "lz_kernels.hpp"

namespace lz {

namespace {

constexpr int NTHR = 256;
constexpr int CB = 64;           // value columns of the state per workgroup
constexpr int KBP = 32;          // ring slots per register block of key rows
constexpr int NKB = 4;           // key blocks in flight at once (a 128-slot window in one round)
constexpr int NVR = 4;           // value rows per thread loaded ahead of the softmax

// FEAT: the state update and readout use phi(k), phi(q) given as fp32 log features lk, lq
// [B,H,d] (S <- diag(exp g) S + exp(lk)^T v, o_gla = exp(lq) S); the window keeps q and k.
template <typename T, int D, bool FEAT>
__global__ __launch_bounds__(NTHR) void decode_kernel(DecodeArgs a) {
  constexpr int NP = D / CB;                  // column parts per head
  constexpr int F4C = CB / 4;                 // float4 per row of the part's state columns
  constexpr int RS = NTHR / F4C;              // state rows per pass
  constexpr int RPT = D / RS;                 // state rows per thread
  constexpr int VEC = Tr<T>::VEC;
  constexpr int VPR = D / VEC;                // 16-byte vectors per key row
  constexpr int RPP = NTHR / VPR;             // key rows per pass
  constexpr int NR = (KBP + RPP - 1) / RPP;   // key vectors per thread per block
  constexpr int NMP = (16 + RPP - 1) / RPP;   // meta-key passes (M <= 16)
  constexpr int SVP = CB / VEC;               // 16-byte vectors of the part's columns of a value row
  constexpr int SRP = NTHR / SVP;             // value rows per pass
  static_assert(D % CB == 0 && NTHR % F4C == 0 && RPT * RS == D && NTHR % VPR == 0 && NTHR % SVP == 0,
                "thread maps");

  extern __shared__ __align__(16) float slog[];   // [W + 16] logits of the ring slots and the meta keys,
                                                  // then their probabilities
  __shared__ float sgla[NTHR / 64][CB], sswa[NTHR / 64][CB];
  __shared__ float sq[D], sk[D], sv[D];
  __shared__ float sstat[2][NTHR / 64];

  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  // workgroup -> (head, part): the NP parts of a head are 8 workgroups apart (one XCD) and
  // dispatched together; a last group of fewer than 8 heads takes its parts consecutively
  const int BH = a.B * a.H, full = BH / 8 * 8, g = blockIdx.x;
  int bh, part;
  if (g < full * NP) {
    bh = g / (8 * NP) * 8 + g % 8;
    part = g / 8 % NP;
  } else {
    bh = full + (g - full * NP) / NP;
    part = (g - full * NP) % NP;
  }
  const int b = bh / a.H, h = bh % a.H;
  const int W = a.W, M = a.M;
  const int c0 = part * CB;                   // first value column of the part
  const size_t vo = (size_t)bh * D;
  const T* rk = reinterpret_cast<const T*>(a.ring_k) + (size_t)bh * W * D;
  const T* rv = reinterpret_cast<const T*>(a.ring_v) + (size_t)bh * W * D;

  // ---- issue the step's loads: the part's state columns, the first key block (slots clamped,
  // masked when used: no load waits for pos), pos, meta keys, inputs
  const int c4 = tid % F4C, r0 = tid / F4C;
  float* S = a.state + (size_t)bh * D * D + c0;
  f32x4 st[RPT];
#pragma unroll
  for (int u = 0; u < RPT; ++u) st[u] = *reinterpret_cast<const f32x4*>(S + (size_t)(r0 + u * RS) * D + 4 * c4);
  const int cv = tid % VPR, s0 = tid / VPR;
  V16 kr[NKB][NR];
  // NKB blocks of key rows from slot `base` (rows clamped into the ring, masked when used)
  auto load_keys = [&](int base) {
#pragma unroll
    for (int j = 0; j < NKB; ++j)
#pragma unroll
      for (int u = 0; u < NR; ++u)
        kr[j][u] = ldg16(rk + (size_t)min(base + j * KBP + s0 + u * RPP, W - 1) * D + cv * VEC);
  };
  load_keys(0);
  const int pos = a.pos[b];
  const T* mk = reinterpret_cast<const T*>(a.meta_k) + (size_t)h * M * D;
  V16 mkr[NMP];
#pragma unroll
  for (int p = 0; p < NMP; ++p) {
    const int m = s0 + p * RPP;
    mkr[p] = m < M ? ldg16(mk + (size_t)m * D + cv * VEC) : zero16();
  }
  const T* qg = reinterpret_cast<const T*>(a.q) + vo;
  const T* kg = reinterpret_cast<const T*>(a.k) + vo;
  const T* vg = reinterpret_cast<const T*>(a.v) + vo;
  f32x4 vv;
#pragma unroll
  for (int e = 0; e < 4; ++e) vv[e] = Tr<T>::to_f(vg[c0 + 4 * c4 + e]);
  float qi[RPT], ki[RPT], ai[RPT];
#pragma unroll
  for (int u = 0; u < RPT; ++u) {
    const int i = r0 + u * RS;
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

  // ---- state columns: decay + rank-1 update, o_gla = q S of the columns
  {
    f32x4 pq = f32x4{0, 0, 0, 0};
#pragma unroll
    for (int u = 0; u < RPT; ++u) {
      const f32x4 x = ai[u] * st[u] + ki[u] * vv;
      *reinterpret_cast<f32x4*>(S + (size_t)(r0 + u * RS) * D + 4 * c4) = x;
      pq += qi[u] * x;
    }
    // threads sharing c4 differ in the lane bits above log2(F4C), then across waves
#pragma unroll
    for (int m = F4C; m < 64; m <<= 1)
#pragma unroll
      for (int e = 0; e < 4; ++e) pq[e] = xor_sum(pq[e], m);
    if (lane < F4C)
#pragma unroll
      for (int e = 0; e < 4; ++e) sgla[wv][4 * lane + e] = pq[e];
  }
  __syncthreads();   // sq, sk, sv visible

  // the first NVR value rows of this thread (its columns of the part), loaded while the logits
  // and the softmax are formed
  const int cs = tid % SVP, t0 = tid / SVP;
  const int col = c0 + cs * VEC;
  V16 vr[NVR];
#pragma unroll
  for (int u = 0; u < NVR; ++u) vr[u] = ldg16(rv + (size_t)min(t0 + u * SRP, W - 1) * D + col);

  // ---- window logits (log2 units) of the filled slots, then the meta keys
  const int slot = pos % W;
  const int n = min(pos + 1, W);              // filled slots, the new token's included
  const float sl2 = a.scale * LOG2E;
  float lmax = -INFINITY;
  for (int base = 0; base < n; base += NKB * KBP) {
    if (base > 0) load_keys(base);
#pragma unroll
    for (int j = 0; j < NKB; ++j)
#pragma unroll
      for (int u = 0; u < NR; ++u) {
        const int sl = base + j * KBP + s0 + u * RPP;
        float acc = 0.f;
        if (sl == slot) {
#pragma unroll
          for (int e = 0; e < VEC; ++e) acc += sq[cv * VEC + e] * sk[cv * VEC + e];
        } else {
#pragma unroll
          for (int e = 0; e < VEC; ++e) acc += sq[cv * VEC + e] * v16_get(kr[j][u], e, (T*)nullptr);
        }
        acc = group_sum<VPR>(acc);
        if (sl < n && u * RPP < KBP) {
          if (cv == 0) slog[sl] = acc * sl2;
          lmax = fmaxf(lmax, acc * sl2);
        }
      }
  }
#pragma unroll
  for (int p = 0; p < NMP; ++p) {
    const int m = s0 + p * RPP;
    float acc = 0.f;
#pragma unroll
    for (int e = 0; e < VEC; ++e) acc += sq[cv * VEC + e] * v16_get(mkr[p], e, (T*)nullptr);
    acc = group_sum<VPR>(acc);
    if (m < M) {
      if (cv == 0) slog[W + m] = acc * sl2;
      lmax = fmaxf(lmax, acc * sl2);
    }
  }
  lmax = wave_max(lmax);
  if (lane == 0) sstat[0][wv] = lmax;
  __syncthreads();   // logits and maxima visible
  float pmax = sstat[0][0];
#pragma unroll
  for (int i = 1; i < NTHR / 64; ++i) pmax = fmaxf(pmax, sstat[0][i]);
  float lsum = 0.f;
  for (int e = tid; e < n; e += NTHR) {
    const float p = fast_exp2(slog[e] - pmax);
    slog[e] = p;
    lsum += p;
  }
  for (int e = tid; e < M; e += NTHR) {
    const float p = fast_exp2(slog[W + e] - pmax);
    slog[W + e] = p;
    lsum += p;
  }
  lsum = wave_sum(lsum);
  if (lane == 0) sstat[1][wv] = lsum;
  __syncthreads();   // probabilities and partial sums visible

  // ---- unnormalised value sum of the part's columns
  float ow[VEC];
#pragma unroll
  for (int e = 0; e < VEC; ++e) ow[e] = 0.f;
  auto add_row = [&](int sl, const V16& x) {
    const float p = slog[sl];
    if (sl == slot) {
#pragma unroll
      for (int e = 0; e < VEC; ++e) ow[e] += p * sv[col + e];
    } else {
#pragma unroll
      for (int e = 0; e < VEC; ++e) ow[e] += p * v16_get(x, e, (T*)nullptr);
    }
  };
#pragma unroll
  for (int u = 0; u < NVR; ++u)
    if (t0 + u * SRP < n) add_row(t0 + u * SRP, vr[u]);
  for (int sl = t0 + NVR * SRP; sl < n; sl += SRP) add_row(sl, ldg16(rv + (size_t)sl * D + col));
  if (a.meta_v != nullptr) {
    for (int m = t0; m < M; m += SRP) {
      const V16 x = ldg16(reinterpret_cast<const T*>(a.meta_v) + ((size_t)h * M + m) * D + col);
      const float p = slog[W + m];
#pragma unroll
      for (int e = 0; e < VEC; ++e) ow[e] += p * v16_get(x, e, (T*)nullptr);
    }
  }
  // threads sharing cs differ in the lane bits above log2(SVP), then across waves
#pragma unroll
  for (int m = SVP; m < 64; m <<= 1)
#pragma unroll
    for (int e = 0; e < VEC; ++e) ow[e] = xor_sum(ow[e], m);
  if (lane < SVP)
#pragma unroll
    for (int e = 0; e < VEC; ++e) sswa[wv][lane * VEC + e] = ow[e];
  __syncthreads();

  // ---- o of the part's columns, the part's columns of the new key and value into the ring
  float l = 0.f;
#pragma unroll
  for (int i = 0; i < NTHR / 64; ++i) l += sstat[1][i];
  for (int j = tid; j < CB; j += NTHR) {
    float og = 0.f, osw = 0.f;
#pragma unroll
    for (int w2 = 0; w2 < NTHR / 64; ++w2) {
      og += sgla[w2][j];
      osw += sswa[w2][j];
    }
    reinterpret_cast<T*>(a.o)[vo + c0 + j] = Tr<T>::from_f(og + a.mix * osw / l);
    // exact: the LDS copies came from these values
    put_elem(reinterpret_cast<T*>(a.ring_k) + ((size_t)bh * W + slot) * D + c0 + j, sk[c0 + j]);
    put_elem(reinterpret_cast<T*>(a.ring_v) + ((size_t)bh * W + slot) * D + c0 + j, sv[c0 + j]);
  }

}

// pos advances after every workgroup of the step has read it: a launch of its own
__global__ void decode_pos_kernel(int32_t* pos, int B) {
  const int b = blockIdx.x * blockDim.x + threadIdx.x;
  if (b < B) pos[b] = pos[b] + 1;
}

template <typename T, int D>
hipError_t launch_decode_t(const DecodeArgs& a, hipStream_t st) {
  constexpr int NP = D / CB;
  const size_t lds = sizeof(float) * (size_t)(a.W + 16);
  if (a.lq != nullptr)
    hipLaunchKernelGGL((decode_kernel<T, D, true>), dim3(a.B * a.H * NP), dim3(NTHR), lds, st, a);
  else
    hipLaunchKernelGGL((decode_kernel<T, D, false>), dim3(a.B * a.H * NP), dim3(NTHR), lds, st, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(decode_pos_kernel, dim3((a.B + 255) / 256), dim3(256), 0, st, a.pos, a.B);
  return hipGetLastError();
}

}  // namespace

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
