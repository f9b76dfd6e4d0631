// lz_general.hip -- the general path of the layer's forward and backward on gfx950.
//
// The chunkwise algorithm of the fast kernels, for the calls those kernels are not laid out for:
// chunks of 16, 32 or 128 tokens, and fp32 operands at d = 128.  As there (gist.science explainer of
// "Lizard: An Efficient Linearization Framework for Large Language Models", English page §2.A state
// update with a per-key-dimension gate, §2.C gates kept in log space), the state passes from chunk
// to chunk and is stored at every chunk boundary in the operand dtype, and a chunk's outputs come
// from the state entering it plus the chunk's own keys:
//   O_c   = (Q~ K^T masked s <= t, with the gate between s and t) V + Q~ S_c,   Q~ = Q e^b
//   S_c+1 = diag(e^Gamma) S_c + (K e^(Gamma - b))^T V
// Every product runs in fp32 on the vector units, one thread per output element with its operands
// read from LDS or memory; this path is for coverage and exactness, not speed.
//
// Gate exponents are formed from 16-token block sums only -- P, the inclusive prefix of the
// log-gates inside each block, and the block totals T -- never as a difference of two long prefixes:
//   b_t - b_s   = P_t - P_s                                        (t, s in one block)
//               = P_t + (T_bs - P_s) + T_{bs+1} + .. + T_{bt-1}    (s in an earlier block)
//   b_t         = T_{c0} + .. + T_{bt-1} + P_t                     (from the chunk start, block c0)
//   Gamma - b_s = (T_bs - P_s) + T_{bs+1} + .. + T_{last}          (to the chunk's last token)
// Each is as accurate as its own size and every exponential is of a value <= 0 (pairs s <= t), so the
// path is exact for every finite g <= 0 without a sub-block form.
//
// Kernels: gen_prefix (P, T), gen_state (forward state sweep), gen_out (window, intra- and
// inter-chunk outputs), gen_dstate (reverse sweep of the state gradient and the boundary row sums of
// dg), gen_gla_bwd (GLA gradients and dg per chunk), gen_delta, gen_win_bwd (window gradients per
// 64-token tile, added to the GLA parts), gen_meta_fold (meta-key gradients, fixed order).
#include <algorithm>
#include <type_traits>

#include "lz_common.hpp"
#include "lz_kernels.hpp"

namespace lz {
namespace {

constexpr int GTH = 256;   // threads per workgroup
constexpr int JS = 32;     // value columns per workgroup of the sweeps
constexpr int WT = 64;     // tokens per tile of the window backward

__device__ __forceinline__ float tof(float x) { return x; }
__device__ __forceinline__ float tof(bf16_t x) { return bf2f(x.bits); }

size_t rup(size_t x) { return (x + 255) / 256 * 256; }

template <typename K>
hipError_t lds_attr(K kern, size_t bytes) {
  return hipFuncSetAttribute(reinterpret_cast<const void*>(kern), hipFuncAttributeMaxDynamicSharedMemorySize,
                             (int)bytes);
}

// Block sums of one head's gates (Dg = 1 for one gate per token, d otherwise).
struct Gates {
  const float* P;    // [L][Dg] inclusive prefix inside the 16-token block
  const float* Tb;   // [ceil(L/16)][Dg] block totals
  int Dg;
  __device__ __forceinline__ float p(int t, int i) const { return P[(size_t)t * Dg + (Dg == 1 ? 0 : i)]; }
  __device__ __forceinline__ float tb(int m, int i) const { return Tb[(size_t)m * Dg + (Dg == 1 ? 0 : i)]; }
  // b_t - b_s for s <= t
  __device__ float diff(int t, int s, int i) const {
    const int bt = t >> 4, bs = s >> 4;
    if (bt == bs) return p(t, i) - p(s, i);
    float x = p(t, i) + (tb(bs, i) - p(s, i));
    for (int m = bs + 1; m < bt; ++m) x += tb(m, i);
    return x;
  }
  // b_t from the chunk start t0 (a multiple of 16)
  __device__ float pre(int t, int t0, int i) const {
    float x = p(t, i);
    for (int m = t0 >> 4; m < (t >> 4); ++m) x += tb(m, i);
    return x;
  }
  // Gamma - b_s: the gates after s up to the chunk's last token tl
  __device__ float suf(int s, int tl, int i) const {
    float x = tb(s >> 4, i) - p(s, i);
    for (int m = (s >> 4) + 1; m <= (tl >> 4); ++m) x += tb(m, i);
    return x;
  }
  // Gamma: the gates of tokens t0 .. tl
  __device__ float tot(int t0, int tl, int i) const {
    float x = 0.f;
    for (int m = t0 >> 4; m <= (tl >> 4); ++m) x += tb(m, i);
    return x;
  }
};

__device__ __forceinline__ Gates head_gates(const float* P, const float* Tb, int bh, int L, int Dg) {
  const int NB = (L + 15) / 16;
  return Gates{P + (size_t)bh * L * Dg, Tb + (size_t)bh * NB * Dg, Dg};
}

template <typename T>
__device__ __forceinline__ float dot_rows(const T* a, const T* b, int D) {
  float x = 0.f;
  for (int i = 0; i < D; ++i) x += tof(a[i]) * tof(b[i]);
  return x;
}

// ------------------------------------------------------------------ gate block sums
__global__ __launch_bounds__(128) void gen_prefix_kernel(const float* __restrict__ g, float* __restrict__ P,
                                                         float* __restrict__ Tb, int L, int Dg) {
  const int NB = (L + 15) / 16;
  const int bh = blockIdx.x / NB, blk = blockIdx.x % NB, i = threadIdx.x;
  if (i >= Dg) return;
  const float* gp = g + (size_t)bh * L * Dg;
  float* pp = P + (size_t)bh * L * Dg;
  float acc = 0.f;
  for (int u = 0; u < 16; ++u) {
    const int t = 16 * blk + u;
    if (t >= L) break;
    acc += gp[(size_t)t * Dg + i];
    pp[(size_t)t * Dg + i] = acc;
  }
  Tb[((size_t)bh * NB + blk) * Dg + i] = acc;
}

// ------------------------------------------------------------------ forward state sweep
// One workgroup per (b*h, 32 value columns); thread (j, ig) carries rows ig + 8m of column j0 + j.
template <typename T, int D>
__global__ __launch_bounds__(GTH) void gen_state_kernel(const T* __restrict__ k, const T* __restrict__ v,
                                                        const float* __restrict__ P, const float* __restrict__ Tb,
                                                        T* __restrict__ states, float* __restrict__ state_out,
                                                        int L, int C, int Dg) {
  extern __shared__ __align__(16) unsigned char smem[];
  constexpr int NJ = D / JS, NR = D / 8;
  float* sK = reinterpret_cast<float*>(smem);   // [C][D] k e^(Gamma - b)
  float* sV = sK + C * D;                        // [C][JS]
  float* sDec = sV + C * JS;                     // [D] e^Gamma
  const int tid = threadIdx.x, j = tid & 31, ig = tid >> 5;
  const int bh = blockIdx.x / NJ, j0 = JS * (blockIdx.x % NJ);
  const int NC = (L + C - 1) / C;
  const Gates G = head_gates(P, Tb, bh, L, Dg);
  const size_t hoff = (size_t)bh * L * D;
  float acc[NR];
#pragma unroll
  for (int m = 0; m < NR; ++m) acc[m] = 0.f;
  for (int c = 0; c < NC; ++c) {
    const int t0 = c * C, tl = min(t0 + C, L) - 1, Cv = tl - t0 + 1;
    T* st = states + ((size_t)bh * NC + c) * D * D;
#pragma unroll
    for (int m = 0; m < NR; ++m) put_elem(st + (size_t)(ig + 8 * m) * D + j0 + j, acc[m]);   // S entering c
    __syncthreads();
    for (int e = tid; e < C * D; e += GTH) {
      const int t = e / D, i = e % D;
      sK[e] = t < Cv ? tof(k[hoff + (size_t)(t0 + t) * D + i]) * __expf(G.suf(t0 + t, tl, i)) : 0.f;
    }
    for (int e = tid; e < C * JS; e += GTH) {
      const int t = e / JS, jj = e % JS;
      sV[e] = t < Cv ? tof(v[hoff + (size_t)(t0 + t) * D + j0 + jj]) : 0.f;
    }
    for (int i = tid; i < D; i += GTH) sDec[i] = __expf(G.tot(t0, tl, i));
    __syncthreads();
#pragma unroll
    for (int m = 0; m < NR; ++m) {
      const int i = ig + 8 * m;
      float x = sDec[i] * acc[m];
      for (int t = 0; t < Cv; ++t) x += sK[t * D + i] * sV[t * JS + j];
      acc[m] = x;
    }
  }
  if (state_out != nullptr)
#pragma unroll
    for (int m = 0; m < NR; ++m) state_out[((size_t)bh * D + ig + 8 * m) * D + j0 + j] = acc[m];
}

// ------------------------------------------------------------------ forward outputs of one chunk
template <typename T, int D>
__global__ __launch_bounds__(GTH) void gen_out_kernel(FwdArgs a, const T* __restrict__ states,
                                                      const float* __restrict__ P, const float* __restrict__ Tb,
                                                      int C, int Dg) {
  extern __shared__ __align__(16) unsigned char smem[];
  const int LX = max(C * C, C * D);
  float* sX = reinterpret_cast<float*>(smem);   // intra scores [C][C], then q~ [C][D]
  float* sO = sX + LX;                           // [C][D] outputs (fp32)
  float* sP = sO + C * D;                        // [C][32] window probabilities of a key tile
  float* sMx = sP + C * 32;                      // [C] running max of the logits
  float* sL = sMx + C;                           // [C] softmax denominators
  const int tid = threadIdx.x;
  const int L = a.L, W = a.W, M = a.M, NC = (L + C - 1) / C;
  const int bh = blockIdx.x / NC, c = blockIdx.x % NC, h = bh % a.H;
  const int t0 = c * C, tl = min(t0 + C, L) - 1, Cv = tl - t0 + 1;
  const size_t hoff = (size_t)bh * L * D;
  const T* q = reinterpret_cast<const T*>(a.q) + hoff;
  const T* k = reinterpret_cast<const T*>(a.k) + hoff;
  const T* v = reinterpret_cast<const T*>(a.v) + hoff;
  const T* mk = reinterpret_cast<const T*>(a.meta_k) + (size_t)h * M * D;
  const T* mv = a.meta_v ? reinterpret_cast<const T*>(a.meta_v) + (size_t)h * M * D : nullptr;
  const T* S = states + ((size_t)bh * NC + c) * D * D;
  const Gates G = head_gates(P, Tb, bh, L, Dg);
  const float scale = a.scale;

  // anchor window: softmax of each query over the meta keys and the keys in (t - W, t]
  for (int t = tid; t < Cv; t += GTH) {
    const int tq = t0 + t;
    float mx = -INFINITY, l = 0.f;
    auto absorb = [&](float x) {
      if (x > mx) {
        l = l * __expf(mx - x) + 1.f;
        mx = x;
      } else {
        l += __expf(x - mx);
      }
    };
    for (int m = 0; m < M; ++m) absorb(scale * dot_rows(q + (size_t)tq * D, mk + (size_t)m * D, D));
    for (int s = max(tq - W + 1, 0); s <= tq; ++s) absorb(scale * dot_rows(q + (size_t)tq * D, k + (size_t)s * D, D));
    sMx[t] = mx;
    sL[t] = l;
    if (a.lse != nullptr) a.lse[(size_t)bh * L + tq] = mx + __logf(l);
  }
  for (int e = tid; e < Cv * D; e += GTH) sO[e] = 0.f;
  __syncthreads();
  if (M > 0 && mv != nullptr) {
    for (int e = tid; e < Cv * 32; e += GTH) {
      const int t = e / 32, m = e % 32;
      sP[e] = m < M ? __expf(scale * dot_rows(q + (size_t)(t0 + t) * D, mk + (size_t)m * D, D) - sMx[t]) / sL[t]
                    : 0.f;
    }
    __syncthreads();
    for (int e = tid; e < Cv * D; e += GTH) {
      const int t = e / D, jc = e % D;
      float x = 0.f;
      for (int m = 0; m < M; ++m) x += sP[t * 32 + m] * tof(mv[(size_t)m * D + jc]);
      sO[e] += x;
    }
    __syncthreads();
  }
  const int kmin = max(t0 - W + 1, 0);
  for (int kb = kmin; kb <= tl; kb += 32) {
    for (int e = tid; e < Cv * 32; e += GTH) {
      const int t = e / 32, s = kb + e % 32, tq = t0 + t;
      const bool ok = s <= tl && s <= tq && s > tq - W;
      sP[e] = ok ? __expf(scale * dot_rows(q + (size_t)tq * D, k + (size_t)s * D, D) - sMx[t]) / sL[t] : 0.f;
    }
    __syncthreads();
    const int nk = min(32, tl - kb + 1);
    for (int e = tid; e < Cv * D; e += GTH) {
      const int t = e / D, jc = e % D;
      float x = 0.f;
      for (int u = 0; u < nk; ++u) x += sP[t * 32 + u] * tof(v[(size_t)(kb + u) * D + jc]);
      sO[e] += x;
    }
    __syncthreads();
  }
  for (int e = tid; e < Cv * D; e += GTH) {
    const int t = e / D, jc = e % D;
    if (a.o_swa != nullptr) put_elem(reinterpret_cast<T*>(a.o_swa) + hoff + (size_t)(t0 + t) * D + jc, sO[e]);
    sO[e] *= a.mix;
  }
  // GLA, intra-chunk: scores with the gate between key and query, then their values
  for (int e = tid; e < Cv * Cv; e += GTH) {
    const int t = e / Cv, s = e % Cv;
    float x = 0.f;
    if (s <= t)
      for (int i = 0; i < D; ++i)
        x += tof(q[(size_t)(t0 + t) * D + i]) * tof(k[(size_t)(t0 + s) * D + i]) * __expf(G.diff(t0 + t, t0 + s, i));
    sX[t * C + s] = x;
  }
  __syncthreads();
  for (int e = tid; e < Cv * D; e += GTH) {
    const int t = e / D, jc = e % D;
    float x = 0.f;
    for (int s = 0; s <= t; ++s) x += sX[t * C + s] * tof(v[(size_t)(t0 + s) * D + jc]);
    sO[e] += x;
  }
  __syncthreads();
  // inter-chunk: q~ S with q~ = q e^b
  for (int e = tid; e < Cv * D; e += GTH) {
    const int t = e / D, i = e % D;
    sX[e] = tof(q[(size_t)(t0 + t) * D + i]) * __expf(G.pre(t0 + t, t0, i));
  }
  __syncthreads();
  for (int e = tid; e < Cv * D; e += GTH) {
    const int t = e / D, jc = e % D;
    float x = sO[e];
    for (int i = 0; i < D; ++i) x += sX[t * D + i] * tof(S[(size_t)i * D + jc]);
    if (a.o != nullptr) put_elem(reinterpret_cast<T*>(a.o) + hoff + (size_t)(t0 + t) * D + jc, x);
  }
}

__global__ void gen_zero_kernel(float* p, size_t n) {
  const size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = 0.f;
}

// ------------------------------------------------------------------ backward: state gradient sweep
// Reverse over chunks; stores dS_c, the gradient of the state after chunk c, and per 32-column slice
// the boundary row sums of dg, sum_j S_c[i][j] dS_c[i][j] (S_c = the state entering chunk c + 1).
template <typename T, int D>
__global__ __launch_bounds__(GTH) void gen_dstate_kernel(const T* __restrict__ q, const T* __restrict__ dO,
                                                         const T* __restrict__ states,
                                                         const float* __restrict__ P, const float* __restrict__ Tb,
                                                         float* __restrict__ dS, float* __restrict__ bndp, int L,
                                                         int C, int Dg) {
  extern __shared__ __align__(16) unsigned char smem[];
  constexpr int NJ = D / JS, NR = D / 8;
  float* sQ = reinterpret_cast<float*>(smem);   // [C][D] q e^b
  float* sD = sQ + C * D;                        // [C][JS] dO
  float* sDec = sD + C * JS;                     // [D]
  const int tid = threadIdx.x, j = tid & 31, ig = tid >> 5;
  const int bh = blockIdx.x / NJ, jq = blockIdx.x % NJ, j0 = JS * jq;
  const int NC = (L + C - 1) / C;
  const Gates G = head_gates(P, Tb, bh, L, Dg);
  const size_t hoff = (size_t)bh * L * D;
  float acc[NR];
#pragma unroll
  for (int m = 0; m < NR; ++m) acc[m] = 0.f;
  for (int c = NC - 1; c >= 0; --c) {
    const int t0 = c * C, tl = min(t0 + C, L) - 1, Cv = tl - t0 + 1;
    float* dsc = dS + ((size_t)bh * NC + c) * D * D;
#pragma unroll
    for (int m = 0; m < NR; ++m) {
      const int i = ig + 8 * m;
      dsc[(size_t)i * D + j0 + j] = acc[m];
      const float sv = c + 1 < NC ? tof(states[(((size_t)bh * NC + c + 1) * D + i) * D + j0 + j]) : 0.f;
      float x = sv * acc[m];
#pragma unroll
      for (int o = 16; o > 0; o >>= 1) x += __shfl_xor(x, o, WAVE);   // the 32 columns of this slice
      if (j == 0) bndp[(((size_t)bh * NC + c) * NJ + jq) * D + i] = x;
    }
    __syncthreads();
    for (int e = tid; e < C * D; e += GTH) {
      const int t = e / D, i = e % D;
      sQ[e] = t < Cv ? tof(q[hoff + (size_t)(t0 + t) * D + i]) * __expf(G.pre(t0 + t, t0, i)) : 0.f;
    }
    for (int e = tid; e < C * JS; e += GTH) {
      const int t = e / JS, jj = e % JS;
      sD[e] = t < Cv ? tof(dO[hoff + (size_t)(t0 + t) * D + j0 + jj]) : 0.f;
    }
    for (int i = tid; i < D; i += GTH) sDec[i] = __expf(G.tot(t0, tl, i));
    __syncthreads();
#pragma unroll
    for (int m = 0; m < NR; ++m) {
      const int i = ig + 8 * m;
      float x = sDec[i] * acc[m];
      for (int t = 0; t < Cv; ++t) x += sQ[t * D + i] * sD[t * JS + j];
      acc[m] = x;
    }
    __syncthreads();
  }
}

// ------------------------------------------------------------------ backward: GLA gradients of a chunk
// dq, dk, dv of the GLA branch (fp32, to the workspace) and dg:
//   dA_ts = dO_t . v_s,  A_ts = sum_i q k e^(b_t - b_s)                      (s <= t)
//   dq_t  = sum_s dA_ts k_s e^(b_t - b_s) + e^(b_t) (S_c dO_t)
//   dk_s  = sum_t dA_ts q_t e^(b_t - b_s) + e^(Gamma - b_s) (dS_c v_s)
//   dv_s  = sum_t A_ts dO_t + (k_s e^(Gamma - b_s)) dS_c
//   dg_t  = sum_{u >= t in the chunk} (q_u dq_u - k_u dk_u) + sum_j S_c+1 (.) dS_c   (rows)
template <typename T, int D>
__global__ __launch_bounds__(GTH) void gen_gla_bwd_kernel(BwdArgs a, const T* __restrict__ states,
                                                          const float* __restrict__ dS,
                                                          const float* __restrict__ bndp,
                                                          const float* __restrict__ P, const float* __restrict__ Tb,
                                                          float* __restrict__ dqg, float* __restrict__ dkg,
                                                          float* __restrict__ dvg, int C, int Dg) {
  extern __shared__ __align__(16) unsigned char smem[];
  constexpr int NJ = D / JS;
  const int LX = max(C * C, C * D);
  float* sA = reinterpret_cast<float*>(smem);   // A [C][C], then k e^(Gamma - b) [C][D], then d b [C][D]
  float* sdA = sA + LX;                          // dA [C][C]
  float* sBnd = sdA + C * C;                     // [D]
  const int tid = threadIdx.x;
  const int L = a.L, NC = (L + C - 1) / C;
  const int bh = blockIdx.x / NC, c = blockIdx.x % NC;
  const int t0 = c * C, tl = min(t0 + C, L) - 1, Cv = tl - t0 + 1;
  const size_t hoff = (size_t)bh * L * D;
  const T* q = reinterpret_cast<const T*>(a.q) + hoff;
  const T* k = reinterpret_cast<const T*>(a.k) + hoff;
  const T* v = reinterpret_cast<const T*>(a.v) + hoff;
  const T* dO = reinterpret_cast<const T*>(a.dO) + hoff;
  const T* S = states + ((size_t)bh * NC + c) * D * D;           // entering chunk c
  const float* dSc = dS + ((size_t)bh * NC + c) * D * D;         // gradient of the state after chunk c
  const Gates G = head_gates(P, Tb, bh, L, Dg);

  for (int e = tid; e < Cv * Cv; e += GTH) {
    const int t = e / Cv, s = e % Cv;
    float x = 0.f, y = 0.f;
    if (s <= t) {
      for (int i = 0; i < D; ++i)
        x += tof(q[(size_t)(t0 + t) * D + i]) * tof(k[(size_t)(t0 + s) * D + i]) * __expf(G.diff(t0 + t, t0 + s, i));
      y = dot_rows(dO + (size_t)(t0 + t) * D, v + (size_t)(t0 + s) * D, D);
    }
    sA[t * C + s] = x;
    sdA[t * C + s] = y;
  }
  for (int i = tid; i < D; i += GTH) {
    float x = 0.f;
    for (int jq = 0; jq < NJ; ++jq) x += bndp[(((size_t)bh * NC + c) * NJ + jq) * D + i];
    sBnd[i] = x;
  }
  __syncthreads();
  // dv, intra-chunk part
  for (int e = tid; e < Cv * D; e += GTH) {
    const int s = e / D, jc = e % D;
    float x = 0.f;
    for (int t = s; t < Cv; ++t) x += sA[t * C + s] * tof(dO[(size_t)(t0 + t) * D + jc]);
    dvg[hoff + (size_t)(t0 + s) * D + jc] = x;
  }
  __syncthreads();
  for (int e = tid; e < Cv * D; e += GTH) {
    const int s = e / D, i = e % D;
    sA[e] = tof(k[(size_t)(t0 + s) * D + i]) * __expf(G.suf(t0 + s, tl, i));
  }
  __syncthreads();
  // dv, inter-chunk part (same thread per element as above: no race)
  for (int e = tid; e < Cv * D; e += GTH) {
    const int s = e / D, jc = e % D;
    float x = 0.f;
    for (int i = 0; i < D; ++i) x += sA[s * D + i] * dSc[(size_t)i * D + jc];
    dvg[hoff + (size_t)(t0 + s) * D + jc] += x;
  }
  __syncthreads();
  // dq; its term of d b
  for (int e = tid; e < Cv * D; e += GTH) {
    const int t = e / D, i = e % D;
    float x = 0.f;
    for (int s = 0; s <= t; ++s) x += sdA[t * C + s] * tof(k[(size_t)(t0 + s) * D + i]) * __expf(G.diff(t0 + t, t0 + s, i));
    float y = 0.f;
    for (int jc = 0; jc < D; ++jc) y += tof(dO[(size_t)(t0 + t) * D + jc]) * tof(S[(size_t)i * D + jc]);
    x += __expf(G.pre(t0 + t, t0, i)) * y;
    dqg[hoff + (size_t)(t0 + t) * D + i] = x;
    sA[e] = tof(q[(size_t)(t0 + t) * D + i]) * x;
  }
  __syncthreads();
  // dk; its term of d b
  for (int e = tid; e < Cv * D; e += GTH) {
    const int s = e / D, i = e % D;
    float x = 0.f;
    for (int t = s; t < Cv; ++t) x += sdA[t * C + s] * tof(q[(size_t)(t0 + t) * D + i]) * __expf(G.diff(t0 + t, t0 + s, i));
    float y = 0.f;
    for (int jc = 0; jc < D; ++jc) y += dSc[(size_t)i * D + jc] * tof(v[(size_t)(t0 + s) * D + jc]);
    x += __expf(G.suf(t0 + s, tl, i)) * y;
    dkg[hoff + (size_t)(t0 + s) * D + i] = x;
    sA[e] -= tof(k[(size_t)(t0 + s) * D + i]) * x;
  }
  __syncthreads();
  // dg: suffix over the chunk's tokens plus the boundary term
  for (int i = tid; i < D; i += GTH) {
    float run = sBnd[i];
    for (int t = Cv - 1; t >= 0; --t) {
      run += sA[t * D + i];
      sA[t * D + i] = run;
    }
  }
  __syncthreads();
  if (Dg == D) {
    for (int e = tid; e < Cv * D; e += GTH) a.dg[hoff + (size_t)(t0 + e / D) * D + e % D] = sA[e];
  } else {
    for (int t = tid; t < Cv; t += GTH) {
      float x = 0.f;
      for (int i = 0; i < D; ++i) x += sA[t * D + i];
      a.dg[(size_t)bh * L + t0 + t] = x;
    }
  }
}

template <typename T, int D>
__global__ __launch_bounds__(GTH) void gen_delta_kernel(const T* __restrict__ dO, const T* __restrict__ o_swa,
                                                        float* __restrict__ delta, float mix, size_t n) {
  const size_t t = (size_t)blockIdx.x * GTH + threadIdx.x;
  if (t < n) delta[t] = mix * dot_rows(dO + t * D, o_swa + t * D, D);
}

// ------------------------------------------------------------------ backward: window gradients
// One workgroup per (b*h, 64-token tile): the tile's tokens as queries (dq) and as keys (dk, dv),
// added to the GLA parts; per-(b, tile) partial sums of the meta-key gradients.
template <typename T, int D>
__global__ __launch_bounds__(GTH) void gen_win_bwd_kernel(BwdArgs a, const float* __restrict__ dqg,
                                                          const float* __restrict__ dkg,
                                                          const float* __restrict__ dvg,
                                                          const float* __restrict__ delta,
                                                          const float* __restrict__ lse, float* __restrict__ part) {
  extern __shared__ __align__(16) unsigned char smem[];
  float* sDQ = reinterpret_cast<float*>(smem);   // [WT][D]
  float* sDK = sDQ + WT * D;
  float* sDV = sDK + WT * D;
  float* sS = sDV + WT * D;                       // [WT][32] P (dP - delta)
  float* sP = sS + WT * 32;                       // [WT][32] P
  const int tid = threadIdx.x;
  const int L = a.L, W = a.W, M = a.M, H = a.H, NT = (L + WT - 1) / WT;
  const int bh = blockIdx.x / NT, tile = blockIdx.x % NT, b = bh / H, h = bh % H;
  const int t0 = tile * WT, Tv = min(WT, L - t0);
  const size_t hoff = (size_t)bh * L * D;
  const T* q = reinterpret_cast<const T*>(a.q) + hoff;
  const T* k = reinterpret_cast<const T*>(a.k) + hoff;
  const T* v = reinterpret_cast<const T*>(a.v) + hoff;
  const T* dO = reinterpret_cast<const T*>(a.dO) + hoff;
  const T* mk = reinterpret_cast<const T*>(a.meta_k) + (size_t)h * M * D;
  const T* mv = a.meta_v ? reinterpret_cast<const T*>(a.meta_v) + (size_t)h * M * D : nullptr;
  const float* ls = lse + (size_t)bh * L;
  const float* dl = delta + (size_t)bh * L;
  const float scale = a.scale, mix = a.mix;
  for (int e = tid; e < Tv * D; e += GTH) {
    const size_t o = hoff + (size_t)t0 * D + e;
    sDQ[e] = dqg[o];
    sDK[e] = dkg[o];
    sDV[e] = dvg[o];
  }
  __syncthreads();
  if (M > 0) {
    for (int e = tid; e < Tv * 32; e += GTH) {
      const int t = e / 32, m = e % 32, tq = t0 + t;
      float ds = 0.f, pr = 0.f;
      if (m < M) {
        pr = __expf(scale * dot_rows(q + (size_t)tq * D, mk + (size_t)m * D, D) - ls[tq]);
        const float dp = mv ? mix * dot_rows(dO + (size_t)tq * D, mv + (size_t)m * D, D) : 0.f;
        ds = pr * (dp - dl[tq]);
      }
      sS[e] = ds;
      sP[e] = pr;
    }
    __syncthreads();
    for (int e = tid; e < Tv * D; e += GTH) {
      const int t = e / D, i = e % D;
      float x = 0.f;
      for (int m = 0; m < M; ++m) x += sS[t * 32 + m] * tof(mk[(size_t)m * D + i]);
      sDQ[e] += scale * x;
    }
    float* pp = part + ((size_t)b * NT + tile) * H * M * 2 * D + (size_t)h * M * 2 * D;
    for (int e = tid; e < M * D; e += GTH) {
      const int m = e / D, i = e % D;
      float xk = 0.f, xv = 0.f;
      for (int t = 0; t < Tv; ++t) {
        xk += sS[t * 32 + m] * tof(q[(size_t)(t0 + t) * D + i]);
        xv += sP[t * 32 + m] * tof(dO[(size_t)(t0 + t) * D + i]);
      }
      pp[(size_t)m * 2 * D + i] = scale * xk;
      pp[(size_t)m * 2 * D + D + i] = mix * xv;
    }
    __syncthreads();
  }
  // the tile's queries against the keys of their windows
  const int tl = t0 + Tv - 1;
  for (int kb = max(t0 - W + 1, 0); kb <= tl; kb += 32) {
    for (int e = tid; e < Tv * 32; e += GTH) {
      const int t = e / 32, s = kb + e % 32, tq = t0 + t;
      float ds = 0.f;
      if (s <= tl && s <= tq && s > tq - W) {
        const float pr = __expf(scale * dot_rows(q + (size_t)tq * D, k + (size_t)s * D, D) - ls[tq]);
        ds = pr * (mix * dot_rows(dO + (size_t)tq * D, v + (size_t)s * D, D) - dl[tq]);
      }
      sS[e] = ds;
    }
    __syncthreads();
    const int nk = min(32, tl - kb + 1);
    for (int e = tid; e < Tv * D; e += GTH) {
      const int t = e / D, i = e % D;
      float x = 0.f;
      for (int u = 0; u < nk; ++u) x += sS[t * 32 + u] * tof(k[(size_t)(kb + u) * D + i]);
      sDQ[e] += scale * x;
    }
    __syncthreads();
  }
  // the tile's keys against the queries whose windows hold them
  const int qmax = min(tl + W - 1, L - 1);
  for (int qb = t0; qb <= qmax; qb += 32) {
    for (int e = tid; e < Tv * 32; e += GTH) {
      const int sl = e / 32, tq = qb + e % 32, s = t0 + sl;
      float ds = 0.f, pr = 0.f;
      if (tq <= qmax && tq >= s && tq < s + W) {
        pr = __expf(scale * dot_rows(q + (size_t)tq * D, k + (size_t)s * D, D) - ls[tq]);
        ds = pr * (mix * dot_rows(dO + (size_t)tq * D, v + (size_t)s * D, D) - dl[tq]);
      }
      sS[e] = ds;
      sP[e] = pr;
    }
    __syncthreads();
    const int nq = min(32, qmax - qb + 1);
    for (int e = tid; e < Tv * D; e += GTH) {
      const int sl = e / D, i = e % D;
      float xk = 0.f, xv = 0.f;
      for (int u = 0; u < nq; ++u) {
        xk += sS[sl * 32 + u] * tof(q[(size_t)(qb + u) * D + i]);
        xv += sP[sl * 32 + u] * tof(dO[(size_t)(qb + u) * D + i]);
      }
      sDK[e] += scale * xk;
      sDV[e] += mix * xv;
    }
    __syncthreads();
  }
  for (int e = tid; e < Tv * D; e += GTH) {
    const size_t o = hoff + (size_t)t0 * D + e;
    put_elem(reinterpret_cast<T*>(a.dq) + o, sDQ[e]);
    put_elem(reinterpret_cast<T*>(a.dk) + o, sDK[e]);
    put_elem(reinterpret_cast<T*>(a.dv) + o, sDV[e]);
  }
}

// Meta-key gradients: the per-(b, tile) partials summed in index order (bit-reproducible).
__global__ __launch_bounds__(GTH) void gen_meta_fold_kernel(const float* __restrict__ part, float* __restrict__ dmk,
                                                            float* __restrict__ dmv, int slots, int n, int D) {
  const int e = blockIdx.x * GTH + threadIdx.x;   // over H*M*2D
  if (e >= n) return;
  float acc = 0.f;
  for (int s = 0; s < slots; ++s) acc += part[(size_t)s * n + e];
  const int hm = e / (2 * D), col = e % (2 * D);
  if (col < D)
    dmk[(size_t)hm * D + col] = acc;
  else if (dmv != nullptr)
    dmv[(size_t)hm * D + col - D] = acc;
}

// ------------------------------------------------------------------ workspace layouts
struct GenFwdWs { size_t P, Tb, states, total; };
GenFwdWs gen_fwd_ws(int B, int H, int L, int D, int C, int dtype) {
  const size_t BH = (size_t)B * H, NB = (L + 15) / 16, NC = (L + C - 1) / C;
  const size_t esz = dtype == 1 ? 2 : 4;
  GenFwdWs w{};
  w.P = 0;
  w.Tb = rup(4 * BH * L * D);
  w.states = w.Tb + rup(4 * BH * NB * D);
  w.total = w.states + rup(esz * BH * NC * D * D);
  return w;
}

struct GenBwdWs { size_t P, Tb, dS, bnd, dq, dk, dv, delta, part, rc_lse, rc_oswa, rc_states, total, rc_total; };
GenBwdWs gen_bwd_ws(int B, int H, int L, int M, int D, int C, int dtype) {
  const size_t BH = (size_t)B * H, NB = (L + 15) / 16, NC = (L + C - 1) / C, NT = (L + WT - 1) / WT;
  const size_t esz = dtype == 1 ? 2 : 4;
  GenBwdWs w{};
  size_t off = 0;
  w.P = off; off += rup(4 * BH * L * D);
  w.Tb = off; off += rup(4 * BH * NB * D);
  w.dS = off; off += rup(4 * BH * NC * D * D);
  w.bnd = off; off += rup(4 * BH * NC * (D / JS) * D);
  w.dq = off; off += rup(4 * BH * L * D);
  w.dk = off; off += rup(4 * BH * L * D);
  w.dv = off; off += rup(4 * BH * L * D);
  w.delta = off; off += rup(4 * BH * L);
  w.part = off; off += rup(4 * (size_t)B * NT * H * M * 2 * D);
  w.total = off;
  w.rc_lse = off; off += rup(4 * BH * L);
  w.rc_oswa = off; off += rup(esz * BH * L * D);
  w.rc_states = off; off += rup(esz * BH * NC * D * D);
  w.rc_total = off;
  return w;
}

template <typename T, int D>
hipError_t launch_prefix_and_fwd(const FwdArgs& a, int C, float* P, float* Tb, T* states, hipStream_t st) {
  hipError_t e;
  const int BH = a.B * a.H, NB = (a.L + 15) / 16, NC = (a.L + C - 1) / C;
  const int Dg = a.gate ? 1 : D;
  hipLaunchKernelGGL(gen_prefix_kernel, dim3(BH * NB), dim3(128), 0, st, a.g, P, Tb, a.L, Dg);
  const size_t lds1 = sizeof(float) * ((size_t)C * D + (size_t)C * JS + D);
  if ((e = lds_attr(gen_state_kernel<T, D>, lds1)) != hipSuccess) return e;
  hipLaunchKernelGGL((gen_state_kernel<T, D>), dim3(BH * (D / JS)), dim3(GTH), lds1, st,
                     reinterpret_cast<const T*>(a.k), reinterpret_cast<const T*>(a.v), (const float*)P,
                     (const float*)Tb, states, a.state_out, a.L, C, Dg);
  const size_t lds2 = sizeof(float) * ((size_t)std::max(C * C, C * D) + (size_t)C * D + (size_t)C * 32 + 2 * C);
  if ((e = lds_attr(gen_out_kernel<T, D>, lds2)) != hipSuccess) return e;
  hipLaunchKernelGGL((gen_out_kernel<T, D>), dim3(BH * NC), dim3(GTH), lds2, st, a, (const T*)states,
                     (const float*)P, (const float*)Tb, C, Dg);
  return hipGetLastError();
}

template <typename T, int D>
hipError_t launch_fwd_general_t(const FwdArgs& a, int C, hipStream_t st) {
  if (a.L == 0) {
    if (a.state_out != nullptr) {
      const size_t n = (size_t)a.B * a.H * D * D;
      hipLaunchKernelGGL(gen_zero_kernel, dim3((n + 255) / 256), dim3(256), 0, st, a.state_out, n);
    }
    return hipGetLastError();
  }
  const GenFwdWs w = gen_fwd_ws(a.B, a.H, a.L, D, C, std::is_same<T, bf16_t>::value ? 1 : 0);
  unsigned char* ws = reinterpret_cast<unsigned char*>(a.workspace);
  T* states = a.chunk_states != nullptr ? reinterpret_cast<T*>(a.chunk_states) : reinterpret_cast<T*>(ws + w.states);
  return launch_prefix_and_fwd<T, D>(a, C, reinterpret_cast<float*>(ws + w.P), reinterpret_cast<float*>(ws + w.Tb),
                                     states, st);
}

template <typename T, int D>
hipError_t launch_bwd_general_t(const BwdArgs& a0, int C, hipStream_t st) {
  hipError_t e;
  BwdArgs a = a0;
  const int BH = a.B * a.H, L = a.L, M = a.M;
  if (L == 0) {
    if (M > 0) {
      const size_t n = (size_t)a.H * M * D;
      hipLaunchKernelGGL(gen_zero_kernel, dim3((n + 255) / 256), dim3(256), 0, st, a.dmeta_k, n);
      if (a.dmeta_v) hipLaunchKernelGGL(gen_zero_kernel, dim3((n + 255) / 256), dim3(256), 0, st, a.dmeta_v, n);
    }
    return hipGetLastError();
  }
  const int dtype = std::is_same<T, bf16_t>::value ? 1 : 0;
  const GenBwdWs w = gen_bwd_ws(a.B, a.H, L, M, D, C, dtype);
  unsigned char* ws = reinterpret_cast<unsigned char*>(a.workspace);
  float* P = reinterpret_cast<float*>(ws + w.P);
  float* Tb = reinterpret_cast<float*>(ws + w.Tb);
  const int NC = (L + C - 1) / C, NT = (L + WT - 1) / WT, NB = (L + 15) / 16;
  const int Dg = a.gate ? 1 : D;
  const T* states = reinterpret_cast<const T*>(a.chunk_states);
  if (a.lse == nullptr || a.o_swa == nullptr || a.chunk_states == nullptr) {
    // recompute lse, o_swa and the chunk states (the forward also forms the gate block sums)
    FwdArgs f{};
    f.q = a.q; f.k = a.k; f.v = a.v; f.g = a.g; f.meta_k = a.meta_k; f.meta_v = a.meta_v;
    f.o = nullptr;
    f.lse = reinterpret_cast<float*>(ws + w.rc_lse);
    f.o_swa = ws + w.rc_oswa;
    f.B = a.B; f.H = a.H; f.L = L; f.W = a.W; f.M = M; f.scale = a.scale; f.mix = a.mix; f.gate = a.gate;
    T* rs = reinterpret_cast<T*>(ws + w.rc_states);
    if ((e = launch_prefix_and_fwd<T, D>(f, C, P, Tb, rs, st)) != hipSuccess) return e;
    a.lse = f.lse;
    a.o_swa = f.o_swa;
    states = rs;
  } else {
    hipLaunchKernelGGL(gen_prefix_kernel, dim3(BH * NB), dim3(128), 0, st, a.g, P, Tb, L, Dg);
  }
  float* dS = reinterpret_cast<float*>(ws + w.dS);
  float* bnd = reinterpret_cast<float*>(ws + w.bnd);
  float* dqg = reinterpret_cast<float*>(ws + w.dq);
  float* dkg = reinterpret_cast<float*>(ws + w.dk);
  float* dvg = reinterpret_cast<float*>(ws + w.dv);
  float* delta = reinterpret_cast<float*>(ws + w.delta);
  float* part = reinterpret_cast<float*>(ws + w.part);
  const size_t lds3 = sizeof(float) * ((size_t)C * D + (size_t)C * JS + D);
  if ((e = lds_attr(gen_dstate_kernel<T, D>, lds3)) != hipSuccess) return e;
  hipLaunchKernelGGL((gen_dstate_kernel<T, D>), dim3(BH * (D / JS)), dim3(GTH), lds3, st,
                     reinterpret_cast<const T*>(a.q), reinterpret_cast<const T*>(a.dO), states, (const float*)P,
                     (const float*)Tb, dS, bnd, L, C, Dg);
  const size_t lds4 = sizeof(float) * ((size_t)std::max(C * C, C * D) + (size_t)C * C + D);
  if ((e = lds_attr(gen_gla_bwd_kernel<T, D>, lds4)) != hipSuccess) return e;
  hipLaunchKernelGGL((gen_gla_bwd_kernel<T, D>), dim3(BH * NC), dim3(GTH), lds4, st, a, states, (const float*)dS,
                     (const float*)bnd, (const float*)P, (const float*)Tb, dqg, dkg, dvg, C, Dg);
  const size_t ntok = (size_t)BH * L;
  hipLaunchKernelGGL((gen_delta_kernel<T, D>), dim3((unsigned)((ntok + GTH - 1) / GTH)), dim3(GTH), 0, st,
                     reinterpret_cast<const T*>(a.dO), reinterpret_cast<const T*>(a.o_swa), delta, a.mix, ntok);
  const size_t lds5 = sizeof(float) * (3 * (size_t)WT * D + 2 * (size_t)WT * 32);
  if ((e = lds_attr(gen_win_bwd_kernel<T, D>, lds5)) != hipSuccess) return e;
  hipLaunchKernelGGL((gen_win_bwd_kernel<T, D>), dim3(BH * NT), dim3(GTH), lds5, st, a, (const float*)dqg,
                     (const float*)dkg, (const float*)dvg, (const float*)delta, a.lse, part);
  if (M > 0) {
    const int n = a.H * M * 2 * D;
    hipLaunchKernelGGL(gen_meta_fold_kernel, dim3((n + GTH - 1) / GTH), dim3(GTH), 0, st, (const float*)part,
                       a.dmeta_k, a.dmeta_v, a.B * NT, n, D);
  }
  return hipGetLastError();
}

}  // namespace

size_t fwd_general_workspace_bytes(int B, int H, int L, int D, int C, int dtype, bool states_given) {
  if (L == 0) return 0;
  const GenFwdWs w = gen_fwd_ws(B, H, L, D, C, dtype);
  return states_given ? w.states : w.total;
}

size_t bwd_general_workspace_bytes(int B, int H, int L, int M, int D, int C, int dtype, bool recompute) {
  if (L == 0) return 0;
  const GenBwdWs w = gen_bwd_ws(B, H, L, M, D, C, dtype);
  return recompute ? w.rc_total : w.total;
}

hipError_t launch_fwd_general(const FwdArgs& a, int dtype, int D, int C, hipStream_t st) {
  if (dtype == 1) {
    if (D == 128) return launch_fwd_general_t<bf16_t, 128>(a, C, st);
    if (D == 64) return launch_fwd_general_t<bf16_t, 64>(a, C, st);
  } else {
    if (D == 128) return launch_fwd_general_t<float, 128>(a, C, st);
    if (D == 64) return launch_fwd_general_t<float, 64>(a, C, st);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_bwd_general(const BwdArgs& a, int dtype, int D, int C, hipStream_t st) {
  if (dtype == 1) {
    if (D == 128) return launch_bwd_general_t<bf16_t, 128>(a, C, st);
    if (D == 64) return launch_bwd_general_t<bf16_t, 64>(a, C, st);
  } else {
    if (D == 128) return launch_bwd_general_t<float, 128>(a, C, st);
    if (D == 64) return launch_bwd_general_t<float, 64>(a, C, st);
  }
  return hipErrorInvalidValue;
}

}  // namespace lz
