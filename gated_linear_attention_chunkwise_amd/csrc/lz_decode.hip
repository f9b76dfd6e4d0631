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
// One workgroup per (b, h, d_v slice of 64): it streams its fp32 state slice
// from HBM, applies S <- diag(exp g) S + k^T v, reduces o_gla = q S over d_k
// across the workgroup, attends over the M meta keys plus the filled ring
// slots (the slot of the new token is read from the inputs, so no workgroup
// ever reads a ring entry that another one writes), and stores its slice of
// the new key/value.  pos is advanced by a second one-wave kernel so that
// every workgroup of a sequence reads the same pos.
#include "lz_common.hpp"
#include "lz_kernels.hpp"

namespace lz {
namespace {

constexpr int NTHR = 256;

template <typename T, int D, int DVT>
__global__ __launch_bounds__(NTHR) void decode_kernel(DecodeArgs a) {
  constexpr int NJ = D / DVT;
  constexpr int VEC = Tr<T>::VEC;
  constexpr int F4R = DVT / 4;                // float4 per state-slice row
  constexpr int NS = D * F4R / NTHR;          // float4 per thread
  static_assert(D * F4R % NTHR == 0, "state slice map");
  constexpr int NG = NTHR / DVT;              // key groups for the value reduction

  extern __shared__ __align__(16) float dsm[];
  __shared__ float sq[D], sk[D], sa[D], sv[D];
  __shared__ float sred[NTHR / 64][DVT];
  __shared__ float sw[NG][DVT];
  __shared__ float sstat[2][NTHR / 64];

  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int bid = blockIdx.x;
  const int jt = bid % NJ;
  const int bh = bid / NJ;
  const int b = bh / a.H, h = bh % a.H;
  const int j0 = jt * DVT;
  const int W = a.W, M = a.M;
  const int pos = a.pos[b];
  const int slot = pos % W;
  const int n = min(pos + 1, W);
  const size_t vo = (size_t)bh * D;

  const T* qg = reinterpret_cast<const T*>(a.q) + vo;
  const T* kg = reinterpret_cast<const T*>(a.k) + vo;
  const T* vg = reinterpret_cast<const T*>(a.v) + vo;
  for (int i = tid; i < D; i += NTHR) {
    sq[i] = Tr<T>::to_f(qg[i]);
    sk[i] = Tr<T>::to_f(kg[i]);
    sv[i] = Tr<T>::to_f(vg[i]);
    sa[i] = __expf(a.g[vo + i]);
  }
  __syncthreads();

  // ---- GLA: state slice update and partial q.S over this thread's rows
  float* S = a.state + (size_t)bh * D * D + j0;
  f32x4 part = f32x4{0, 0, 0, 0};
  const int c4 = tid % F4R;
  {
    f32x4 st[NS];
#pragma unroll
    for (int u = 0; u < NS; ++u) {
      const int i = (tid + u * NTHR) / F4R;
      st[u] = *reinterpret_cast<const f32x4*>(S + (size_t)i * D + 4 * c4);
    }
#pragma unroll
    for (int u = 0; u < NS; ++u) {
      const int i = (tid + u * NTHR) / F4R;
      const float ai = sa[i], ki = sk[i], qi = sq[i];
      f32x4 x = st[u];
#pragma unroll
      for (int e = 0; e < 4; ++e) x[e] = ai * x[e] + ki * sv[j0 + 4 * c4 + e];
      *reinterpret_cast<f32x4*>(S + (size_t)i * D + 4 * c4) = x;
      part += qi * x;
    }
  }
  // threads sharing c4 within a wave differ in bits above log2(F4R)
#pragma unroll
  for (int m = F4R; m < 64; m <<= 1)
#pragma unroll
    for (int e = 0; e < 4; ++e) part[e] = xor_sum(part[e], m);
  if (lane < F4R)
#pragma unroll
    for (int e = 0; e < 4; ++e) sred[wv][4 * lane + e] = part[e];

  // ---- window logits over meta keys and the filled ring slots
  float* slog = dsm;                          // [M + W]
  const T* rk = reinterpret_cast<const T*>(a.ring_k) + (size_t)bh * W * D;
  const T* rv = reinterpret_cast<const T*>(a.ring_v) + (size_t)bh * W * D;
  const T* mk = reinterpret_cast<const T*>(a.meta_k) + (size_t)h * M * D;
  const float sl2 = a.scale * LOG2E;
  float lmax = -INFINITY;
  for (int e = tid; e < M + n; e += NTHR) {
    float acc = 0.f;
    if (e < M || e - M == slot) {
      if (e < M) {
        const T* kr = mk + (size_t)e * D;
        for (int d = 0; d < D; d += VEC) {
          const V16 x = ldg16(kr + d);
#pragma unroll
          for (int i = 0; i < VEC; ++i) acc += sq[d + i] * v16_get(x, i, (T*)nullptr);
        }
      } else {
        for (int d = 0; d < D; ++d) acc += sq[d] * sk[d];
      }
    } else {
      const T* kr = rk + (size_t)(e - M) * D;
      for (int d = 0; d < D; d += VEC) {
        const V16 x = ldg16(kr + d);
#pragma unroll
        for (int i = 0; i < VEC; ++i) acc += sq[d + i] * v16_get(x, i, (T*)nullptr);
      }
    }
    acc *= sl2;
    slog[e] = acc;
    lmax = fmaxf(lmax, acc);
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

  // ---- o_swa slice: sum_p p * value, keys split over NG groups
  {
    const int jj = tid % DVT, grp = tid / DVT;
    float acc = 0.f;
    for (int s = grp; s < n; s += NG) {
      const float vs = (s == slot) ? sv[j0 + jj] : Tr<T>::to_f(rv[(size_t)s * D + j0 + jj]);
      acc += slog[M + s] * vs;
    }
    if (a.meta_v != nullptr && grp == 0) {
      const T* mv = reinterpret_cast<const T*>(a.meta_v) + (size_t)h * M * D;
      for (int m = 0; m < M; ++m) acc += slog[m] * Tr<T>::to_f(mv[(size_t)m * D + j0 + jj]);
    }
    sw[grp][jj] = acc;
  }
  __syncthreads();
  if (tid < DVT) {
    float osw = 0.f, og = 0.f;
#pragma unroll
    for (int g2 = 0; g2 < NG; ++g2) osw += sw[g2][tid];
#pragma unroll
    for (int w2 = 0; w2 < NTHR / 64; ++w2) og += sred[w2][tid];
    T* o = reinterpret_cast<T*>(a.o) + vo + j0 + tid;
    *o = Tr<T>::from_f(og + a.mix * osw / l);
  }
  // ---- ring: this workgroup's slice of the new key and value
  {
    T* rkw = reinterpret_cast<T*>(a.ring_k) + ((size_t)bh * W + slot) * D;
    T* rvw = reinterpret_cast<T*>(a.ring_v) + ((size_t)bh * W + slot) * D;
    for (int d = jt * (D / NJ) + tid; d < (jt + 1) * (D / NJ); d += NTHR) rkw[d] = kg[d];
    for (int d = j0 + tid; d < j0 + DVT; d += NTHR) rvw[d] = vg[d];
  }
}

__global__ void pos_advance_kernel(int32_t* pos, int B) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < B) pos[i] += 1;
}

template <typename T, int D>
hipError_t launch_decode_t(const DecodeArgs& a, hipStream_t st) {
  constexpr int DVT = 64;
  const int grid = a.B * a.H * (D / DVT);
  const size_t lds = sizeof(float) * (size_t)(a.M + a.W);
  hipLaunchKernelGGL((decode_kernel<T, D, DVT>), dim3(grid), dim3(NTHR), lds, st, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(pos_advance_kernel, dim3((a.B + 255) / 256), dim3(256), 0, st, a.pos, a.B);
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
