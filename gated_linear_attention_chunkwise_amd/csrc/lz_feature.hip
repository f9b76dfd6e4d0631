// lz_feature.hip -- the Hedgehog feature map of the GLA branch, in log space, on gfx950.
//
// The GLA branch keeps its state from feature-mapped keys and reads it with
// feature-mapped queries (gist.science explainer of "Lizard: An Efficient
// Linearization Framework for Large Language Models", English page §2.A,
// state update); the pages name the map a Hedgehog feature map and use its
// non-negativity to absorb the cumulative gate in log space (Chinese page
// §2.3; English page §2.C).  With the two-sided softmax form of the map,
//
//   log phi(x) = [ z - lse(z),  -z - lse(-z) ],   z = x W_h,  W_h [d, d/2]
//
// hedgehog_fwd_kernel writes these log features (fp32) for the layer's
// log-feature entry points, which add the gate prefix before exponentiating.
// One workgroup of four waves per (batch, head, 64 tokens); W_h is staged in
// LDS once per workgroup, x is read as matrix-core operands straight from
// global memory, and z is formed transposed so a lane holds four consecutive
// features of one token: both log-sum-exps are an in-lane pass plus two
// cross-lane steps.
//
// hedgehog_bwd_kernel, from dl = dL/dlog phi:
//   dz = (g+ - p+ sum g+) - (g- - p- sum g-),  p+- = softmax(+-z), g+- the halves of dl
//   dx = dz W_h^T        (dz fed from the accumulators as the matrix-core operand)
//   dW_h = sum_t x_t^T dz_t  over a group of chunks per workgroup, in registers; the
//   groups' partial sums are added in a fixed order by feature_dw_sum_kernel.
#include "lz_common.hpp"
#include "lz_kernels.hpp"

namespace lz {
namespace {

constexpr int NTHR_FM = 256;

template <typename T, int D>
struct FmLayout {
  static constexpr int F = D / 2;
  static constexpr int LDW = F + Tr<T>::PAD;   // W_h [D][F]
  static constexpr int LDX = D + Tr<T>::PAD;   // x chunk [C][D]
  static constexpr int LDZ = F + Tr<T>::PAD;   // dz chunk [C][F]
  static constexpr size_t oW = 0;
  static constexpr size_t oX = oW + sizeof(T) * D * LDW;
  static constexpr size_t oZ = oX + sizeof(T) * CHUNK * LDX;
  static constexpr size_t bytes = oZ + sizeof(T) * CHUNK * LDZ;
};

// W_h [D][F] row-major to LDS
template <typename T, int D>
__device__ __forceinline__ void stage_w(T* sW, const T* w, int tid) {
  using LY = FmLayout<T, D>;
  constexpr int F = LY::F, VEC = Tr<T>::VEC;
  for (int idx = tid; idx < D * F / VEC; idx += NTHR_FM) {
    const int row = idx / (F / VEC), cv = idx % (F / VEC);
    *reinterpret_cast<V16*>(sW + row * LY::LDW + cv * VEC) = ldg16(w + (size_t)row * F + cv * VEC);
  }
}

// z for this wave's 16 tokens, transposed: z[j] lane (r, kg) = z[token r][16 j + 4 kg + e].
// A operand fragments come from `xsrc` rows (global or LDS through ldx).
template <typename T, int D>
__device__ __forceinline__ void form_z(f32x4 (&z)[D / 32], const typename Tr<T>::frag (&xf)[D / 32], const T* sW,
                                       int lane) {
  using LY = FmLayout<T, D>;
  constexpr int NB = LY::F / 16, KS = D / 32;
  const int kg = lane >> 4;
#pragma unroll
  for (int j = 0; j < NB; ++j) z[j] = f32x4{0, 0, 0, 0};
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    const int kk = 32 * ks + 8 * kg;
#pragma unroll
    for (int j = 0; j < NB; ++j) mma32(z[j], ld_frag_tr(sW, LY::LDW, kk, kk + 4, 16 * j, lane), xf[ks]);
  }
}

// log-sum-exp over the F features of this lane's token (sign s = +1 or -1 applied to z)
template <int NB>
__device__ __forceinline__ float lse_row(const f32x4 (&z)[NB], float s) {
  float m = -INFINITY;
#pragma unroll
  for (int j = 0; j < NB; ++j)
#pragma unroll
    for (int e = 0; e < 4; ++e) m = fmaxf(m, s * z[j][e]);
  m = xor_max(xor_max(m, 16), 32);
  float l = 0.f;
#pragma unroll
  for (int j = 0; j < NB; ++j)
#pragma unroll
    for (int e = 0; e < 4; ++e) l += __expf(s * z[j][e] - m);
  l = xor_sum(xor_sum(l, 16), 32);
  return m + __logf(l);
}

// workgroup -> (b*h, chunk); the chunks of one head share an XCD
__device__ __forceinline__ void fm_map(int bid, int BH, int NC, int& bh, int& c) {
  if ((BH & 7) == 0) {
    const int x = bid % 8, y = bid / 8;
    c = y % NC;
    bh = (y / NC) * 8 + x;
  } else {
    bh = bid / NC;
    c = bid % NC;
  }
}

template <typename T, int D>
__global__ __launch_bounds__(NTHR_FM) void hedgehog_fwd_kernel(FeatArgs a) {
  using LY = FmLayout<T, D>;
  using frag = typename Tr<T>::frag;
  constexpr int F = LY::F, NB = F / 16, KS = D / 32;
  extern __shared__ __align__(16) unsigned char smem[];
  T* sW = reinterpret_cast<T*>(smem + LY::oW);
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, r = lane & 15, kg = lane >> 4;
  const int L = a.L, NC = (L + CHUNK - 1) / CHUNK;
  int bh, c;
  fm_map(blockIdx.x, a.B * a.H, NC, bh, c);
  const int h = bh % a.H;
  const T* x = reinterpret_cast<const T*>(a.x) + (size_t)bh * L * D;
  const int tok = c * CHUNK + 16 * w + r;
  frag xf[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) xf[ks] = ldg_row_frag<T>(x, D, tok, 32 * ks + 8 * kg, L);
  stage_w<T, D>(sW, reinterpret_cast<const T*>(a.w) + (size_t)h * D * F, tid);
  __syncthreads();
  f32x4 z[NB];
  form_z<T, D>(z, xf, sW, lane);
  const float lp = lse_row<NB>(z, 1.f), lm = lse_row<NB>(z, -1.f);
  if (tok < L) {
    float* out = a.lphi + ((size_t)bh * L + tok) * D;
#pragma unroll
    for (int j = 0; j < NB; ++j) {
      const int f = 16 * j + 4 * kg;
      *reinterpret_cast<f32x4*>(out + f) = f32x4{z[j][0] - lp, z[j][1] - lp, z[j][2] - lp, z[j][3] - lp};
      *reinterpret_cast<f32x4*>(out + F + f) =
          f32x4{-z[j][0] - lm, -z[j][1] - lm, -z[j][2] - lm, -z[j][3] - lm};
    }
  }
}

// One workgroup per (head, group of `a.cpg` consecutive (batch, chunk) slots); three per CU,
// as many as the LDS allows (the registers are held to 168).
template <typename T, int D>
__global__ __launch_bounds__(NTHR_FM, 3) void hedgehog_bwd_kernel(FeatArgs a) {
  using LY = FmLayout<T, D>;
  using frag = typename Tr<T>::frag;
  constexpr int F = LY::F, NB = F / 16, KS = D / 32, VEC = Tr<T>::VEC;
  constexpr int JD = D / 16;                      // 16-wide blocks of d (dx columns)
  extern __shared__ __align__(16) unsigned char smem[];
  T* sW = reinterpret_cast<T*>(smem + LY::oW);
  T* sX = reinterpret_cast<T*>(smem + LY::oX);
  T* sZ = reinterpret_cast<T*>(smem + LY::oZ);
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, r = lane & 15, kg = lane >> 4;
  const int L = a.L, NC = (L + CHUNK - 1) / CHUNK, slots = a.B * NC;
  const int h = blockIdx.x % a.H, grp = blockIdx.x / a.H;
  const int s_begin = grp * a.cpg, s_end = min(slots, s_begin + a.cpg);
  stage_w<T, D>(sW, reinterpret_cast<const T*>(a.w) + (size_t)h * D * F, tid);

  // dW_h partial: wave w owns rows d = (D/4) w .. +D/4 over all F features
  constexpr int DR = D / 4, IB = DR / 16;
  f32x4 dw[IB][NB];
#pragma unroll
  for (int i = 0; i < IB; ++i)
#pragma unroll
    for (int j = 0; j < NB; ++j) dw[i][j] = f32x4{0, 0, 0, 0};

  // The next chunk's x tile and dl rows are loaded (unconditionally, rows clamped into the
  // sequence) while the current chunk is processed, and masked when they are taken.
  constexpr int NXV = CHUNK * D / VEC / NTHR_FM;   // 16-byte vectors of the x tile per thread
  static_assert(CHUNK * D / VEC % NTHR_FM == 0, "x tile splits evenly over the threads");
  const int u = 16 * w + r;
  V16 xn[NXV];
  f32x4 gpn[NB], gmn[NB];
  auto fetch_x = [&](int sl) {
    const int b = sl / NC, c = sl % NC, bh = b * a.H + h, t0 = c * CHUNK;
    const T* x = reinterpret_cast<const T*>(a.x) + (size_t)bh * L * D;
#pragma unroll
    for (int i = 0; i < NXV; ++i) {
      const int idx = tid + i * NTHR_FM, row = idx / (D / VEC), cv = idx % (D / VEC);
      xn[i] = ldg16(x + (size_t)min(t0 + row, L - 1) * D + cv * VEC);
    }
  };
  auto fetch_dl = [&](int sl) {
    const int b = sl / NC, c = sl % NC, bh = b * a.H + h, t0 = c * CHUNK;
    const float* dlr = a.dl + ((size_t)bh * L + min(t0 + u, L - 1)) * D;
#pragma unroll
    for (int j = 0; j < NB; ++j) {
      gpn[j] = *reinterpret_cast<const f32x4*>(dlr + 16 * j + 4 * kg);
      gmn[j] = *reinterpret_cast<const f32x4*>(dlr + F + 16 * j + 4 * kg);
    }
  };
  if (s_begin < s_end) {
    fetch_x(s_begin);
    fetch_dl(s_begin);
  }
  for (int sl = s_begin; sl < s_end; ++sl) {
    const int b = sl / NC, c = sl % NC, bh = b * a.H + h, t0 = c * CHUNK;
    const int tok = t0 + u;
    const bool ok = tok < L;
    __syncthreads();   // the previous chunk's readers of sX / sZ are done (and W is staged)
    // x chunk to LDS (rows past the end as zeros: they add nothing to dW), then the next x
#pragma unroll
    for (int i = 0; i < NXV; ++i) {
      const int idx = tid + i * NTHR_FM, row = idx / (D / VEC), cv = idx % (D / VEC);
      *reinterpret_cast<V16*>(sX + row * LY::LDX + cv * VEC) = t0 + row < L ? xn[i] : zero16();
    }
    fetch_x(min(sl + 1, s_end - 1));
    __syncthreads();
    frag xf[KS];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) xf[ks] = ld_frag(sX, LY::LDX, u, 32 * ks + 8 * kg);
    f32x4 z[NB];
    form_z<T, D>(z, xf, sW, lane);
    const float lp = lse_row<NB>(z, 1.f), lm = lse_row<NB>(z, -1.f);
    // dz in the same lane layout
    // this lane's dl (a token past the end: zero), then the next chunk's
    f32x4 gp[NB], gm[NB];
    float sp = 0.f, sm = 0.f;
#pragma unroll
    for (int j = 0; j < NB; ++j) {
      gp[j] = ok ? gpn[j] : f32x4{0, 0, 0, 0};
      gm[j] = ok ? gmn[j] : f32x4{0, 0, 0, 0};
#pragma unroll
      for (int e = 0; e < 4; ++e) { sp += gp[j][e]; sm += gm[j][e]; }
    }
    sp = xor_sum(xor_sum(sp, 16), 32);
    sm = xor_sum(xor_sum(sm, 16), 32);
    f32x4 dz[NB];
#pragma unroll
    for (int j = 0; j < NB; ++j)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float pp = __expf(z[j][e] - lp), pm = __expf(-z[j][e] - lm);
        dz[j][e] = (gp[j][e] - pp * sp) - (gm[j][e] - pm * sm);
      }
    fetch_dl(min(sl + 1, s_end - 1));
    // dz chunk to LDS for the dW product (token rows, feature columns)
#pragma unroll
    for (int j = 0; j < NB; ++j) st4(sZ + u * LY::LDZ + 16 * j + 4 * kg, dz[j][0], dz[j][1], dz[j][2], dz[j][3]);
    // dx = dz W^T: blocks transposed (d rows, token columns), dz fed from the accumulators
    f32x4 dx[JD];
#pragma unroll
    for (int jd = 0; jd < JD; ++jd) dx[jd] = f32x4{0, 0, 0, 0};
#pragma unroll
    for (int p = 0; p < NB / 2; ++p) {
      frag op;
      pack_acc(op, dz[2 * p], dz[2 * p + 1]);
#pragma unroll
      for (int jd = 0; jd < JD; ++jd)
        mma32(dx[jd], ld_frag_perm(sW, LY::LDW, 16 * jd + r, 2 * p, 2 * p + 1, kg), op);
    }
    if (ok) {
      T* dxr = reinterpret_cast<T*>(a.dx) + ((size_t)bh * L + tok) * D;
#pragma unroll
      for (int jd = 0; jd < JD; ++jd) stg4(dxr + 16 * jd + 4 * kg, dx[jd][0], dx[jd][1], dx[jd][2], dx[jd][3]);
    }
    __syncthreads();   // dz of every wave in LDS
    // dW_h[d][f] += sum over the chunk's tokens of x[t][d] dz[t][f]
#pragma unroll
    for (int ks = 0; ks < CHUNK / 32; ++ks) {
      const int kk = 32 * ks + 8 * kg;
      frag fz[NB];
#pragma unroll
      for (int j = 0; j < NB; ++j) fz[j] = ld_frag_tr(sZ, LY::LDZ, kk, kk + 4, 16 * j, lane);
#pragma unroll
      for (int i = 0; i < IB; ++i) {
        const frag fx = ld_frag_tr(sX, LY::LDX, kk, kk + 4, DR * w + 16 * i, lane);
#pragma unroll
        for (int j = 0; j < NB; ++j) mma32(dw[i][j], fx, fz[j]);
      }
    }
  }
  // partial dW_h of this group: lane holds dW[d = DR w + 16 i + 4 kg + e][f = 16 j + r]
  float* out = a.dw_part + ((size_t)grp * a.H + h) * D * F;
#pragma unroll
  for (int i = 0; i < IB; ++i)
#pragma unroll
    for (int j = 0; j < NB; ++j)
#pragma unroll
      for (int e = 0; e < 4; ++e) out[(size_t)(DR * w + 16 * i + 4 * kg + e) * F + 16 * j + r] = dw[i][j][e];
}

// dW = sum over the groups, in group order
__global__ __launch_bounds__(256) void feature_dw_sum_kernel(const float* __restrict__ part, float* __restrict__ dw,
                                                             size_t n, int groups) {
  const size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n) return;
  float s = 0.f;
  for (int gi = 0; gi < groups; ++gi) s += part[(size_t)gi * n + i];
  dw[i] = s;
}

void feature_groups(int B, int H, int L, int& cpg, int& groups) {
  const int slots = B * ((L + CHUNK - 1) / CHUNK);
  int want = (1024 + H - 1) / H;                 // ~1024 workgroups
  want = want < 1 ? 1 : (want > slots ? slots : want);
  cpg = (slots + want - 1) / want;
  groups = slots > 0 ? (slots + cpg - 1) / cpg : 0;
}

template <typename T, int D>
hipError_t feat_fwd_t(const FeatArgs& a, hipStream_t st) {
  const int NC = (a.L + CHUNK - 1) / CHUNK;
  constexpr size_t lds = FmLayout<T, D>::bytes;
  hipLaunchKernelGGL((hedgehog_fwd_kernel<T, D>), dim3(a.B * a.H * NC), dim3(NTHR_FM), lds, st, a);
  return hipGetLastError();
}

template <typename T, int D>
hipError_t feat_bwd_t(const FeatArgs& a0, hipStream_t st) {
  FeatArgs a = a0;
  int groups;
  feature_groups(a.B, a.H, a.L, a.cpg, groups);
  a.dw_part = reinterpret_cast<float*>(a.workspace);
  constexpr size_t lds = FmLayout<T, D>::bytes;
  hipLaunchKernelGGL((hedgehog_bwd_kernel<T, D>), dim3(a.H * groups), dim3(NTHR_FM), lds, st, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const size_t n = (size_t)a.H * D * (D / 2);
  hipLaunchKernelGGL(feature_dw_sum_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st,
                     (const float*)a.dw_part, a.dw, n, groups);
  return hipGetLastError();
}

}  // namespace

size_t feature_workspace_bytes(int B, int H, int L, int D) {
  int cpg, groups;
  feature_groups(B, H, L, cpg, groups);
  return (size_t)groups * H * D * (D / 2) * sizeof(float);
}

hipError_t launch_feature_fwd(const FeatArgs& a, int dtype, int D, hipStream_t st) {
  if (dtype == 1) return D == 64 ? feat_fwd_t<bf16_t, 64>(a, st) : feat_fwd_t<bf16_t, 128>(a, st);
  return feat_fwd_t<float, 64>(a, st);
}

hipError_t launch_feature_bwd(const FeatArgs& a, int dtype, int D, hipStream_t st) {
  if (a.L == 0) {   // no tokens: dW = 0
    const size_t n = (size_t)a.H * D * (D / 2);
    hipLaunchKernelGGL(feature_dw_sum_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st,
                       (const float*)nullptr, a.dw, n, 0);
    return hipGetLastError();
  }
  if (dtype == 1) return D == 64 ? feat_bwd_t<bf16_t, 64>(a, st) : feat_bwd_t<bf16_t, 128>(a, st);
  return feat_bwd_t<float, 64>(a, st);
}

}  // namespace lz
