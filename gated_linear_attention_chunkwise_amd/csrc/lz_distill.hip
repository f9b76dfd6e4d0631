// lz_distill.hip -- the stage-1 attention-approximation loss on gfx950.
//
// The first training stage fits the linearized layer to the teacher's
// softmax attention with a mean squared error (gist.science explainer of
// "Lizard: An Efficient Linearization Framework for Large Language Models",
// English page §2, "Stage 1: Attention Approximation"; French page "Étape 1";
// Chinese page, first training stage).  For one layer:
//
//   o_T  = causal softmax attention of the teacher's q, k, v (scale s)
//   loss = sum over every element of (o_S - o_T)^2 / N,   N = B*H*L*d
//   dO   = 2 (o_S - o_T) / N          (the gradient the layer backward takes)
//
// teacher_mse_kernel runs the teacher attention flash-style and applies the
// loss in its epilogue, so o_T never reaches HBM: one workgroup of four waves
// per (batch, head, block of 128 queries); wave w owns queries 32w .. 32w+31
// of the block as two 16-query blocks that share every key and value
// fragment it reads.  Key/value tiles of 64 tokens pass through two LDS
// stages (the next tile loads into registers while the current one is
// used).  Score tiles are formed transposed (keys x queries) so a lane holds
// one query's scores; the online softmax works in base 2 and the
// probabilities feed P V straight from registers; the output accumulates
// transposed (d x queries).  Workgroups of later (longer) query blocks start
// first, and all blocks of one head share an XCD.  Each workgroup writes one
// partial sum of squares; loss_reduce_kernel adds them in a fixed order.
#include "lz_common.hpp"
#include "lz_kernels.hpp"

namespace lz {
namespace {

constexpr int TQ = 128;        // queries per workgroup
constexpr int TK = 64;         // keys per tile
// four waves of 32 queries: eight waves of 16 read the same K and V tiles for half the
// queries each (slower), two waves of 64 do not fit their tiles and accumulators in registers
constexpr int NW_TE = 4;                   // waves per workgroup
constexpr int NQB_TE = TQ / (16 * NW_TE);  // 16-query blocks per wave
constexpr int NTHR_TE = 64 * NW_TE;

template <typename T, int D>
struct TeLayout {
  static constexpr int LDQ = D + Tr<T>::PAD;
  static constexpr size_t tile = sizeof(T) * TK * LDQ;
  static constexpr size_t bytes = 4 * tile;   // stage s: keys at 2s, values at 2s + 1
  static_assert(bytes <= 80 * 1024, "two workgroups per CU");
  static_assert(NQB_TE * 16 * NW_TE == TQ, "query blocks");
};

// Online-softmax update of one query row (this lane's query) with four key
// blocks of logits x (base-2 units, -inf where masked); x becomes the
// unnormalised probabilities.
template <int JB>
__device__ __forceinline__ void te_absorb(f32x4 (&x)[4], float& mrun, float& lpart, f32x4 (&O)[JB]) {
  float mx = -INFINITY;
#pragma unroll
  for (int b = 0; b < 4; ++b)
#pragma unroll
    for (int i = 0; i < 4; ++i) mx = fmaxf(mx, x[b][i]);
  mx = xor_max(mx, 16);
  mx = xor_max(mx, 32);
  const float mnew = fmaxf(mrun, mx);
  if (__any(mnew != mrun)) {   // wave-uniform: rescale only when some query's running max moved
    const float alpha = (mrun == -INFINITY) ? 0.f : fast_exp2(mrun - mnew);
    lpart *= alpha;
#pragma unroll
    for (int j = 0; j < JB; ++j) O[j] *= alpha;
  }
  const float mref = (mnew == -INFINITY) ? 0.f : mnew;
  mrun = mnew;
#pragma unroll
  for (int b = 0; b < 4; ++b)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float p = fast_exp2(x[b][i] - mref);
      x[b][i] = p;
      lpart += p;
    }
}

// Four consecutive values of T from global memory as floats.
__device__ __forceinline__ f32x4 ldg4f(const float* p) { return *reinterpret_cast<const f32x4*>(p); }
__device__ __forceinline__ f32x4 ldg4f(const bf16_t* p) {
  const bf16x4 x = *reinterpret_cast<const bf16x4*>(p);
  return f32x4{(float)x[0], (float)x[1], (float)x[2], (float)x[3]};
}

template <typename T, int D>
__global__ __launch_bounds__(NTHR_TE, 2) void teacher_mse_kernel(DistillArgs a) {
  constexpr int NQ = NQB_TE, QW = 16 * NQ;        // query blocks / queries per wave
  using LY = TeLayout<T, D>;
  using frag = typename Tr<T>::frag;
  constexpr int VEC = Tr<T>::VEC, LDQ = LY::LDQ;
  constexpr int JB = D / 16, KS = D / 32;
  constexpr int NVT = TK * (D / VEC) / NTHR_TE;   // 16-byte vectors per thread of a [TK][D] tile

  extern __shared__ __align__(16) unsigned char smem[];
  __shared__ float red[NTHR_TE / 64];

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, r = lane & 15, kg = lane >> 4;
  const int L = a.L, BH = a.B * a.H, NQB = (L + TQ - 1) / TQ;
  // workgroup -> (head, query block).  With B*H a multiple of 8, workgroup bid runs on XCD
  // bid % 8, and each XCD takes its heads one after another, every query block of a head
  // (longest first) before the next head: the blocks in flight on an XCD then stream the same
  // keys and values, which stay in its L2.  Otherwise the longest blocks of all heads go first.
  const int bid = blockIdx.x;
  int bh, qb;
  if ((BH & 7) == 0) {
    const int x = bid & 7, slot = bid >> 3;
    bh = (slot / NQB) * 8 + x;
    qb = NQB - 1 - slot % NQB;
  } else {
    bh = bid % BH;
    qb = NQB - 1 - bid / BH;
  }
  const size_t hoff = (size_t)bh * L * D;
  const T* q = reinterpret_cast<const T*>(a.q) + hoff;
  const T* k = reinterpret_cast<const T*>(a.k) + hoff;
  const T* v = reinterpret_cast<const T*>(a.v) + hoff;
  const float sl2 = a.scale * LOG2E;
  const int q0 = qb * TQ, qw = q0 + QW * w;       // first query of the block / of this wave
  int tq[NQ];                                     // this lane's queries
#pragma unroll
  for (int b = 0; b < NQ; ++b) tq[b] = qw + 16 * b + r;

  frag qf[NQ][KS];
#pragma unroll
  for (int b = 0; b < NQ; ++b)
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) qf[b][ks] = ldg_row_frag<T>(q, D, tq[b], 32 * ks + 8 * kg, L);

  // key / value tiles: rows past the end are loaded from the last row; causality hides them
  V16 wk[NVT], wv[NVT];
  auto load_tile = [&](int kt) {
#pragma unroll
    for (int u = 0; u < NVT; ++u) {
      const int idx = tid + u * NTHR_TE, row = idx / (D / VEC), cv = idx % (D / VEC);
      const size_t o = (size_t)min(kt * TK + row, L - 1) * D + cv * VEC;
      wk[u] = ldg16(k + o);
      wv[u] = ldg16(v + o);
    }
  };
  auto store_tile = [&](int stage) {
    T* sK = reinterpret_cast<T*>(smem + (2 * stage) * LY::tile);
    T* sV = reinterpret_cast<T*>(smem + (2 * stage + 1) * LY::tile);
#pragma unroll
    for (int u = 0; u < NVT; ++u) {
      const int idx = tid + u * NTHR_TE, row = idx / (D / VEC), cv = idx % (D / VEC);
      *reinterpret_cast<V16*>(sK + row * LDQ + cv * VEC) = wk[u];
      *reinterpret_cast<V16*>(sV + row * LDQ + cv * VEC) = wv[u];
    }
  };

  f32x4 O[NQ][JB];
  float mrun[NQ], lpart[NQ];
#pragma unroll
  for (int b = 0; b < NQ; ++b) {
#pragma unroll
    for (int j = 0; j < JB; ++j) O[b][j] = f32x4{0, 0, 0, 0};
    mrun[b] = -INFINITY;
    lpart[b] = 0.f;
  }

  const int ktmax = min(L - 1, q0 + TQ - 1) / TK;   // last key tile the block sees
  load_tile(0);
  store_tile(0);
  __syncthreads();
  for (int kt = 0; kt <= ktmax; ++kt) {
    const int stage = kt & 1;
    const bool more = kt < ktmax;
    if (more) load_tile(kt + 1);
    const T* sK = reinterpret_cast<const T*>(smem + (2 * stage) * LY::tile);
    const T* sV = reinterpret_cast<const T*>(smem + (2 * stage + 1) * LY::tile);
    const int kbase = kt * TK;
    if (kbase + TK - 1 <= qw) {
      // every key of the tile precedes every query of the wave: no mask, no branch, no drain
      f32x4 x[NQ][4];
      // a wave issues the products of a tile at raised priority and its softmax at the
      // normal one: of the two waves sharing a SIMD, the one with matrix work is served
      // first, and the other's softmax fills the remaining issue slots
      __builtin_amdgcn_s_setprio(1);
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) {
#pragma unroll
        for (int b = 0; b < NQ; ++b) x[b][kb] = f32x4{0, 0, 0, 0};
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
          const frag kf = ld_frag(sK, LDQ, 16 * kb + r, 32 * ks + 8 * kg);
#pragma unroll
          for (int b = 0; b < NQ; ++b) mma32(x[b][kb], kf, qf[b][ks]);
        }
      }
      __builtin_amdgcn_s_setprio(0);
#pragma unroll
      for (int b = 0; b < NQ; ++b) {
#pragma unroll
        for (int kb = 0; kb < 4; ++kb) x[b][kb] *= sl2;
        te_absorb<JB>(x[b], mrun[b], lpart[b], O[b]);
      }
      __builtin_amdgcn_s_setprio(1);
#pragma unroll
      for (int p = 0; p < 2; ++p) {
        frag bop[NQ];
#pragma unroll
        for (int b = 0; b < NQ; ++b) pack_acc(bop[b], x[b][2 * p], x[b][2 * p + 1]);
#pragma unroll
        for (int jb = 0; jb < JB; ++jb) {
          const frag vf = ld_frag_tr(sV, LDQ, 32 * p + 4 * kg, 32 * p + 16 + 4 * kg, 16 * jb, lane);
#pragma unroll
          for (int b = 0; b < NQ; ++b) mma32(O[b][jb], vf, bop[b]);
        }
      }
      __builtin_amdgcn_s_setprio(0);
    } else if (kbase <= qw + QW - 1) {   // the diagonal: some keys are visible to some queries
      bool vis[NQ][4];
      f32x4 x[NQ][4];
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) {
        const int s0 = kbase + 16 * kb;
#pragma unroll
        for (int b = 0; b < NQ; ++b) {
          vis[b][kb] = s0 <= qw + 16 * b + 15;
          x[b][kb] = f32x4{0, 0, 0, 0};
        }
        if (vis[NQ - 1][kb]) {   // the last block sees every key an earlier block sees
#pragma unroll
          for (int ks = 0; ks < KS; ++ks) {
            const frag kf = ld_frag(sK, LDQ, 16 * kb + r, 32 * ks + 8 * kg);
#pragma unroll
            for (int b = 0; b < NQ; ++b)
              if (vis[b][kb]) mma32(x[b][kb], kf, qf[b][ks]);
          }
        }
      }
#pragma unroll
      for (int b = 0; b < NQ; ++b) {
#pragma unroll
        for (int kb = 0; kb < 4; ++kb)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int s = kbase + 16 * kb + 4 * kg + i;
            x[b][kb][i] = (vis[b][kb] && s <= tq[b]) ? x[b][kb][i] * sl2 : -INFINITY;
          }
        if (vis[b][0]) te_absorb<JB>(x[b], mrun[b], lpart[b], O[b]);
      }
#pragma unroll
      for (int p = 0; p < 2; ++p) {
        if (!(vis[NQ - 1][2 * p] || vis[NQ - 1][2 * p + 1])) continue;
        frag bop[NQ];
        bool vb[NQ];
#pragma unroll
        for (int b = 0; b < NQ; ++b) {
          pack_acc(bop[b], x[b][2 * p], x[b][2 * p + 1]);
          vb[b] = vis[b][2 * p] || vis[b][2 * p + 1];
        }
#pragma unroll
        for (int jb = 0; jb < JB; ++jb) {
          const frag vf = ld_frag_tr(sV, LDQ, 32 * p + 4 * kg, 32 * p + 16 + 4 * kg, 16 * jb, lane);
#pragma unroll
          for (int b = 0; b < NQ; ++b)
            if (vb[b]) mma32(O[b][jb], vf, bop[b]);
        }
      }
    }
    if (more) store_tile(stage ^ 1);   // that stage was last read before the previous barrier
    __syncthreads();
  }

  // epilogue: o_T = O / l; dO = 2 (o_S - o_T) / N; sum of squares for the loss
  // Every o_S value is loaded (raw, rows clamped into the sequence) before the first dO
  // store: the compiler cannot tell the two tensors apart, so a load after a store would
  // wait for a full memory round trip each time.
  const T* os = reinterpret_cast<const T*>(a.o_s) + hoff;
  T* dO = reinterpret_cast<T*>(a.dO) + hoff;
  using R4 = decltype(ld4raw(os));
  R4 sraw[NQ][JB];
#pragma unroll
  for (int b = 0; b < NQ; ++b)
#pragma unroll
    for (int jb = 0; jb < JB; ++jb) sraw[b][jb] = ld4raw(os + (size_t)min(tq[b], L - 1) * D + 16 * jb + 4 * kg);
  const float g2 = 2.f * a.inv_n;
  float sq = 0.f;
#pragma unroll
  for (int b = 0; b < NQ; ++b) {
    const float l = xor_sum(xor_sum(lpart[b], 16), 32);
    const float inv = 1.f / l;
    if (tq[b] < L) {
#pragma unroll
      for (int jb = 0; jb < JB; ++jb) {
        const size_t o = (size_t)tq[b] * D + 16 * jb + 4 * kg;
        f32x4 d;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          d[e] = (float)sraw[b][jb][e] - inv * O[b][jb][e];
          sq += d[e] * d[e];
        }
        stg4(dO + o, g2 * d[0], g2 * d[1], g2 * d[2], g2 * d[3]);
      }
    }
  }
  sq = xor_sum(xor_sum(row_sum16(sq), 16), 32);
  if (lane == 0) red[w] = sq;
  __syncthreads();
  if (tid == 0) {
    float t = 0.f;
#pragma unroll
    for (int i = 0; i < NTHR_TE / 64; ++i) t += red[i];
    a.partial[bid] = t;
  }
}

// loss = (sum of the partials, in index order per thread, then a fixed tree) / N
__global__ __launch_bounds__(256) void loss_reduce_kernel(const float* __restrict__ part, int n, double inv_n,
                                                          float* __restrict__ loss) {
  __shared__ double s[256];
  double t = 0.0;
  for (int i = threadIdx.x; i < n; i += 256) t += part[i];
  s[threadIdx.x] = t;
  __syncthreads();
  for (int h = 128; h > 0; h >>= 1) {
    if ((int)threadIdx.x < h) s[threadIdx.x] += s[threadIdx.x + h];
    __syncthreads();
  }
  if (threadIdx.x == 0) *loss = (float)(s[0] * inv_n);
}

template <typename T, int D>
hipError_t launch_distill_t(const DistillArgs& a, hipStream_t st) {
  using LY = TeLayout<T, D>;
  const int nwg = a.B * a.H * ((a.L + TQ - 1) / TQ);
  if (a.L > 0) {
    // set on every launch: idempotent and cheap, and no process-wide flag to race on
    hipError_t ea = hipFuncSetAttribute(reinterpret_cast<const void*>(teacher_mse_kernel<T, D>),
                                        hipFuncAttributeMaxDynamicSharedMemorySize, (int)LY::bytes);
    if (ea != hipSuccess) return ea;
    hipLaunchKernelGGL((teacher_mse_kernel<T, D>), dim3(nwg), dim3(NTHR_TE), LY::bytes, st, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  const double n = (double)a.B * a.H * a.L * D;
  hipLaunchKernelGGL(loss_reduce_kernel, dim3(1), dim3(256), 0, st, a.partial, a.L > 0 ? nwg : 0,
                     n > 0 ? 1.0 / n : 0.0, a.loss);
  return hipGetLastError();
}

}  // namespace

size_t distill_workspace_bytes(int B, int H, int L) {
  return (size_t)B * H * ((L + TQ - 1) / TQ) * sizeof(float);
}

hipError_t launch_distill(const DistillArgs& a, int dtype, int D, hipStream_t st) {
  if (dtype == 1) return D == 64 ? launch_distill_t<bf16_t, 64>(a, st) : launch_distill_t<bf16_t, 128>(a, st);
  return launch_distill_t<float, 64>(a, st);
}

}  // namespace lz
