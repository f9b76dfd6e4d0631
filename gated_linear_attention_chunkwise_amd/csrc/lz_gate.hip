// lz_gate.hip -- the gate projection of the layer and its backward on gfx950.
//
// The learnable gating module (gist.science explainer of "Lizard: An
// Efficient Linearization Framework for Large Language Models", English page
// §2.A "Adaptive Memory Control"; Chinese page §2.1) makes the decay of token
// t from its input: Gamma_t = sigmoid(W x_t).  The layer consumes the gate in
// log space (English page §2.C), so the forward here produces
//
//   g = log sigmoid(x W^T) / tau        x [B,L,d_model], W [Ng,d_model]
//
// written straight into the layer's gate layout [B,H,L,d_k] (row n = h*d_k+i
// of W) or [B,H,L] (scalar gate, row n = h), fp32.  The backward uses
// d log sigmoid(z)/dz = 1 - sigmoid(z) = -expm1(tau*g), so it needs g, not z:
//
//   dz = -dg * expm1(tau*g) / tau   (token-major [T, Ng], operand dtype)
//   dx = dz W,   dW = dz^T x        (T = B*L tokens)
//
// Every product is one launch of the same LDS-tiled MFMA GEMM.  Each operand
// tile is copied from a row-major source with the source's contiguous
// direction along the LDS rows; when that direction is the contraction index
// the MFMA fragment is a plain 16-byte LDS read, otherwise it is the gfx950
// LDS transpose read.  The forward fuses the log-sigmoid, the temperature and
// the scatter into the gate layout into its epilogue; dW is split over tokens
// when its output alone has too few tiles to fill the chip, and the splits are
// summed in a fixed order (deterministic).
#include <math.h>

#include "lz_common.hpp"
#include "lz_kernels.hpp"

namespace lz {
namespace {

enum { EPI_GATE = 0, EPI_STORE = 1, EPI_F32 = 2 };

struct GemmArgs {
  // A: AKC ? [M][K] : [K][M]; B: BKC ? [N][K] : [K][N]; row-major, leading dims lda / ldb;
  // a_rows x a_cols and b_rows x b_cols are the valid extents (whole 16-byte vectors)
  const void* A; int lda, a_rows, a_cols;
  const void* Bm; int ldb, b_rows, b_cols;
  int M, N;
  int kper, ksplit, k_total;   // contraction split over blockIdx.y, kper a multiple of BK
  void* C; int ldc;            // EPI_STORE: T [M][ldc]; EPI_F32: fp32, + split * M * ldc when ksplit > 1
  float* g; int B, H, L, dk, sg; float tau;   // EPI_GATE: rows are tokens, columns gate rows n
};

// Row padding (elements) of an LDS operand tile.  Tiles read with 16-byte rows of
// fragments (contraction index along the row) take 16 bytes; tiles read with the
// transpose read (four rows of 32 bytes per 16 lanes) take 32 bytes, so the four rows
// of one read start 8 banks apart.
template <typename T, bool KC>
constexpr int tile_pad() { return sizeof(T) == 2 ? (KC ? 8 : 16) : 4; }

// One operand tile: R rows x C contiguous columns of a row-major source, held
// in registers as 16-byte vectors between its global load and its LDS store
// (rows of C + PAD elements).
template <typename T, int R, int C, int NT, int PAD>
struct TileLd {
  static constexpr int VEC = Tr<T>::VEC;
  static constexpr int NV = R * C / VEC / NT;
  static_assert(NV * VEC * NT == R * C, "tile must split evenly over the threads");
  V16 v[NV];
  uint32_t ok = 0;
  __device__ void load(const T* src, int ld, int row0, int col0, int rows, int cols, int tid) {
    ok = 0;
#pragma unroll
    for (int u = 0; u < NV; ++u) {
      const int idx = tid + u * NT, r = idx / (C / VEC), c = (idx % (C / VEC)) * VEC;
      const int gr = row0 + r, gc = col0 + c;
      const bool valid = gr < rows && gc < cols;
      ok |= uint32_t(valid) << u;
      // unconditional load at a clamped address; invalid vectors are zeroed at the LDS store
      v[u] = ldg16(src + (size_t)min(gr, rows - 1) * ld + min(gc, cols - VEC));
    }
  }
  __device__ void store(T* lds, int tid) const {
#pragma unroll
    for (int u = 0; u < NV; ++u) {
      const int idx = tid + u * NT, r = idx / (C / VEC), c = (idx % (C / VEC)) * VEC;
      *reinterpret_cast<V16*>(lds + r * (C + PAD) + c) = ((ok >> u) & 1u) ? v[u] : zero16();
    }
  }
};

// log sigmoid(z) = min(z, 0) - log1p(exp(-|z|)), short enough to unroll over a whole
// accumulator tile: exp and log from the base-2 hardware instructions, and log1p(u) as
// log(w) * u / (w - 1) with w = 1 + u, which cancels the rounding of w (Goldberg, "What
// every computer scientist should know about floating-point arithmetic", 1991, Theorem 4).
__device__ __forceinline__ float log_sigmoid(float z) {
  const float u = __builtin_amdgcn_exp2f(-fabsf(z) * 1.44269504088896341f);   // in (0, 1]
  const float w = 1.f + u;
  const float l = w == 1.f ? u : __builtin_amdgcn_logf(w) * 0.693147180559945309f * (u * __builtin_amdgcn_rcpf(w - 1.f));
  return fminf(z, 0.f) - l;
}

// C[M][N] = sum_k A[m][k] B[k][n] over this workgroup's split of k.
// WGM x WGN waves, each owning a (BM/WGM) x (BN/WGN) block of C in 16 x 16 MFMA tiles.
template <typename T, bool AKC, bool BKC, int EPI, int BM, int BN, int BK, int WGM, int WGN>
struct GemmShape {
  static constexpr int PA = tile_pad<T, AKC>(), PB = tile_pad<T, BKC>();
  // LDS tiles: [rows][cols + pad] with the source's contiguous direction along the rows
  static constexpr int AR = AKC ? BM : BK, AC = AKC ? BK : BM;
  static constexpr int BR = BKC ? BN : BK, BC = BKC ? BK : BN;
  static constexpr int A_ELEMS = AR * (AC + PA), B_ELEMS = BR * (BC + PB);
  static constexpr size_t lds_bytes = 2 * sizeof(T) * (size_t)(A_ELEMS + B_ELEMS);   // two stages
  // the largest tiles keep two register sets of tiles in flight (smaller ones would lose
  // occupancy to the extra registers)
  static constexpr bool DEEP = BM * BN >= 256 * 256;
};

// C[M][N] = sum_k A[m][k] B[k][n] over this workgroup's split of k.
// WGM x WGN waves, each owning a (BM/WGM) x (BN/WGN) block of C in 16 x 16 MFMA tiles.
// Two LDS stages: the tiles of a later step are loaded to registers while step k is
// multiplied from one stage, then stored to the other; one barrier per step.
template <typename T, bool AKC, bool BKC, int EPI, int BM, int BN, int BK, int WGM, int WGN>
__global__ __launch_bounds__(64 * WGM * WGN) void gemm_kernel(GemmArgs a) {
  using SH = GemmShape<T, AKC, BKC, EPI, BM, BN, BK, WGM, WGN>;
  constexpr int NT = 64 * WGM * WGN;
  constexpr int TM = BM / WGM, TN = BN / WGN, MB = TM / 16, NB = TN / 16;
  constexpr int AR = SH::AR, AC = SH::AC, BR = SH::BR, BC = SH::BC, PA = SH::PA, PB = SH::PB;
  static_assert(BK % 32 == 0 && TM % 16 == 0 && TN % 16 == 0, "tile shape");
  using FragT = typename Tr<T>::frag;

  extern __shared__ __align__(16) unsigned char smem[];
  T* const lds = reinterpret_cast<T*>(smem);   // stage s: A at s * (A + B) elements, then B

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, r = lane & 15, kg = lane >> 4;
  const int wm0 = (wave / WGN) * TM, wn0 = (wave % WGN) * TN;

  // workgroup -> output tile; with a whole number of tiles per XCD, each XCD takes a
  // contiguous run of tiles (n fastest), so the A rows of a run share that XCD's L2
  const int mtiles = (a.M + BM - 1) / BM, ntiles = (a.N + BN - 1) / BN, ntot = mtiles * ntiles;
  int tile = blockIdx.x;
  if ((ntot & 7) == 0) tile = (tile & 7) * (ntot >> 3) + (tile >> 3);
  const int m0 = (tile / ntiles) * BM, n0 = (tile % ntiles) * BN;
  const int split = blockIdx.y;
  const int kbeg = split * a.kper, kend = min(a.k_total, kbeg + a.kper);

  const T* Ag = reinterpret_cast<const T*>(a.A);
  const T* Bg = reinterpret_cast<const T*>(a.Bm);
  auto load = [&](auto& xa, auto& xb, int k0) {
    if (AKC) xa.load(Ag, a.lda, m0, k0, a.a_rows, a.a_cols, tid);
    else     xa.load(Ag, a.lda, k0, m0, a.a_rows, a.a_cols, tid);
    if (BKC) xb.load(Bg, a.ldb, n0, k0, a.b_rows, a.b_cols, tid);
    else     xb.load(Bg, a.ldb, k0, n0, a.b_rows, a.b_cols, tid);
  };
  auto store = [&](const auto& xa, const auto& xb, int stage) {
    T* sa = lds + stage * (SH::A_ELEMS + SH::B_ELEMS);
    xa.store(sa, tid);
    xb.store(sa + SH::A_ELEMS, tid);
  };

  f32x4 acc[MB][NB];
#pragma unroll
  for (int i = 0; i < MB; ++i)
#pragma unroll
    for (int j = 0; j < NB; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  auto multiply = [&](int stage) {
    const T* sA = lds + stage * (SH::A_ELEMS + SH::B_ELEMS);
    const T* sB = sA + SH::A_ELEMS;
#pragma unroll
    for (int ks = 0; ks < BK / 32; ++ks) {
      const int kk = 32 * ks + 8 * kg;
      FragT fa[MB], fb[NB];
#pragma unroll
      for (int i = 0; i < MB; ++i) {
        if constexpr (AKC) fa[i] = ld_frag(sA, AC + PA, wm0 + 16 * i + r, kk);
        else               fa[i] = ld_frag_tr(sA, AC + PA, kk, kk + 4, wm0 + 16 * i, lane);
      }
#pragma unroll
      for (int j = 0; j < NB; ++j) {
        if constexpr (BKC) fb[j] = ld_frag(sB, BC + PB, wn0 + 16 * j + r, kk);
        else               fb[j] = ld_frag_tr(sB, BC + PB, kk, kk + 4, wn0 + 16 * j, lane);
      }
#pragma unroll
      for (int i = 0; i < MB; ++i)
#pragma unroll
        for (int j = 0; j < NB; ++j) mma32(acc[i][j], fb[j], fa[i]);   // C^T blocks: lanes hold row runs of C
    }
  };

  TileLd<T, AR, AC, NT, PA> ta0;
  TileLd<T, BR, BC, NT, PB> tb0;
  if constexpr (SH::DEEP) {
    // Two register sets of tiles: tile t is loaded into set t % 2 two steps before it is
    // stored, so a step's loads have two steps of products to arrive.  The loads are
    // unconditional (the last steps repeat the last tile) and the loop runs in pairs of
    // steps, so that no path reaches a wait with a set's loads looking recent.
    TileLd<T, AR, AC, NT, PA> ta1;
    TileLd<T, BR, BC, NT, PB> tb1;
    const int nsteps = kend > kbeg ? (kend - kbeg + BK - 1) / BK : 0;
    const int klast = kbeg + (nsteps > 0 ? nsteps - 1 : 0) * BK;
    auto kstep = [&](int t) { return min(kbeg + t * BK, klast); };
    if (nsteps > 0) {
      // tile 0 to LDS stage 0, tile 1 in set 1, tile 2 in set 0
      load(ta0, tb0, kstep(0));
      store(ta0, tb0, 0);
      load(ta1, tb1, kstep(1));
      load(ta0, tb0, kstep(2));
      __syncthreads();
      int t = 0;
      // step t multiplies stage t % 2, stores tile t + 1 (set (t + 1) % 2) into the other
      // stage, then loads tile t + 3 into that set
      for (; t + 2 <= nsteps; t += 2) {
        multiply(0);
        store(ta1, tb1, 1);
        load(ta1, tb1, kstep(t + 3));
        __syncthreads();
        multiply(1);
        store(ta0, tb0, 0);
        load(ta0, tb0, kstep(t + 4));
        __syncthreads();
      }
      if (t < nsteps) multiply(0);
    }
  } else {
    // one register set: the tiles of step k+1 are loaded while step k is multiplied
    if (kbeg < kend) {
      load(ta0, tb0, kbeg);
      store(ta0, tb0, 0);
      __syncthreads();
    }
    int stage = 0;
    for (int k0 = kbeg; k0 < kend; k0 += BK) {
      const bool more = k0 + BK < kend;
      if (more) load(ta0, tb0, k0 + BK);   // next tiles in flight while this one is multiplied
      multiply(stage);
      if (more) store(ta0, tb0, stage ^ 1);   // that stage was last read before the previous barrier
      __syncthreads();
      stage ^= 1;
    }
  }

  // epilogue: the blocks were formed transposed, so lane holds C[m][n .. n+3] with
  // m = m0 + wm0 + 16 i + r, n = n0 + wn0 + 16 j + 4 kg (four consecutive columns)
  if constexpr (EPI == EPI_GATE) {
    // m = token b*L + t, n = gate row; the gate offset splits into a row part and a column
    // part: per key dimension ((b*H*L + t) * dk) + (h*L*dk + i) with n = h*dk + i (the four
    // columns are four consecutive i of one head), scalar (b*H*L + t) + n*L
    const float inv_tau = 1.f / a.tau;
    size_t colp[NB];
#pragma unroll
    for (int j = 0; j < NB; ++j) {
      const int n = n0 + wn0 + 16 * j + 4 * kg;
      const int h = a.sg ? n : n / a.dk;
      colp[j] = a.sg ? (size_t)n * a.L : (size_t)h * a.L * a.dk + (n - h * a.dk);
    }
#pragma unroll
    for (int i = 0; i < MB; ++i) {
      const int m = m0 + wm0 + 16 * i + r;
      if (m >= a.M) continue;
      const int b = m / a.L, t = m - b * a.L;
      const size_t rowp = ((size_t)b * a.H * a.L + t) * (a.sg ? 1 : a.dk);
#pragma unroll
      for (int j = 0; j < NB; ++j) {
        const int n = n0 + wn0 + 16 * j + 4 * kg;
        const f32x4 v = acc[i][j];
        if (!a.sg) {
          if (n < a.N)   // N = H*dk is a multiple of 4
            *reinterpret_cast<f32x4*>(a.g + rowp + colp[j]) =
                f32x4{log_sigmoid(v[0]) * inv_tau, log_sigmoid(v[1]) * inv_tau, log_sigmoid(v[2]) * inv_tau,
                      log_sigmoid(v[3]) * inv_tau};
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e)
            if (n + e < a.N) a.g[rowp + colp[j] + (size_t)e * a.L] = log_sigmoid(v[e]) * inv_tau;
        }
      }
    }
  } else {
    // N is d_model, a multiple of 32: the four columns are all in range together
#pragma unroll
    for (int i = 0; i < MB; ++i) {
      const int m = m0 + wm0 + 16 * i + r;
      if (m >= a.M) continue;
#pragma unroll
      for (int j = 0; j < NB; ++j) {
        const int n = n0 + wn0 + 16 * j + 4 * kg;
        if (n >= a.N) continue;
        const f32x4 v = acc[i][j];
        if constexpr (EPI == EPI_STORE) {
          st4(reinterpret_cast<T*>(a.C) + (size_t)m * a.ldc + n, v[0], v[1], v[2], v[3]);
        } else {
          float* out = reinterpret_cast<float*>(a.C) + (a.ksplit > 1 ? (size_t)split * a.M * a.ldc : 0);
          *reinterpret_cast<f32x4*>(out + (size_t)m * a.ldc + n) = v;
        }
      }
    }
  }
}

// dz[t][n] = -dg * expm1(tau * g) / tau, token-major with leading dimension ldz (Ng rounded
// up to whole 16-byte vectors; the padding columns are written as zero).
template <typename T>
__global__ __launch_bounds__(256) void gate_dz_kernel(const float* __restrict__ g, const float* __restrict__ dg,
                                                      T* __restrict__ dz, int B, int H, int L, int dk, int sg,
                                                      int ldz, float tau) {
  const int T_ = B * L, n4 = ldz / 4;
  const size_t idx = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= (size_t)T_ * n4) return;
  float out[4];
  if (sg) {
    // one gate per head: column n = h; consecutive threads take consecutive tokens
    const int tt = (int)(idx % T_), c = (int)(idx / T_) * 4;
    const int b = tt / L, t = tt - b * L;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int h = c + e;
      const size_t o = ((size_t)b * H + min(h, H - 1)) * L + t;
      const float gv = g[o], d = dg[o];
      out[e] = h < H ? -d * expm1f(tau * gv) / tau : 0.f;
    }
    T* p = dz + (size_t)tt * ldz + c;
#pragma unroll
    for (int e = 0; e < 4; ++e) p[e] = Tr<T>::from_f(out[e]);
  } else {
    const int tt = (int)(idx / n4), c = (int)(idx % n4) * 4;
    const int b = tt / L, t = tt - b * L, h = c / dk, i = c - h * dk;
    const size_t o = (((size_t)b * H + h) * L + t) * dk + i;
    const f32x4 gv = *reinterpret_cast<const f32x4*>(g + o);
    const f32x4 d = *reinterpret_cast<const f32x4*>(dg + o);
#pragma unroll
    for (int e = 0; e < 4; ++e) out[e] = -d[e] * expm1f(tau * gv[e]) / tau;
    T* p = dz + (size_t)tt * ldz + c;
    if constexpr (sizeof(T) == 2) {
      *reinterpret_cast<bf16x4*>(p) = bf16x4{(__bf16)out[0], (__bf16)out[1], (__bf16)out[2], (__bf16)out[3]};
    } else {
      *reinterpret_cast<f32x4*>(p) = f32x4{out[0], out[1], out[2], out[3]};
    }
  }
}

// dW = sum over the token splits, in split order.
__global__ __launch_bounds__(256) void split_sum_kernel(const float* __restrict__ part, float* __restrict__ out,
                                                        size_t n4, int ksplit) {
  const size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n4) return;
  f32x4 s = reinterpret_cast<const f32x4*>(part)[i];
  for (int k = 1; k < ksplit; ++k) {
    const f32x4 v = reinterpret_cast<const f32x4*>(part)[(size_t)k * n4 + i];
    s += v;
  }
  reinterpret_cast<f32x4*>(out)[i] = s;
}

__global__ __launch_bounds__(256) void zero4_kernel(float* __restrict__ out, size_t n4) {
  const size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n4) reinterpret_cast<f32x4*>(out)[i] = f32x4{0.f, 0.f, 0.f, 0.f};
}

template <typename T, bool AKC, bool BKC, int EPI, int BM, int BN, int BK, int WGM, int WGN>
hipError_t run_gemm(const GemmArgs& a, hipStream_t st) {
  constexpr size_t lds = GemmShape<T, AKC, BKC, EPI, BM, BN, BK, WGM, WGN>::lds_bytes;
  static_assert(lds <= 160 * 1024, "LDS budget");
  auto kern = gemm_kernel<T, AKC, BKC, EPI, BM, BN, BK, WGM, WGN>;
  // set on every launch: idempotent and cheap, and no process-wide flag to race on
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (e != hipSuccess) return e;
  const int tiles = ((a.M + BM - 1) / BM) * ((a.N + BN - 1) / BN);
  hipLaunchKernelGGL(kern, dim3(tiles, a.ksplit), dim3(64 * WGM * WGN), lds, st, a);
  return hipGetLastError();
}

// Split of a contraction of length K over workgroups so that `tiles` output tiles make at
// least ~1024 workgroups; kper is a multiple of bk.
void split_k(int K, int tiles, int bk, int& ksplit, int& kper) {
  const int steps = (K + bk - 1) / bk;
  int want = (1024 + tiles - 1) / tiles;
  want = want < 1 ? 1 : (want > steps ? steps : want);
  const int per_steps = (steps + want - 1) / want;
  kper = per_steps * bk;
  ksplit = K > 0 ? (K + kper - 1) / kper : 1;
}

int dz_ld(int Ng, int dtype) {
  const int vec = dtype == 1 ? 8 : 4;
  return (Ng + vec - 1) / vec * vec;
}

// Tile shapes.  Gate rows Ng = H*d_k (per key dimension: a square, MFMA-bound problem at
// d_model ~ Ng) or H (scalar: a skinny product bound by streaming x or dx).
// contraction depth of the skinny (scalar-gate) products: deep steps keep enough bytes in flight
constexpr int fwd_bk_scalar(int dtype) { return dtype == 1 ? 256 : 128; }
constexpr int dw_bk_scalar(int dtype) { return dtype == 1 ? 128 : 64; }

size_t align256(size_t n) { return (n + 255) & ~(size_t)255; }

// output tiles of the per-key-dimension dW product (256 x 256 for bf16, 128 x 128 for fp32)
int dw_tiles(int Ng, int Dm, int dtype) {
  const int t = dtype == 1 ? 256 : 128;
  return ((Ng + t - 1) / t) * ((Dm + t - 1) / t);
}

size_t dw_part_bytes(int T_, int Ng, int Dm, bool sg, int dtype) {
  int ksplit, kper;
  if (sg) split_k(T_, ((Ng + 31) / 32) * ((Dm + 127) / 128), dw_bk_scalar(dtype), ksplit, kper);
  else    split_k(T_, dw_tiles(Ng, Dm, dtype), 32, ksplit, kper);
  return ksplit > 1 ? (size_t)ksplit * Ng * Dm * sizeof(float) : 0;
}

template <typename T>
hipError_t gate_fwd_t(const GateArgs& p, hipStream_t st) {
  const int T_ = p.B * p.L, Ng = p.sg ? p.H : p.H * p.dk;
  GemmArgs a{};
  a.A = p.x; a.lda = p.d_model; a.a_rows = T_; a.a_cols = p.d_model;
  a.Bm = p.w; a.ldb = p.d_model; a.b_rows = Ng; a.b_cols = p.d_model;
  a.M = T_; a.N = Ng; a.ksplit = 1; a.k_total = p.d_model; a.kper = p.d_model;
  a.g = p.g; a.B = p.B; a.H = p.H; a.L = p.L; a.dk = p.dk; a.sg = p.sg; a.tau = p.tau;
  constexpr int DT = sizeof(T) == 2 ? 1 : 0;
  if (p.sg) return run_gemm<T, true, true, EPI_GATE, 64, 32, fwd_bk_scalar(DT), 4, 1>(a, st);
  if constexpr (DT == 1) return run_gemm<T, true, true, EPI_GATE, 256, 256, 32, 4, 2>(a, st);
  return run_gemm<T, true, true, EPI_GATE, 128, 128, 32, 2, 2>(a, st);
}

template <typename T>
hipError_t gate_bwd_t(const GateArgs& p, hipStream_t st) {
  const int T_ = p.B * p.L, Ng = p.sg ? p.H : p.H * p.dk, ldz = dz_ld(Ng, sizeof(T) == 2 ? 1 : 0);
  T* dz = reinterpret_cast<T*>(p.workspace);
  float* part = reinterpret_cast<float*>(reinterpret_cast<char*>(p.workspace) +
                                         align256((size_t)T_ * ldz * sizeof(T)));
  {
    const size_t n = (size_t)T_ * (ldz / 4);
    hipLaunchKernelGGL(gate_dz_kernel<T>, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st, p.g, p.dg, dz, p.B,
                       p.H, p.L, p.dk, p.sg, ldz, p.tau);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  hipError_t e;
  {
    // dx [T][d_model] = dz [T][Ng] . W [Ng][d_model]
    GemmArgs a{};
    a.A = dz; a.lda = ldz; a.a_rows = T_; a.a_cols = ldz;
    a.Bm = p.w; a.ldb = p.d_model; a.b_rows = Ng; a.b_cols = p.d_model;
    a.M = T_; a.N = p.d_model; a.ksplit = 1; a.k_total = Ng; a.kper = Ng;
    a.C = p.dx; a.ldc = p.d_model;
    // scalar gate: one 32-deep step per tile, bound by writing dx
    bool big = false;
    if constexpr (sizeof(T) == 2) {
      if (!p.sg) { e = run_gemm<T, true, false, EPI_STORE, 256, 256, 32, 4, 2>(a, st); big = true; }
    }
    if (!big) e = run_gemm<T, true, false, EPI_STORE, 128, 128, 32, 2, 2>(a, st);
    if (e != hipSuccess) return e;
  }
  {
    // dW [Ng][d_model] = dz^T . x, contraction over the tokens
    GemmArgs a{};
    a.A = dz; a.lda = ldz; a.a_rows = T_; a.a_cols = ldz;
    a.Bm = p.x; a.ldb = p.d_model; a.b_rows = T_; a.b_cols = p.d_model;
    a.M = Ng; a.N = p.d_model; a.k_total = T_; a.ldc = p.d_model;
    int ksplit, kper;
    constexpr int DT = sizeof(T) == 2 ? 1 : 0;
    if (p.sg) split_k(T_, ((Ng + 31) / 32) * ((p.d_model + 127) / 128), dw_bk_scalar(DT), ksplit, kper);
    else      split_k(T_, dw_tiles(Ng, p.d_model, DT), 32, ksplit, kper);
    a.ksplit = ksplit; a.kper = kper;
    a.C = ksplit > 1 ? (void*)part : (void*)p.dw;
    if (p.sg) e = run_gemm<T, false, false, EPI_F32, 32, 128, dw_bk_scalar(DT), 1, 4>(a, st);
    else if constexpr (DT == 1) e = run_gemm<T, false, false, EPI_F32, 256, 256, 32, 4, 2>(a, st);
    else                        e = run_gemm<T, false, false, EPI_F32, 128, 128, 32, 2, 2>(a, st);
    if (e != hipSuccess) return e;
    if (ksplit > 1) {
      const size_t n4 = (size_t)Ng * p.d_model / 4;
      hipLaunchKernelGGL(split_sum_kernel, dim3((unsigned)((n4 + 255) / 256)), dim3(256), 0, st, part, p.dw, n4,
                         ksplit);
      e = hipGetLastError();
    }
  }
  return e;
}

}  // namespace

size_t gate_bwd_workspace_bytes(int B, int H, int L, int dk, int sg, int d_model, int dtype) {
  const int T_ = B * L, Ng = sg ? H : H * dk;
  const size_t esz = dtype == 1 ? 2 : 4;
  return align256((size_t)T_ * dz_ld(Ng, dtype) * esz) + dw_part_bytes(T_, Ng, d_model, sg != 0, dtype);
}

hipError_t launch_gate_fwd(const GateArgs& a, int dtype, hipStream_t st) {
  return dtype == 1 ? gate_fwd_t<bf16_t>(a, st) : gate_fwd_t<float>(a, st);
}

hipError_t launch_gate_bwd(const GateArgs& a, int dtype, hipStream_t st) {
  if (a.L == 0) {   // no tokens: dx is empty and dW is zero
    const size_t n4 = (size_t)(a.sg ? a.H : a.H * a.dk) * a.d_model / 4;
    hipLaunchKernelGGL(zero4_kernel, dim3((unsigned)((n4 + 255) / 256)), dim3(256), 0, st, a.dw, n4);
    return hipGetLastError();
  }
  return dtype == 1 ? gate_bwd_t<bf16_t>(a, st) : gate_bwd_t<float>(a, st);
}

}  // namespace lz
