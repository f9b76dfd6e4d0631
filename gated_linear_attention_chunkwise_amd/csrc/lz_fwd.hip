// lz_fwd.hip -- forward pass of the Lizard hybrid attention layer on gfx950.
//
// Two launches (more when the sweep runs in sequence segments):
//   sweep_kernel (lz_sweep.hip)  the GLA state recurrence over chunks, in
//                 64-row blocks of the state; writes the state entering every chunk
//   out_kernel    one workgroup (4 waves, 16 queries each) per (batch, head,
//                 chunk of C = 64 tokens), all of d_v, so every score is
//                 computed once:
//
//   GLA branch (gist.science explainer of "Lizard: An Efficient
//   Linearization Framework for Large Language Models", English page §2.A
//   state update, §2.C log-space gate handling):
//     b_t  = chunk-local inclusive cumulative sum of the log-gates (fp32)
//     q~_t = q_t * exp(b_t),  k^_s = k_s * exp(-b_s)      (gate folded into q, k)
//     O    = (q~ k^T masked s<=t) V  +  q~ S_c             (bf16 matrix cores)
//   Only chunk-local sums are exponentiated, so no global cumulative gate
//   (which underflows fp32 at long L) ever appears.
//
//   Anchor window (English page §2.A): online softmax of q_t against the M
//   meta keys and keys s in (t-W, t], meta values optional.  The raw key and
//   value tiles of the (at most three) chunks the window reaches are staged
//   in LDS one after the other, the next one loading while the current one is
//   used.
//
//   Output (English page §2.A, final output): o = O_gla + mix * O_swa.
//
// Every score tile is computed transposed (keys x queries) so that one lane
// holds one query's scores: row max / row sum need two cross-lane steps, and
// the probabilities feed the next matrix product straight from registers.
// The outputs are accumulated transposed as well (d_v x queries).
#include <type_traits>

#include "lz_common.hpp"
#include "lz_kernels.hpp"

namespace lz {
namespace {

constexpr int C = CHUNK;
constexpr int NTHR = 256;

// Online-softmax update of one query row (this lane's query) with NB key
// blocks of logits x (log2 units, -inf where masked); x is overwritten with
// the unnormalised probabilities.
template <int NB, int JB>
__device__ __forceinline__ void absorb(f32x4 (&x)[NB], float& mrun, float& lpart, f32x4 (&OW)[JB]) {
  float mx = -INFINITY;
#pragma unroll
  for (int b = 0; b < NB; ++b)
#pragma unroll
    for (int i = 0; i < 4; ++i) mx = fmaxf(mx, x[b][i]);
  mx = xor_max(mx, 16);
  mx = xor_max(mx, 32);
  const float mnew = fmaxf(mrun, mx);
  const float alpha = (mrun == -INFINITY) ? 0.f : fast_exp2(mrun - mnew);
  const float mref = (mnew == -INFINITY) ? 0.f : mnew;   // nothing visible yet: every p is 0
  mrun = mnew;
  lpart *= alpha;
#pragma unroll
  for (int j = 0; j < JB; ++j) OW[j] *= alpha;
#pragma unroll
  for (int b = 0; b < NB; ++b)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float p = fast_exp2(x[b][i] - mref);
      x[b][i] = p;
      lpart += p;
    }
}

template <typename T, int D>
struct OutLayout {
  static constexpr int PAD = Tr<T>::PAD;
  static constexpr int VEC = Tr<T>::VEC;
  static constexpr int LDQ = D + PAD;      // [C][D] tiles, row-major
  static constexpr int LDMV = 16 + PAD;    // sMvt: [D][16]
  static constexpr size_t tile = sizeof(T) * C * LDQ;
  static constexpr size_t oK = 0;          // raw keys of a window chunk, then q~
  static constexpr size_t oV = tile;       // values of a window chunk (ends with this chunk's)
  static constexpr size_t oX = 2 * tile;   // k^ (sub-block path: keys folded to their block end)
  static constexpr size_t oS = 3 * tile;   // 64 rows of the entering state; gate-scan scratch before
  static constexpr size_t oMk = 4 * tile;
  static constexpr size_t oMvt = oMk + sizeof(T) * 16 * LDQ;
  static constexpr size_t bytes = oMvt + sizeof(T) * D * LDMV;
  static_assert(sizeof(float) * ScanMap<D, VEC, NTHR>::NTG * D <= tile, "scan scratch fits");
  static_assert(bytes <= 80 * 1024, "two workgroups per CU");
  // sub-block path only: the fp32 block-local gate prefixes [C][D+4], the 16-token block
  // totals [4][D] and the diagonal blocks' choice
  static constexpr int LDBF = D + 4;
  static constexpr size_t oB = bytes;
  static constexpr size_t oBT = oB + sizeof(float) * C * LDBF;
  static constexpr size_t oPair = oBT + sizeof(float) * 4 * D;
  static constexpr size_t strong_bytes = oPair + sizeof(int) * 4;
  static_assert(strong_bytes <= 160 * 1024, "LDS budget");
};

__device__ __forceinline__ void set_elem(bf16x8& f, int e, float x) { f[e] = (__bf16)x; }
__device__ __forceinline__ void set_elem(f32x8& f, int e, float x) { f[e] = x; }

// One chunk of the forward: 64 queries over all of d_v.
// CONT: the segment continues a sequence (key history in the ring, position offset pos[b]).
// SG: one log-gate per head and token (g [B,H,L]), broadcast over the key dimensions.
// FEAT: the GLA branch reads the fp32 log features lq, lk of phi(q), phi(k) and absorbs the
// gate in log space (q~ = exp(lq + b), k^ = exp(lk - b)); the window keeps the raw q, k.
// STRONG: the intra-chunk scores by 16-token blocks.  Folding the gate into q and k relative
// to the chunk start needs e^(-b) inside the floating-point range, which fails when a column's
// gate sums to less than -kStrongGate over the chunk.  Here the score of query t against key
// s of key block j is sum_i q_t e^(b_t - rho_j) * k_s e^(rho_j - b_s), rho_j = b at the last
// token of block j: both factors are at most 1 for every j below the query's block; on the
// diagonal block the query factor stays below e^kStrongGate unless the block itself decays
// more than that, and such a block takes the exact pairwise form sum_i q k e^(b_t - b_s).  The
// exponents come from block-local sums (the prefix P and suffix S inside a 16-token block, the
// block totals T), never from differences of chunk-cumulative sums, so each is as accurate as
// its own size: b_t - rho_j = P_t + T_{j+1} + .. + T_{i-1} (t in block i), rho_j - b_s = S_s.
// Without STRONG, a chunk flagged by the state sweep is appended to the dispatch list and left
// to the STRONG launch.
template <typename T, int D, bool CONT, bool SG, bool FEAT, bool STRONG>
__device__ __forceinline__ void out_chunk(const FwdArgs& a, const T* __restrict__ cstates, int bh, int c,
                                          unsigned char* smem, int tid) {
  using LY = OutLayout<T, D>;
  using SM = ScanMap<D, Tr<T>::VEC, NTHR>;
  using frag = typename Tr<T>::frag;
  constexpr int VEC = LY::VEC, TPT = SM::TPT, GV = SM::GV;
  constexpr int JB = D / 16, KS = D / 32, LDQ = LY::LDQ, LDBF = LY::LDBF;
  constexpr int NVT = C * (D / VEC) / NTHR;   // 16-byte vectors per thread of a [C][D] tile
  constexpr int NSH = D / 64;                 // 64-row slices of the state

  T* sK = reinterpret_cast<T*>(smem + LY::oK);
  T* sV = reinterpret_cast<T*>(smem + LY::oV);
  T* sX = reinterpret_cast<T*>(smem + LY::oX);
  T* sS = reinterpret_cast<T*>(smem + LY::oS);
  float* sScan = reinterpret_cast<float*>(smem + LY::oS);
  T* sMk = reinterpret_cast<T*>(smem + LY::oMk);
  T* sMvt = reinterpret_cast<T*>(smem + LY::oMvt);
  float* sB = reinterpret_cast<float*>(smem + LY::oB);       // STRONG only
  float* sBT = reinterpret_cast<float*>(smem + LY::oBT);     // STRONG only
  int* sPair = reinterpret_cast<int*>(smem + LY::oPair);     // STRONG only

  const int lane = tid & 63, w = tid >> 6;
  const int r = lane & 15, kg = lane >> 4;
  const int L = a.L, NC = (L + C - 1) / C, M = a.M, W = a.W;
  // fast path: the sweep's strong-column masks of this chunk (checked once the loads are out)
  uint64_t smask = 0;
  if constexpr (!STRONG) {
    const uint64_t* mp = reinterpret_cast<const uint64_t*>(a.strong + ((size_t)bh * NC + c) * (D / 16));
    smask = mp[0];
    if constexpr (D == 128) smask |= mp[1];
  }
  const int h = bh % a.H;
  const size_t hoff = (size_t)bh * L * D;
  const T* q = reinterpret_cast<const T*>(a.q) + hoff;
  const T* k = reinterpret_cast<const T*>(a.k) + hoff;
  const T* v = reinterpret_cast<const T*>(a.v) + hoff;
  const float* g = a.g + (SG ? (size_t)bh * L : hoff);
  const T* Sc = cstates + ((size_t)bh * NC + c) * D * D;
  const float sl2 = a.scale * LOG2E;
  const int t0 = c * C;
  const int tq = t0 + 16 * w + r;               // this lane's query
  const bool qvalid = tq < L;
  const int qlo = t0 + 16 * w;                  // first query of this wave

  // ---- loads: this chunk's q, k, g (gate scan map), the first window tile, query operands
  const int cg = tid % SM::VPR, tg = tid / SM::VPR;
  V16 rq[TPT], rk[TPT];
  f32x4 lqv[TPT][VEC / 4], lkv[TPT][VEC / 4];   // FEAT: log features of the GLA branch
  f32x4 rg[TPT][GV];
#pragma unroll
  for (int u = 0; u < TPT; ++u) {
    const int t = t0 + tg * TPT + u;
    const bool ok = t < L;
    if constexpr (!FEAT) {   // (log features are loaded just before the GLA fold)
      rq[u] = ok ? ldg16(q + (size_t)t * D + cg * VEC) : zero16();
      rk[u] = ok ? ldg16(k + (size_t)t * D + cg * VEC) : zero16();
    }
#pragma unroll
    for (int e = 0; e < GV; ++e)
      if constexpr (SG) {
        const float x = ok ? g[t] : 0.f;
        rg[u][e] = f32x4{x, x, x, x};
      } else {
        rg[u][e] = ok ? *reinterpret_cast<const f32x4*>(g + (size_t)t * D + cg * VEC + 4 * e) : f32x4{0, 0, 0, 0};
      }
  }
  // Continuation: the P tokens before this segment are key positions -P .. -1; the last
  // min(P, W) of them sit in the ring, position s in slot (P + s) mod W.
  const int P = CONT ? a.pos[bh / a.H] : 0;
  const int smin = -min(P, W);                  // oldest key position held
  const T* ringk = reinterpret_cast<const T*>(a.ring_k) + (size_t)bh * W * D;
  const T* ringv = reinterpret_cast<const T*>(a.ring_v) + (size_t)bh * W * D;
  V16 wk[NVT], wv[NVT];
  auto load_tile = [&](int kt) {
#pragma unroll
    for (int u = 0; u < NVT; ++u) {
      const int idx = tid + u * NTHR, row = idx / (D / VEC), cv = idx % (D / VEC);
      const int t = kt * C + row;
      if (!CONT || t >= 0) {
        wk[u] = t < L ? ldg16(k + (size_t)t * D + cv * VEC) : zero16();
        wv[u] = t < L ? ldg16(v + (size_t)t * D + cv * VEC) : zero16();
      } else {
        const size_t o = (size_t)((P + t) % W) * D + cv * VEC;
        wk[u] = t >= smin ? ldg16(ringk + o) : zero16();
        wv[u] = t >= smin ? ldg16(ringv + o) : zero16();
      }
    }
  };
  // oldest key chunk any query of this chunk sees (negative: ring history)
  const int s_lo = CONT ? max(t0 - W + 1, smin) : max(t0 - W + 1, 0);
  const int kt_lo = s_lo >= 0 ? s_lo / C : -((C - 1 - s_lo) / C);
  load_tile(kt_lo);
  frag qf[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) qf[ks] = ldg_row_frag<T>(q, D, tq, 32 * ks + 8 * kg, L);

  if constexpr (!STRONG) {
    if (smask != 0) {   // the sub-block launch takes this chunk
      if (tid == 0) a.list[atomicAdd(a.list_count, 1)] = bh * NC + c;
      return;
    }
  }

  // meta keys / values (values only when given: absent ones add nothing to the weighted value sum)
  for (int e = tid; e < 16 * (D / VEC); e += NTHR) {
    const int m = e / (D / VEC), cv = e % (D / VEC);
    V16 x = zero16();
    if (m < M) x = ldg16(reinterpret_cast<const T*>(a.meta_k) + ((size_t)h * M + m) * D + cv * VEC);
    *reinterpret_cast<V16*>(sMk + m * LDQ + cv * VEC) = x;
  }
  if (a.meta_v != nullptr) {
    for (int e = tid; e < D * 16; e += NTHR) {
      const int j = e / 16, m = e % 16;
      const float x = m < M ? Tr<T>::to_f(reinterpret_cast<const T*>(a.meta_v)[((size_t)h * M + m) * D + j]) : 0.f;
      put_elem(sMvt + j * LY::LDMV + m, x);
    }
  }

  // ---- anchor window: online softmax over the meta keys and keys in (t-W, t]
  f32x4 OW[JB];
#pragma unroll
  for (int j = 0; j < JB; ++j) OW[j] = f32x4{0, 0, 0, 0};
  float mrun = -INFINITY, lpart = 0.f;
  V16 rs0[NVT], rs1[NVT];
  auto load_state = [&](V16 (&dst)[NVT], int hs) {
#pragma unroll
    for (int u = 0; u < NVT; ++u) {
      const int idx = tid + u * NTHR, row = idx / (D / VEC), cv = idx % (D / VEC);
      dst[u] = ldg16(Sc + (size_t)(64 * hs + row) * D + cv * VEC);
    }
  };
  for (int kt = kt_lo; kt <= c; ++kt) {
    __syncthreads();   // the previous tile's readers are done
#pragma unroll
    for (int u = 0; u < NVT; ++u) {
      const int idx = tid + u * NTHR, row = idx / (D / VEC), cv = idx % (D / VEC);
      *reinterpret_cast<V16*>(sK + row * LDQ + cv * VEC) = wk[u];
      *reinterpret_cast<V16*>(sV + row * LDQ + cv * VEC) = wv[u];
    }
    if (kt < c) {
      load_tile(kt + 1);
    } else {
      load_state(rs0, 0);   // last window tile: fetch the entering state's first rows meanwhile
    }
    __syncthreads();

    if (kt == kt_lo && M > 0) {
      f32x4 xm[1];
      xm[0] = f32x4{0, 0, 0, 0};
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) mma32(xm[0], ld_frag(sMk, LDQ, r, 32 * ks + 8 * kg), qf[ks]);
#pragma unroll
      for (int i = 0; i < 4; ++i) xm[0][i] = (4 * kg + i < M) ? xm[0][i] * sl2 : -INFINITY;
      absorb<1, JB>(xm, mrun, lpart, OW);
      if (a.meta_v != nullptr) {   // (without meta values the sinks only enter the denominator)
        frag bop;
        pack_acc(bop, xm[0], f32x4{0, 0, 0, 0});
#pragma unroll
        for (int jb = 0; jb < JB; ++jb) mma32(OW[jb], ld_frag_perm(sMvt, LY::LDMV, 16 * jb + r, 0, 0, kg), bop);
      }
    }

    const int kbase = kt * C;
    // tiles this wave's queries cannot see (the oldest chunk for the first query blocks) are skipped
    if (kbase > qlo + 15 || kbase + C - 1 < qlo - W + 1) continue;
    f32x4 x[4];
    bool vis[4];
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
      const int s0 = kbase + 16 * kb;
      vis[kb] = (s0 <= qlo + 15) && (s0 + 15 >= qlo - W + 1);
      x[kb] = f32x4{0, 0, 0, 0};
      if (vis[kb]) {
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) mma32(x[kb], ld_frag(sK, LDQ, 16 * kb + r, 32 * ks + 8 * kg), qf[ks]);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int s = s0 + 4 * kg + i;
        const bool ok = vis[kb] && s <= tq && s > tq - W && (!CONT || s >= smin);
        x[kb][i] = ok ? x[kb][i] * sl2 : -INFINITY;
      }
    }
    absorb<4, JB>(x, mrun, lpart, OW);
#pragma unroll
    for (int p = 0; p < 2; ++p)
      if (vis[2 * p] || vis[2 * p + 1]) {
        frag bop;
        pack_acc(bop, x[2 * p], x[2 * p + 1]);
#pragma unroll
        for (int jb = 0; jb < JB; ++jb)
          mma32(OW[jb], ld_frag_tr(sV, LDQ, 32 * p + 4 * kg, 32 * p + 16 + 4 * kg, 16 * jb, lane), bop);
      }
  }
  if constexpr (NSH > 1) load_state(rs1, 1);

  // window epilogue: o_swa and lse; OW becomes mix * O_swa, the GLA terms add onto it
  {
    const float l = xor_sum(xor_sum(lpart, 16), 32);
    const float inv = 1.f / l;
    if constexpr (STRONG || CONT) {
      if (qvalid && a.o_swa != nullptr) {
        T* srow = reinterpret_cast<T*>(a.o_swa) + hoff + (size_t)tq * D;
#pragma unroll
        for (int jb = 0; jb < JB; ++jb) {
          const f32x4 y = inv * OW[jb];
          stg4(srow + 16 * jb + 4 * kg, y[0], y[1], y[2], y[3]);
        }
      }
    } else if (a.o_swa != nullptr) {
      // fast path (a continuation writes it directly): o_swa goes to the k^ tile (unused by the
      // window) and leaves from there as whole rows, 16 bytes a lane, once the next barrier has
      // published it
#pragma unroll
      for (int jb = 0; jb < JB; ++jb) {
        const f32x4 y = inv * OW[jb];
        st4(sX + (16 * w + r) * LDQ + 16 * jb + 4 * kg, y[0], y[1], y[2], y[3]);
      }
    }
    if (qvalid && a.lse != nullptr && kg == 0) a.lse[(size_t)bh * L + tq] = (mrun + __log2f(l)) * 0.6931471805599453f;
    const float f = a.mix * inv;
#pragma unroll
    for (int jb = 0; jb < JB; ++jb) OW[jb] *= f;
  }

  // ---- GLA branch
  __syncthreads();   // every wave is done with the last key tile
  if constexpr (!STRONG && !CONT) {
    // o_swa from the k^ tile (the fold writes k^ there only after the gate scan's barrier)
    if (a.o_swa != nullptr) {
#pragma unroll
      for (int u = 0; u < NVT; ++u) {
        const int idx = tid + u * NTHR, row = idx / (D / VEC), cv = idx % (D / VEC);
        if (t0 + row < L)
          *reinterpret_cast<V16*>(reinterpret_cast<T*>(a.o_swa) + hoff + (size_t)(t0 + row) * D + cv * VEC) =
              *reinterpret_cast<const V16*>(sX + row * LDQ + cv * VEC);
      }
    }
  }
  f32x4 sufl[TPT][GV];   // STRONG: block-local exclusive suffixes S of this thread's tokens
  {
    if constexpr (FEAT) {
#pragma unroll
      for (int u = 0; u < TPT; ++u)
#pragma unroll
        for (int e = 0; e < VEC / 4; ++e) {
          const size_t o = hoff + (size_t)min(t0 + tg * TPT + u, L - 1) * D + cg * VEC + 4 * e;
          lqv[u][e] = *reinterpret_cast<const f32x4*>(a.lq + o);
          lkv[u][e] = *reinterpret_cast<const f32x4*>(a.lk + o);
        }
    }
    f32x4 tot[GV];
    f32x4 pinl[TPT][GV];   // STRONG: in-thread inclusive prefixes
    if constexpr (STRONG) {
#pragma unroll
      for (int e = 0; e < GV; ++e) {
        pinl[0][e] = rg[0][e];
#pragma unroll
        for (int u = 1; u < TPT; ++u) pinl[u][e] = pinl[u - 1][e] + rg[u][e];
        sufl[TPT - 1][e] = f32x4{0, 0, 0, 0};
#pragma unroll
        for (int u = TPT - 2; u >= 0; --u) sufl[u][e] = sufl[u + 1][e] + rg[u + 1][e];
      }
    }
    chunk_prefix<D, VEC, NTHR, TPT, GV>(rg, tot, sScan, cg, tg);
    if constexpr (STRONG) {
      // block-local prefixes P (to LDS), suffixes S (kept in registers) and the block totals T
      // (to LDS), from the token groups' totals the prefix left in the scan scratch
      constexpr int GPB = 16 / TPT;               // token groups per 16-token block
      const int blk = tg / GPB, lg = tg % GPB;
#pragma unroll
      for (int e = 0; e < GV; ++e) {
        f32x4 ep = f32x4{0, 0, 0, 0}, es = ep, tb = ep;
#pragma unroll
        for (int j = 0; j < GPB; ++j) {
          const f32x4 o = *reinterpret_cast<const f32x4*>(sScan + (blk * GPB + j) * D + cg * VEC + 4 * e);
          tb += o;
          if (j < lg) ep += o;
          if (j > lg) es += o;
        }
#pragma unroll
        for (int u = 0; u < TPT; ++u) {
          *reinterpret_cast<f32x4*>(sB + (tg * TPT + u) * LDBF + cg * VEC + 4 * e) = pinl[u][e] + ep;
          sufl[u][e] += es;
        }
        if (lg == 0) *reinterpret_cast<f32x4*>(sBT + blk * D + cg * VEC + 4 * e) = tb;
      }
    }
#pragma unroll
    for (int u = 0; u < TPT; ++u) {
      // q~ = q e^b (the inter-chunk operand), and on the fast path k^ = k e^-b
      const bool in = t0 + tg * TPT + u < L;   // rows past the end: -inf, a zero operand as in the raw form
      float qt[VEC], kh[VEC];
#pragma unroll
      for (int e = 0; e < VEC; ++e) {
        const float bb = rg[u][e >> 2][e & 3];
        if constexpr (FEAT) {
          qt[e] = gate_op<true>(in ? lqv[u][e >> 2][e & 3] : -INFINITY, bb);
          if constexpr (!STRONG) kh[e] = gate_op<true>(in ? lkv[u][e >> 2][e & 3] : -INFINITY, -bb);
        } else {
          qt[e] = gate_op<false>(v16_get(rq[u], e, (T*)nullptr), bb);
          if constexpr (!STRONG) kh[e] = gate_op<false>(v16_get(rk[u], e, (T*)nullptr), -bb);
        }
      }
      const int t = tg * TPT + u;
      st_vec(sK + t * LDQ + cg * VEC, qt);
      if constexpr (!STRONG) st_vec(sX + t * LDQ + cg * VEC, kh);
    }
  }
  if constexpr (STRONG) {
    // keys folded to the end of their own block: k e^S, at most |k|
#pragma unroll
    for (int u = 0; u < TPT; ++u) {
      const int t = tg * TPT + u;
      const bool in = t0 + t < L;
      float kh[VEC];
#pragma unroll
      for (int e = 0; e < VEC; ++e) {
        const float x = sufl[u][e >> 2][e & 3];
        if constexpr (FEAT)
          kh[e] = gate_op<true>(in ? lkv[u][e >> 2][e & 3] : -INFINITY, x);
        else
          kh[e] = gate_op<false>(v16_get(rk[u], e, (T*)nullptr), x);
      }
      st_vec(sX + t * LDQ + cg * VEC, kh);
    }
  }
  __syncthreads();   // q~, k^ visible; scan scratch free
  if constexpr (STRONG) {
    // diagonal blocks whose own decay exceeds the factoring's range (bf16) or its accurate range
    // (fp32) take the pairwise form (the barrier before the intra-chunk part publishes it)
    constexpr float kPairSpan = std::is_same<T, float>::value ? 16.f : kStrongGate;
    if (w == 0) {
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) {
        float span = 0.f;
        for (int col = lane; col < D; col += WAVE) span = fmaxf(span, -sBT[kb * D + col]);
        span = wave_max(span);
        if (lane == 0) sPair[kb] = span > kPairSpan ? 1 : 0;
      }
    }
  }
#pragma unroll
  for (int u = 0; u < NVT; ++u) {
    const int idx = tid + u * NTHR, row = idx / (D / VEC), cv = idx % (D / VEC);
    *reinterpret_cast<V16*>(sS + row * LDQ + cv * VEC) = rs0[u];
  }
  __syncthreads();
  {
    // intra-chunk: O^T += V^T (q~ k^T masked)^T
    f32x4 sc[4];
    if constexpr (STRONG) {
      // this wave's queries: block-local gate prefixes and the raw operand (log features) in the
      // operand layout
      f32x4 bq[KS][2];
      float qs[KS][8];
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        bq[ks][0] = ld4f(sB + (16 * w + r) * LDBF + 32 * ks + 8 * kg);
        bq[ks][1] = ld4f(sB + (16 * w + r) * LDBF + 32 * ks + 8 * kg + 4);
        if constexpr (FEAT) {
          const float* lp = a.lq + hoff + (size_t)min(tq, L - 1) * D + 32 * ks + 8 * kg;
          const f32x4 l0 = ld4f(lp), l1 = ld4f(lp + 4);
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            qs[ks][e] = qvalid ? l0[e] : -INFINITY;
            qs[ks][4 + e] = qvalid ? l1[e] : -INFINITY;
          }
        } else {
#pragma unroll
          for (int e = 0; e < 8; ++e) qs[ks][e] = (float)qf[ks][e];
        }
      }
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) {
        sc[kb] = f32x4{0, 0, 0, 0};
        if (kb <= w) {
          if (kb == w && sPair[w] != 0) {
            // exact pairwise scores: query 16w + r against keys 16w + 4kg + i, every column (the
            // same block: b_t - b_s = P_t - P_s)
            const int tl = 16 * w + r;
            const size_t tr = (size_t)min(t0 + tl, L - 1) * D;
            for (int f = 0; f < D; f += 4) {
              const f32x4 bt = ld4f(sB + tl * LDBF + f);
              const f32x4 qv = FEAT ? ld4f(a.lq + hoff + tr + f) : ld4f(q + tr + f);
#pragma unroll
              for (int i = 0; i < 4; ++i) {
                const int sl = 16 * w + 4 * kg + i;
                const size_t sr = (size_t)min(t0 + sl, L - 1) * D;
                const f32x4 bs = ld4f(sB + sl * LDBF + f);
                const f32x4 kv = FEAT ? ld4f(a.lk + hoff + sr + f) : ld4f(k + sr + f);
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                  const float x = fminf(bt[e] - bs[e], 0.f);   // keys after the query are masked below
                  sc[kb][i] += FEAT ? __expf(qv[e] + kv[e] + x) : qv[e] * kv[e] * __expf(x);
                }
              }
            }
          } else {
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
              // b_t - rho_kb: P_t + T_{kb+1} + .. + T_{w-1} below the diagonal, P_t - T_w on it
              f32x4 h[2];
#pragma unroll
              for (int h2 = 0; h2 < 2; ++h2) {
                const int col = 32 * ks + 8 * kg + 4 * h2;
                if (kb < w) {
                  h[h2] = f32x4{0, 0, 0, 0};
                  for (int m = kb + 1; m < w; ++m) h[h2] += ld4f(sBT + m * D + col);
                } else {
                  h[h2] = -ld4f(sBT + w * D + col);
                }
              }
              frag qop;
#pragma unroll
              for (int e = 0; e < 8; ++e)
                set_elem(qop, e, gate_op<FEAT>(qs[ks][e], bq[ks][e >> 2][e & 3] + h[e >> 2][e & 3]));
              mma32(sc[kb], ld_frag(sX, LDQ, 16 * kb + r, 32 * ks + 8 * kg), qop);
            }
          }
          if (kb == w) {
#pragma unroll
            for (int i = 0; i < 4; ++i)
              if (4 * kg + i > r) sc[kb][i] = 0.f;
          }
        }
      }
    } else {
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) {
        sc[kb] = f32x4{0, 0, 0, 0};
        if (kb <= w) {
#pragma unroll
          for (int ks = 0; ks < KS; ++ks)
            mma32(sc[kb], ld_frag(sX, LDQ, 16 * kb + r, 32 * ks + 8 * kg), ld_frag(sK, LDQ, 16 * w + r, 32 * ks + 8 * kg));
          if (kb == w) {
#pragma unroll
            for (int i = 0; i < 4; ++i)
              if (4 * kg + i > r) sc[kb][i] = 0.f;
          }
        }
      }
    }
#pragma unroll
    for (int p = 0; p < 2; ++p)
      if (2 * p <= w) {
        frag bop;
        pack_acc(bop, sc[2 * p], sc[2 * p + 1]);
#pragma unroll
        for (int jb = 0; jb < JB; ++jb)
          mma32(OW[jb], ld_frag_tr(sV, LDQ, 32 * p + 4 * kg, 32 * p + 16 + 4 * kg, 16 * jb, lane), bop);
      }
  }
  // inter-chunk: O^T += S_c^T q~^T, 64 state rows at a time
#pragma unroll
  for (int hs = 0; hs < NSH; ++hs) {
    if (hs > 0) {
      __syncthreads();
#pragma unroll
      for (int u = 0; u < NVT; ++u) {
        const int idx = tid + u * NTHR, row = idx / (D / VEC), cv = idx % (D / VEC);
        *reinterpret_cast<V16*>(sS + row * LDQ + cv * VEC) = rs1[u];
      }
      __syncthreads();
    }
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      const frag fq = ld_frag(sK, LDQ, 16 * w + r, 64 * hs + 32 * ks + 8 * kg);
#pragma unroll
      for (int jb = 0; jb < JB; ++jb)
        mma32(OW[jb], ld_frag_tr(sS, LDQ, 32 * ks + 8 * kg, 32 * ks + 8 * kg + 4, 16 * jb, lane), fq);
    }
  }
  // o (none when the backward recomputes lse and o_swa).  Fast path: through LDS (the value tile is
  // free once every wave's products are done), so that each lane writes 16-byte runs of whole rows;
  // the sub-block path, at its register limit, stores its accumulators directly.
  if constexpr (STRONG) {
    if (qvalid && a.o != nullptr) {
      T* orow = reinterpret_cast<T*>(a.o) + hoff + (size_t)tq * D;
#pragma unroll
      for (int jb = 0; jb < JB; ++jb) stg4(orow + 16 * jb + 4 * kg, OW[jb][0], OW[jb][1], OW[jb][2], OW[jb][3]);
    }
  } else if (a.o != nullptr) {
    __syncthreads();
#pragma unroll
    for (int jb = 0; jb < JB; ++jb)
      st4(sV + (16 * w + r) * LDQ + 16 * jb + 4 * kg, OW[jb][0], OW[jb][1], OW[jb][2], OW[jb][3]);
    __syncthreads();
#pragma unroll
    for (int u = 0; u < NVT; ++u) {
      const int idx = tid + u * NTHR, row = idx / (D / VEC), cv = idx % (D / VEC);
      if (t0 + row < L)
        *reinterpret_cast<V16*>(reinterpret_cast<T*>(a.o) + hoff + (size_t)(t0 + row) * D + cv * VEC) =
            *reinterpret_cast<const V16*>(sV + row * LDQ + cv * VEC);
    }
  }
}

// The fast path: one workgroup per (batch, head, chunk); consecutive chunks of one head share
// an XCD.  Chunks flagged by the sweep go to the dispatch list instead.
template <typename T, int D, bool CONT, bool SG, bool FEAT>
__global__ __launch_bounds__(NTHR, 2) void out_kernel(FwdArgs a, const T* __restrict__ cstates) {
  extern __shared__ __align__(16) unsigned char smem[];
  const int NC = (a.L + C - 1) / C, BH = a.B * a.H;
  int bh, c;
  const int bid = blockIdx.x;
  if ((BH & 7) == 0) {
    const int x = bid % 8, y = bid / 8;
    c = y % NC;
    bh = (y / NC) * 8 + x;
  } else {
    bh = bid / NC;
    c = bid % NC;
  }
  out_chunk<T, D, CONT, SG, FEAT, false>(a, cstates, bh, c, smem, threadIdx.x);
}

// The sub-block path over the dispatch list (persistent workgroups; an empty list ends at once).
template <typename T, int D, bool CONT, bool SG, bool FEAT>
__global__ __launch_bounds__(NTHR, 1) void out_strong_kernel(FwdArgs a, const T* __restrict__ cstates) {
  extern __shared__ __align__(16) unsigned char smem[];
  const int NC = (a.L + C - 1) / C;
  const int n = *a.list_count;
  for (int i = blockIdx.x; i < n; i += gridDim.x) {
    const int id = a.list[i];
    __syncthreads();   // the previous chunk's LDS readers are done
    // the thread index passes through an empty asm so that nothing derived from it is hoisted out
    // of this loop (it would stay live, and spill, across the whole chunk)
    int tid = threadIdx.x;
    asm volatile("" : "+v"(tid));
    out_chunk<T, D, CONT, SG, FEAT, true>(a, cstates, id / NC, id % NC, smem, tid);
  }
}

__global__ void zero_state_kernel(float* p, size_t n) {
  const size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = 0.f;
}

template <typename K>
hipError_t set_lds(K kern, size_t bytes) {
  // every launch: idempotent and cheap, and no process-wide flag to race on
  return hipFuncSetAttribute(reinterpret_cast<const void*>(kern), hipFuncAttributeMaxDynamicSharedMemorySize,
                             (int)bytes);
}

// Workgroups of the sub-block launch: persistent, one per compute unit.
constexpr int kStrongGrid = 256;

template <typename T, int D>
hipError_t launch_fwd_t(const FwdArgs& args, hipStream_t st) {
  using LY = OutLayout<T, D>;
  hipError_t e;
  if (args.L == 0) {
    if (args.state_out != nullptr) {
      const size_t n = (size_t)args.B * args.H * D * D;
      hipLaunchKernelGGL(zero_state_kernel, dim3((n + 255) / 256), dim3(256), 0, st, args.state_out, n);
    }
    return hipGetLastError();
  }
  // workspace: segment buffers of the sweep (when it runs in segments), the strong-gate
  // dispatch, then the chunk states (when they are not an output)
  FwdArgs a = args;
  const int NC = (a.L + C - 1) / C;
  const int NS = sweep_segments(a.B, a.H, a.L, D);
  const size_t segb = fwd_segment_bytes(a.B, a.H, a.L, D);
  unsigned char* ws = reinterpret_cast<unsigned char*>(a.workspace);
  const StrongDispatch sd = dispatch_layout(ws + segb, a.B, a.H, a.L, D);
  a.strong = sd.mask;
  a.list = sd.list;
  a.list_count = sd.count;
  void* states = a.chunk_states != nullptr ? a.chunk_states : ws + segb + dispatch_bytes(a.B, a.H, a.L, D);
  const bool feat = a.lk != nullptr;
  SweepArgs sw{feat ? (const void*)a.lk : a.k, a.v, a.g, nullptr, states, nullptr, a.state_out, a.state_in,
               a.B, a.H, a.L, NS, (NC + NS - 1) / NS, nullptr, nullptr, nullptr, a.gate, feat ? 1 : 0,
               nullptr, nullptr, 0.f, sd.mask, sd.count};
  if (NS > 1) {
    const size_t mat = (size_t)a.B * a.H * NS * D * D * sizeof(float);
    sw.seg_in = reinterpret_cast<float*>(ws);
    sw.seg_fin = reinterpret_cast<float*>(ws + mat);
    sw.seg_gtot = reinterpret_cast<float*>(ws + 2 * mat);
  }
  if ((e = launch_sweep(sw, std::is_same<T, bf16_t>::value ? 1 : 0, D, false, st)) != hipSuccess) return e;
  // variants: continuation (bit 0), scalar gate (bit 1), log features (bit 2; per-dimension gates)
  const int variant = (a.pos != nullptr ? 1 : 0) + (a.gate ? 2 : 0) + (feat ? 4 : 0);
  if (variant >= 6) return hipErrorInvalidValue;
  decltype(&out_kernel<T, D, false, false, false>) kern =
      variant == 0 ? out_kernel<T, D, false, false, false> : variant == 1 ? out_kernel<T, D, true, false, false>
      : variant == 2 ? out_kernel<T, D, false, true, false> : variant == 3 ? out_kernel<T, D, true, true, false>
      : variant == 4 ? out_kernel<T, D, false, false, true> : out_kernel<T, D, true, false, true>;
  decltype(&out_strong_kernel<T, D, false, false, false>) skern =
      variant == 0 ? out_strong_kernel<T, D, false, false, false>
      : variant == 1 ? out_strong_kernel<T, D, true, false, false>
      : variant == 2 ? out_strong_kernel<T, D, false, true, false>
      : variant == 3 ? out_strong_kernel<T, D, true, true, false>
      : variant == 4 ? out_strong_kernel<T, D, false, false, true> : out_strong_kernel<T, D, true, false, true>;
  if ((e = set_lds(kern, LY::bytes)) != hipSuccess) return e;
  if ((e = set_lds(skern, LY::strong_bytes)) != hipSuccess) return e;
  const int nchunks = a.B * a.H * NC;
  hipLaunchKernelGGL(kern, dim3(nchunks), dim3(NTHR), LY::bytes, st, a, (const T*)states);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  hipLaunchKernelGGL(skern, dim3(min(nchunks, kStrongGrid)), dim3(NTHR), LY::strong_bytes, st, a,
                     (const T*)states);
  return hipGetLastError();
}

// After a continued segment: its last min(L, W) keys / values go to ring slots (P + t) mod W.
// Runs after the out kernel has read the old ring (stream order).
template <typename T, int D>
__global__ __launch_bounds__(NTHR) void ring_advance_kernel(FwdArgs a) {
  constexpr int VEC = Tr<T>::VEC;
  const int bh = blockIdx.x, L = a.L, W = a.W;
  const int P = a.pos[bh / a.H];
  const int nw = min(L, W);
  const size_t hoff = (size_t)bh * L * D;
  const T* k = reinterpret_cast<const T*>(a.k) + hoff;
  const T* v = reinterpret_cast<const T*>(a.v) + hoff;
  T* rk = reinterpret_cast<T*>(a.ring_k) + (size_t)bh * W * D;
  T* rv = reinterpret_cast<T*>(a.ring_v) + (size_t)bh * W * D;
  for (int e = threadIdx.x; e < nw * (D / VEC); e += NTHR) {
    const int j = e / (D / VEC), cv = e % (D / VEC);
    const int t = L - nw + j;
    const size_t slot = (size_t)((P + t) % W);
    stg16(rk + slot * D + cv * VEC, ldg16(k + (size_t)t * D + cv * VEC));
    stg16(rv + slot * D + cv * VEC, ldg16(v + (size_t)t * D + cv * VEC));
  }
}

__global__ void pos_advance_kernel(int32_t* pos, int B, int L) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < B) pos[i] += L;
}

template <typename T, int D>
hipError_t launch_fwd_continue_t(const FwdArgs& a, hipStream_t st) {
  if (a.L == 0) return hipSuccess;   // no tokens: state, ring and pos stay as they are
  hipError_t e = launch_fwd_t<T, D>(a, st);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((ring_advance_kernel<T, D>), dim3(a.B * a.H), dim3(NTHR), 0, st, a);
  hipLaunchKernelGGL(pos_advance_kernel, dim3((a.B + 255) / 256), dim3(256), 0, st, a.pos, a.B, a.L);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_fwd_continue(const FwdArgs& a, int dtype, int D, hipStream_t st) {
  if (dtype == 1) {
    if (D == 128) return launch_fwd_continue_t<bf16_t, 128>(a, st);
    if (D == 64) return launch_fwd_continue_t<bf16_t, 64>(a, st);
  } else {
    if (D == 64) return launch_fwd_continue_t<float, 64>(a, st);
  }
  return hipErrorInvalidValue;
}

size_t fwd_segment_bytes(int B, int H, int L, int D) {
  const int NS = sweep_segments(B, H, L, D);
  if (NS <= 1) return 0;
  const size_t mat = (size_t)B * H * NS * D * D * sizeof(float);
  const size_t vec = (size_t)B * H * NS * D * sizeof(float);
  return 2 * mat + (vec + 255) / 256 * 256;
}

size_t dispatch_bytes(int B, int H, int L, int D) {
  const size_t n = (size_t)B * H * ((L + C - 1) / C);
  return 256 + (4 * n + 255) / 256 * 256 + (2 * n * (D / 16) + 255) / 256 * 256;
}

StrongDispatch dispatch_layout(void* base, int B, int H, int L, int D) {
  unsigned char* p = reinterpret_cast<unsigned char*>(base);
  const size_t n = (size_t)B * H * ((L + C - 1) / C);
  StrongDispatch d;
  d.count = reinterpret_cast<int32_t*>(p);
  d.list = reinterpret_cast<int32_t*>(p + 256);
  d.mask = reinterpret_cast<uint16_t*>(p + 256 + (4 * n + 255) / 256 * 256);
  (void)D;
  return d;
}

size_t fwd_aux_bytes(int B, int H, int L, int D) {
  return L > 0 ? fwd_segment_bytes(B, H, L, D) + dispatch_bytes(B, H, L, D) : 0;
}

size_t fwd_workspace_bytes(int B, int H, int L, int D, int dtype) {
  return fwd_aux_bytes(B, H, L, D) + (size_t)B * H * ((L + C - 1) / C) * D * D * (dtype == 1 ? 2 : 4);
}

hipError_t launch_fwd(const FwdArgs& a, int dtype, int D, hipStream_t st) {
  if (dtype == 1) {
    if (D == 128) return launch_fwd_t<bf16_t, 128>(a, st);
    if (D == 64) return launch_fwd_t<bf16_t, 64>(a, st);
  } else if (dtype == 0) {
    if (D == 64) return launch_fwd_t<float, 64>(a, st);
  }
  return hipErrorInvalidValue;
}

}  // namespace lz
