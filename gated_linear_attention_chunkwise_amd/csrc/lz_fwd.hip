// lz_fwd.hip -- forward pass of the Lizard hybrid attention layer on gfx950.
//
// One workgroup (4 waves) owns one (batch, head, d_v tile) and sweeps the
// sequence in chunks of C = 64 tokens.  Per chunk it computes
//
//   GLA branch (gist.science explainer of "Lizard: An Efficient
//   Linearization Framework for Large Language Models", English page §2.A
//   state update, §2.C log-space gate handling):
//     b_t  = chunk-local inclusive cumulative sum of the log-gates (fp32)
//     q~_t = q_t * exp(b_t),  k^_s = k_s * exp(-b_s)      (gate folded into q, k)
//     O    = (q~ k^T masked s<=t) V  +  q~ S_prev           (bf16 matrix cores)
//     S    = diag(exp(b_end)) * (S_prev + k^T V)           (fp32 state in registers)
//   Only chunk-local sums are exponentiated, so no global cumulative gate
//   (which underflows fp32 at long L) ever appears.
//
//   Anchor window (English page §2.A): online softmax of q_t against the M
//   meta keys and keys s in (t-W, t], meta values optional.  The raw keys
//   and the transposed values of the last three chunks live in LDS rings, so
//   the window reads no global memory; the query operands are issued before
//   the next chunk's prefetch (vector-memory counters retire in order, so a
//   wait on them never waits for the prefetch).
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

constexpr int C = 64;
constexpr int NTHR = 256;

template <typename T, int D, int DVT>
struct FwdLayout {
  static constexpr int PAD = Tr<T>::PAD;
  static constexpr int VEC = Tr<T>::VEC;
  static constexpr int LDQ = D + PAD;     // sQt, sKh, sMk rows
  static constexpr int LDST = D + PAD;    // sSt : [DVT][D]  (transposed state, operand type)
  static constexpr int LDVR = DVT + PAD;  // ring: [3][C][DVT] value tiles, row-major
  static constexpr int LDMV = 16 + PAD;   // sMvt: [DVT][16]
  static constexpr int VPR = D / VEC;     // 16-byte vectors per q/k row
  static constexpr int NTG = NTHR / VPR;  // token groups of the gate scan
  static constexpr int TPT = C / NTG;     // tokens per thread
  static constexpr int GV = VEC / 4;      // float4 gate vectors per (token, column group)
  static constexpr int VVR = DVT / VEC;   // 16-byte vectors per value-row slice
  static constexpr int NVV = (C * VVR + NTHR - 1) / NTHR;
  static constexpr int IB = D / 64;       // state row blocks per wave
  static constexpr int JB = DVT / 16;     // 16-wide d_v blocks
  static constexpr int KS = D / 32;       // K steps over the head dim
  static constexpr size_t oQt = 0;
  static constexpr size_t oKh = oQt + sizeof(T) * C * LDQ;
  static constexpr size_t oSt = oKh + sizeof(T) * C * LDQ;
  static constexpr size_t oRing = oSt + sizeof(T) * DVT * LDST;
  static constexpr size_t oKring = oRing + sizeof(T) * 3 * C * LDVR;   // raw keys of the last 3 chunks [3][C][D]
  static constexpr size_t oMk = oKring + sizeof(T) * 3 * C * LDQ;
  static constexpr size_t oMvt = oMk + sizeof(T) * 16 * LDQ;
  static constexpr size_t oScan = oMvt + sizeof(T) * DVT * LDMV;
  static constexpr size_t oDec = oScan + sizeof(float) * NTG * D;
  static constexpr size_t bytes = oDec + sizeof(float) * D;
  static_assert(bytes <= 160 * 1024, "LDS budget exceeded");
  static_assert(NTG * TPT == C && TPT >= 1, "gate scan thread map");
  static_assert(D % 64 == 0 && DVT % 16 == 0 && DVT <= D, "tile shape");
};

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
  mrun = mnew;
  lpart *= alpha;
#pragma unroll
  for (int j = 0; j < JB; ++j) OW[j] *= alpha;
#pragma unroll
  for (int b = 0; b < NB; ++b)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float p = fast_exp2(x[b][i] - mnew);
      x[b][i] = p;
      lpart += p;
    }
}

template <typename T, int D, int DVT>
__global__ __launch_bounds__(NTHR, 1) void fwd_kernel(FwdArgs a) {
  using LY = FwdLayout<T, D, DVT>;
  using frag = typename Tr<T>::frag;
  constexpr int VEC = LY::VEC, TPT = LY::TPT, GV = LY::GV, JB = LY::JB, KS = LY::KS, IB = LY::IB;
  constexpr int NJ = D / DVT;

  extern __shared__ __align__(16) unsigned char smem[];
  T* sQt = reinterpret_cast<T*>(smem + LY::oQt);
  T* sKh = reinterpret_cast<T*>(smem + LY::oKh);
  T* sSt = reinterpret_cast<T*>(smem + LY::oSt);
  T* sRing = reinterpret_cast<T*>(smem + LY::oRing);
  T* sKring = reinterpret_cast<T*>(smem + LY::oKring);
  T* sMk = reinterpret_cast<T*>(smem + LY::oMk);
  T* sMvt = reinterpret_cast<T*>(smem + LY::oMvt);
  float* sScan = reinterpret_cast<float*>(smem + LY::oScan);
  float* sDec = reinterpret_cast<float*>(smem + LY::oDec);

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int r = lane & 15, kg = lane >> 4;

  // workgroup -> (batch*head, d_v tile); the d_v tiles of one head land on one XCD
  const int BH = a.B * a.H;
  int bh, jt;
  {
    const int bid = blockIdx.x;
    if ((BH & 7) == 0) {
      const int grp = bid / (8 * NJ), x = bid % (8 * NJ);
      bh = grp * 8 + (x & 7);
      jt = x >> 3;
    } else {
      bh = bid / NJ;
      jt = bid % NJ;
    }
  }
  const int h = bh % a.H;
  const int j0 = jt * DVT;
  const int L = a.L;
  const int NC = (L + C - 1) / C;
  const size_t hoff = (size_t)bh * L * D;
  const T* q = reinterpret_cast<const T*>(a.q) + hoff;
  const T* k = reinterpret_cast<const T*>(a.k) + hoff;
  const T* v = reinterpret_cast<const T*>(a.v) + hoff;
  const float* g = a.g + hoff;
  const float sl2 = a.scale * LOG2E;
  const int M = a.M;
  const bool has_mv = a.meta_v != nullptr;   // absent meta values are staged as zeros

  // ---- one-time staging: meta keys / values, zero state
  for (int e = tid; e < 16 * (D / VEC); e += NTHR) {
    const int m = e / (D / VEC), cv = e % (D / VEC);
    V16 x = zero16();
    if (m < M) x = ldg16(reinterpret_cast<const T*>(a.meta_k) + ((size_t)h * M + m) * D + cv * VEC);
    *reinterpret_cast<V16*>(sMk + m * LY::LDQ + cv * VEC) = x;
  }
  for (int e = tid; e < DVT * 16; e += NTHR) {
    const int j = e / 16, m = e % 16;
    float x = 0.f;
    if (has_mv && m < M) x = Tr<T>::to_f(reinterpret_cast<const T*>(a.meta_v)[((size_t)h * M + m) * D + j0 + j]);
    put_elem(sMvt + j * LY::LDMV + m, x);
  }
  for (int e = tid; e < DVT * LY::LDST; e += NTHR) put_elem(sSt + e, 0.f);

  // ---- prefetch registers (thread owns column group cg, tokens tg*TPT .. +TPT)
  const int cg = tid % LY::VPR, tg = tid / LY::VPR;
  V16 rq[TPT], rk[TPT], rv[LY::NVV];
  f32x4 rg[TPT][GV];
  auto prefetch = [&](int c) {
#pragma unroll
    for (int u = 0; u < TPT; ++u) {
      const int t = c * C + tg * TPT + u;
      const bool ok = t < L;
      rq[u] = ok ? ldg16(q + (size_t)t * D + cg * VEC) : zero16();
      rk[u] = ok ? ldg16(k + (size_t)t * D + cg * VEC) : zero16();
#pragma unroll
      for (int e = 0; e < GV; ++e)
        rg[u][e] = ok ? *reinterpret_cast<const f32x4*>(g + (size_t)t * D + cg * VEC + 4 * e) : f32x4{0, 0, 0, 0};
    }
#pragma unroll
    for (int u = 0; u < LY::NVV; ++u) {
      const int idx = tid + u * NTHR;
      rv[u] = zero16();
      if (idx < C * LY::VVR) {
        const int s = idx / LY::VVR, vc = idx % LY::VVR;
        const int t = c * C + s;
        if (t < L) rv[u] = ldg16(v + (size_t)t * D + j0 + vc * VEC);
      }
    }
  };

  f32x4 accS[IB][JB];
#pragma unroll
  for (int i = 0; i < IB; ++i)
#pragma unroll
    for (int j = 0; j < JB; ++j) accS[i][j] = f32x4{0, 0, 0, 0};

  if (NC > 0) prefetch(0);

  for (int c = 0; c < NC; ++c) {
    const int slot = c % 3;
    T* vt_cur = sRing + slot * C * LY::LDVR;
    __syncthreads();   // (1) previous chunk's readers of every staged tile are done

    // (2) value tile and raw keys -> rings (row-major); local gate prefix -> scan scratch
#pragma unroll
    for (int u = 0; u < LY::NVV; ++u) {
      const int idx = tid + u * NTHR;
      if (idx < C * LY::VVR) {
        const int s = idx / LY::VVR, vc = idx % LY::VVR;
        *reinterpret_cast<V16*>(vt_cur + s * LY::LDVR + vc * VEC) = rv[u];
      }
    }
    {
      T* kr = sKring + slot * C * LY::LDQ;
#pragma unroll
      for (int u = 0; u < TPT; ++u) *reinterpret_cast<V16*>(kr + (tg * TPT + u) * LY::LDQ + cg * VEC) = rk[u];
    }
    // this wave's query operands for the window, issued ahead of the next prefetch
    const int tq = c * C + 16 * w + r;
    frag qf[KS];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
      qf[ks] = (tq < L) ? ldg_frag<T>(q + (size_t)tq * D + 32 * ks + 8 * kg) : zero_frag<T>();
#pragma unroll
    for (int u = 1; u < TPT; ++u)
#pragma unroll
      for (int e = 0; e < GV; ++e) rg[u][e] += rg[u - 1][e];
#pragma unroll
    for (int e = 0; e < GV; ++e)
      *reinterpret_cast<f32x4*>(sScan + tg * D + cg * VEC + 4 * e) = rg[TPT - 1][e];
    __syncthreads();   // (4)

    // (5) chunk-local inclusive cumulative log-gate b, gate folded into q and k
    {
      f32x4 excl[GV], tot[GV];
#pragma unroll
      for (int e = 0; e < GV; ++e) { excl[e] = f32x4{0, 0, 0, 0}; tot[e] = f32x4{0, 0, 0, 0}; }
      for (int p = 0; p < LY::NTG; ++p) {
#pragma unroll
        for (int e = 0; e < GV; ++e) {
          const f32x4 x = *reinterpret_cast<const f32x4*>(sScan + p * D + cg * VEC + 4 * e);
          tot[e] += x;
          if (p < tg) excl[e] += x;
        }
      }
      if (tg == 0) {
#pragma unroll
        for (int e = 0; e < GV; ++e)
#pragma unroll
          for (int i = 0; i < 4; ++i) sDec[cg * VEC + 4 * e + i] = __expf(tot[e][i]);
      }
#pragma unroll
      for (int u = 0; u < TPT; ++u) {
        float qt[VEC], kh[VEC];
#pragma unroll
        for (int e = 0; e < VEC; ++e) {
          const float bb = rg[u][e >> 2][e & 3] + excl[e >> 2][e & 3];
          qt[e] = v16_get(rq[u], e, (T*)nullptr) * __expf(bb);
          kh[e] = v16_get(rk[u], e, (T*)nullptr) * __expf(-bb);
        }
        const int t = tg * TPT + u;
        st_vec(sQt + t * LY::LDQ + cg * VEC, qt);
        st_vec(sKh + t * LY::LDQ + cg * VEC, kh);
      }
    }
    if (c + 1 < NC) prefetch(c + 1);
    __syncthreads();   // (6)

    // state entering the first chunk (zero) for the backward pass
    if (c == 0 && a.chunk_states != nullptr) {
      T* dst = reinterpret_cast<T*>(a.chunk_states) + (size_t)bh * NC * D * D;
      for (int e = tid; e < D * DVT; e += NTHR) put_elem(dst + (size_t)(e / DVT) * D + j0 + e % DVT, 0.f);
    }

    const int qlo = c * C + 16 * w;       // first query of this wave
    // (7) GLA: O^T = V^T (q~ k^T masked)^T + S^T q~^T
    f32x4 OG[JB];
#pragma unroll
    for (int j = 0; j < JB; ++j) OG[j] = f32x4{0, 0, 0, 0};
    {
      f32x4 sc[4];
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) {
        sc[kb] = f32x4{0, 0, 0, 0};
        if (kb <= w) {
#pragma unroll
          for (int ks = 0; ks < KS; ++ks)
            mma32(sc[kb], ld_frag(sKh, LY::LDQ, 16 * kb + r, 32 * ks + 8 * kg),
                  ld_frag(sQt, LY::LDQ, 16 * w + r, 32 * ks + 8 * kg));
          mfma_drain();
          if (kb == w) {
#pragma unroll
            for (int i = 0; i < 4; ++i)
              if (4 * kg + i > r) sc[kb][i] = 0.f;
          }
        }
      }
#pragma unroll
      for (int jb = 0; jb < JB; ++jb) {
#pragma unroll
        for (int p = 0; p < 2; ++p) {
          if (2 * p <= w) {
            frag bop;
            pack_acc(bop, sc[2 * p], sc[2 * p + 1]);
            mma32(OG[jb], ld_frag_tr(vt_cur, LY::LDVR, 32 * p + 4 * kg, 32 * p + 16 + 4 * kg, 16 * jb, lane), bop);
          }
        }
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
          mma32(OG[jb], ld_frag(sSt, LY::LDST, 16 * jb + r, 32 * ks + 8 * kg),
                ld_frag(sQt, LY::LDQ, 16 * w + r, 32 * ks + 8 * kg));
      }
    }

    // (8) anchor window: online softmax over meta keys + keys in (t-W, t]
    f32x4 OW[JB];
#pragma unroll
    for (int j = 0; j < JB; ++j) OW[j] = f32x4{0, 0, 0, 0};
    float mrun = -INFINITY, lpart = 0.f;
    if (M > 0) {
      f32x4 xm[1];
      xm[0] = f32x4{0, 0, 0, 0};
#pragma unroll
      for (int ks = 0; ks < KS; ++ks)
        mma32(xm[0], ld_frag(sMk, LY::LDQ, r, 32 * ks + 8 * kg), qf[ks]);
#pragma unroll
      for (int i = 0; i < 4; ++i) xm[0][i] = (4 * kg + i < M) ? xm[0][i] * sl2 : -INFINITY;
      mfma_drain();
      absorb<1, JB>(xm, mrun, lpart, OW);
      {   // meta values (zero-filled in LDS when absent: no branch around the product)
        frag bop;
        pack_acc(bop, xm[0], f32x4{0, 0, 0, 0});
#pragma unroll
        for (int jb = 0; jb < JB; ++jb) mma32(OW[jb], ld_frag_perm(sMvt, LY::LDMV, 16 * jb + r, 0, 0, kg), bop);
      }
      mfma_drain();
    }

    const int kt_lo = max(0, c * C - a.W + 1) / C;   // oldest key tile any query of the chunk sees
    for (int kt = c; kt >= kt_lo; --kt) {
      const int kbase = kt * C;
      const T* vt = sRing + (kt % 3) * C * LY::LDVR;
      const T* kt_rows = sKring + (kt % 3) * C * LY::LDQ;
      f32x4 x[4];
      bool vis[4];
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) {
        const int s0 = kbase + 16 * kb;
        vis[kb] = (s0 <= qlo + 15) && (s0 + 15 >= qlo - a.W + 1);
        x[kb] = f32x4{0, 0, 0, 0};
        if (vis[kb]) {
#pragma unroll
          for (int ks = 0; ks < KS; ++ks)
            mma32(x[kb], ld_frag(kt_rows, LY::LDQ, 16 * kb + r, 32 * ks + 8 * kg), qf[ks]);
          mfma_drain();
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int s = s0 + 4 * kg + i;
          const bool ok = vis[kb] && s <= tq && s > tq - a.W;
          x[kb][i] = ok ? x[kb][i] * sl2 : -INFINITY;
        }
      }
      absorb<4, JB>(x, mrun, lpart, OW);
#pragma unroll
      for (int jb = 0; jb < JB; ++jb)
#pragma unroll
        for (int p = 0; p < 2; ++p)
          if (vis[2 * p] || vis[2 * p + 1]) {
            frag bop;
            pack_acc(bop, x[2 * p], x[2 * p + 1]);
            mma32(OW[jb], ld_frag_tr(vt, LY::LDVR, 32 * p + 4 * kg, 32 * p + 16 + 4 * kg, 16 * jb, lane), bop);
          }
    }

    // (9) epilogue: o = O_gla + mix * O_swa / l, optional lse and o_swa
    mfma_drain();
    {
      float l = xor_sum(xor_sum(lpart, 16), 32);
      const float inv = 1.f / l;
      if (tq < L) {
        T* orow = reinterpret_cast<T*>(a.o) + hoff + (size_t)tq * D + j0;
#pragma unroll
        for (int jb = 0; jb < JB; ++jb) {
          const f32x4 y = OG[jb] + (a.mix * inv) * OW[jb];
          stg4(orow + 16 * jb + 4 * kg, y[0], y[1], y[2], y[3]);
        }
        if (a.o_swa != nullptr) {
          T* srow = reinterpret_cast<T*>(a.o_swa) + hoff + (size_t)tq * D + j0;
#pragma unroll
          for (int jb = 0; jb < JB; ++jb) {
            const f32x4 y = inv * OW[jb];
            stg4(srow + 16 * jb + 4 * kg, y[0], y[1], y[2], y[3]);
          }
        }
        if (a.lse != nullptr && jt == 0 && kg == 0)
          a.lse[(size_t)bh * L + tq] = (mrun + __log2f(l)) * 0.6931471805599453f;
      }
    }

    // (10)/(11) state update S <- diag(exp b_end) (S + k^ T V); needed unless this is the last chunk
    const bool need_state = (c + 1 < NC) || (a.state_out != nullptr);
    if (need_state) {
      __syncthreads();   // every wave is done reading sSt
#pragma unroll
      for (int ib = 0; ib < IB; ++ib) {
        const int i0 = 16 * (w * IB + ib);
        float dec[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) dec[i] = sDec[i0 + 4 * kg + i];
#pragma unroll
        for (int jb = 0; jb < JB; ++jb) {
#pragma unroll
          for (int ks = 0; ks < C / 32; ++ks)
            mma32(accS[ib][jb], ld_frag_tr(sKh, LY::LDQ, 32 * ks + 8 * kg, 32 * ks + 8 * kg + 4, i0, lane),
                  ld_frag_tr(vt_cur, LY::LDVR, 32 * ks + 8 * kg, 32 * ks + 8 * kg + 4, 16 * jb, lane));
#pragma unroll
          for (int i = 0; i < 4; ++i) accS[ib][jb][i] *= dec[i];
          st4(sSt + (16 * jb + r) * LY::LDST + i0 + 4 * kg, accS[ib][jb][0], accS[ib][jb][1],
              accS[ib][jb][2], accS[ib][jb][3]);
          // state entering the next chunk, row-major [d_k][d_v], for the backward pass
          if (a.chunk_states != nullptr && c + 1 < NC) {
            T* dst = reinterpret_cast<T*>(a.chunk_states) + ((size_t)bh * NC + c + 1) * D * D + j0 + 16 * jb + r;
#pragma unroll
            for (int i = 0; i < 4; ++i) put_elem(dst + (size_t)(i0 + 4 * kg + i) * D, accS[ib][jb][i]);
          }
        }
      }
    }
  }

  if (a.state_out != nullptr) {
    float* so = a.state_out + (size_t)bh * D * D;
#pragma unroll
    for (int ib = 0; ib < IB; ++ib) {
      const int i0 = 16 * (w * IB + ib);
#pragma unroll
      for (int jb = 0; jb < JB; ++jb)
#pragma unroll
        for (int i = 0; i < 4; ++i) so[(size_t)(i0 + 4 * kg + i) * D + j0 + 16 * jb + r] = accS[ib][jb][i];
    }
  }
}

template <typename T, int D, int DVT>
hipError_t launch_fwd_t(const FwdArgs& a, hipStream_t st) {
  using LY = FwdLayout<T, D, DVT>;
  auto kern = fwd_kernel<T, D, DVT>;
  static bool attr_set = false;   // idempotent; a race only repeats the same call
  if (!attr_set) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)LY::bytes);
    if (e != hipSuccess) return e;
    attr_set = true;
  }
  const int grid = a.B * a.H * (D / DVT);
  hipLaunchKernelGGL(kern, dim3(grid), dim3(NTHR), LY::bytes, st, a);
  return hipGetLastError();
}

template <typename T, int D>
hipError_t launch_fwd_d(const FwdArgs& a, hipStream_t st) {
  // widest d_v tile (64 for bf16, 32 for fp32: LDS) that still gives >= 240 workgroups
  const long bh = (long)a.B * a.H;
  if constexpr (!std::is_same<T, float>::value) {
    if (bh * (D / 64) >= 240) return launch_fwd_t<T, D, 64>(a, st);
  }
  if (bh * (D / 32) >= 240) return launch_fwd_t<T, D, 32>(a, st);
  return launch_fwd_t<T, D, 16>(a, st);
}

}  // namespace

hipError_t launch_fwd(const FwdArgs& a, int dtype, int D, hipStream_t st) {
  if (dtype == 1) {
    if (D == 128) return launch_fwd_d<bf16_t, 128>(a, st);
    if (D == 64) return launch_fwd_d<bf16_t, 64>(a, st);
  } else if (dtype == 0) {
    if (D == 64) return launch_fwd_d<float, 64>(a, st);
  }
  return hipErrorInvalidValue;
}

}  // namespace lz
