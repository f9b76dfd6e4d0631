// lz_bwd.hip -- backward pass of the Lizard hybrid attention layer on gfx950.
//
// The explainer pages ("Lizard: An Efficient Linearization Framework for
// Large Language Models", gist.science) give no backward; these kernels
// compute the exact gradient of the forward in lz_fwd.hip.  With the gate
// folded into q and k inside each chunk (b = chunk-local inclusive cumsum of
// g, q~ = q e^b, k^ = k e^-b, Gamma = b at the chunk end) the chunk maps
//   O   = (q~ k^T  masked s<=t) V + q~ S_prev,      S = e^Gamma (S_prev + k^T V)
// and, writing dS for dL/dS (from later chunks) and dS' = e^Gamma * dS (rows),
//   dq~ = (dO V^T masked) k^ + dO S_prev^T          dq = dq~ e^b
//   dk^ = (dO V^T masked)^T q~ + V dS'^T            dk = dk^ e^-b
//   dv  = (q~ k^T masked)^T dO + k^ dS'
//   dS_prev = dS' + q~^T dO
//   dg_r = rowsum(S * dS) + sum_{u >= r in chunk} (q~ dq~ - k^ dk^)_u
// Only chunk-local gate sums are exponentiated; the chunk-boundary term of
// dg is the direct rowsum, so no long telescoping sum (which cancels
// catastrophically in low precision) is ever formed.
//
// Kernels, in launch order:
//   sweep_kernel   (lz_sweep.hip) reverse sweep over chunks per (b, h, 64-row
//                  block of dS; with few heads, per sequence segment after a
//                  reduce pass and a reverse scan over the segments): carries
//                  dS in fp32 registers, stores dS' (operand dtype, transposed)
//                  and the fp32 boundary rowsums;
//                  the row blocks of each head also form the window row dots
//                  D_t = mix * dO_t . o_swa_t from the dO rows they stream
//                  (each block a share of the token rows)
//   chunk_kernel   one workgroup per (b, h, chunk): every GLA gradient plus
//                  the anchor-window gradients (query side for dq, key side
//                  for dk and dv) and per-chunk meta-key partial sums
//   dmeta_fold_kernel, dmeta_kernel
//                  deterministic sum of the meta partials over batch and chunks
// With log features (lizard_attn_bwd_feat) the GLA operands are exp(lq + b) and
// exp(lk - b), and the GLA gradients of q and k leave as dlq = q~ dq~ and
// dlk = k^ dk^ (the terms of the gate gradient) instead of joining dq and dk.
#include <type_traits>

#include "lz_common.hpp"
#include "lz_kernels.hpp"

namespace lz {
namespace {

constexpr int C = 64;
constexpr int NTHR = 256;
constexpr int DVTA = 64;   // d_v tile of the state-gradient sweep
constexpr int NTHR_CK = 512;   // chunk kernel: 8 waves, two per token block

size_t round_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

struct WsLayout {
  size_t delta, dS, bnd, dmeta, seg, total;
};

WsLayout ws_layout(int B, int H, int L, int M, int D, int dtype) {
  const size_t NC = (size_t)(L + C - 1) / C;
  const size_t NJ = (size_t)(D + DVTA - 1) / DVTA;
  const size_t esz = dtype == 1 ? 2 : 4;
  WsLayout w{};
  w.delta = 0;
  size_t off = round_up(sizeof(float) * (size_t)B * H * L, 256);
  w.dS = off;
  off += round_up(esz * (size_t)B * H * NC * D * D, 256);
  w.bnd = off;
  off += round_up(sizeof(float) * (size_t)B * H * NC * NJ * D, 256);
  w.dmeta = off;
  off += round_up(sizeof(float) * (size_t)B * NC * H * M * 2 * D, 256);
  w.seg = off;   // segment buffers of the reverse sweep when it runs in segments (few heads)
  off += round_up(fwd_segment_bytes(B, H, L, D), 256);
  w.total = off;
  return w;
}

// ------------------------------------------------------------ chunk kernel
template <typename T, int D>
struct CkLayout {
  static constexpr int PAD = Tr<T>::PAD;
  static constexpr int LDQ = D + PAD;    // row-major [C][D] and [D][D] tiles
  static constexpr int LDB = D + 4;      // fp32 gate-gradient rows
  static constexpr int LDC = C + PAD;    // [16][C] meta tiles
  static constexpr int LDM = 16 + PAD;   // [D][16] meta keys transposed
  static constexpr size_t tile = sizeof(T) * C * LDQ;
  static constexpr size_t oQt = 0;            // q~ ; window: key tile of an earlier chunk
  static constexpr size_t oKh = tile;         // k^ ; window: query tile of a later chunk
  static constexpr size_t oEb = 2 * tile;     // e^b; window: dO tile of a later chunk
  static constexpr size_t odO = 3 * tile;     // dO of this chunk
  static constexpr size_t oV = 4 * tile;      // v of this chunk; window: value tile of an earlier chunk
  static constexpr size_t oBig = 5 * tile;    // dS'^T [D][D] | d b [C][LDB] fp32
  static constexpr size_t bigBytes = sizeof(T) * D * LDQ > sizeof(float) * C * LDB ? sizeof(T) * D * LDQ
                                                                                   : sizeof(float) * C * LDB;
  static constexpr size_t oMkT = oBig + bigBytes;                    // meta keys^T [D][16]
  static constexpr size_t oDLm = oMkT + sizeof(T) * D * LDM;         // dl_meta^T [16][C]
  static constexpr size_t oPm = oDLm + sizeof(T) * 16 * LDC;         // mix * p_meta^T [16][C]
  static constexpr size_t oLse = oPm + sizeof(T) * 16 * LDC;         // lse of 3 chunks (log2 units)
  static constexpr size_t oDel = oLse + sizeof(float) * 3 * C;       // delta of 3 chunks
  static constexpr size_t oBnd = oDel + sizeof(float) * 3 * C;       // boundary term of dg [D]
  static constexpr size_t oTot = oBnd + sizeof(float) * D;           // per-block column totals of d b [4][D]
  static constexpr size_t bytes = oTot + sizeof(float) * 4 * D;
  static_assert(bytes <= 160 * 1024, "LDS budget exceeded");
};

// Four consecutive LDS elements as floats.
__device__ __forceinline__ f32x4 lds4(const float* p) { return *reinterpret_cast<const f32x4*>(p); }
__device__ __forceinline__ f32x4 lds4(const bf16_t* p) {
  const bf16x4 x = *reinterpret_cast<const bf16x4*>(p);
  return f32x4{(float)x[0], (float)x[1], (float)x[2], (float)x[3]};
}

// One workgroup per (b, h, chunk), eight waves in two roles over the four
// 16-token blocks of the chunk: waves 0..3 accumulate dq (GLA and the window
// seen from the query side), waves 4..7 accumulate dk and dv (GLA and the
// window seen from the key side), so every score tile is formed once.
// Accumulators are kept transposed: acc[x][e] belongs to token 16*wb + r of
// the chunk and column 16*x + 4*kg + e.
// SG: one log-gate per head and token (g, dg [B,H,L]).
// FEAT: the GLA branch reads fp32 log features lq, lk (q~ = exp(lq + b), k^ = exp(lk - b)) and
// its q / k gradients leave as dlq = q~ dq~, dlk = k^ dk^; dq, dk keep the window part only.
template <typename T, int D, bool SG, bool FEAT>
__global__ __launch_bounds__(NTHR_CK, 1) void chunk_kernel(BwdArgs a, const T* __restrict__ wsdS,
                                                            const float* __restrict__ wsbnd) {
  using LY = CkLayout<T, D>;
  using frag = typename Tr<T>::frag;
  constexpr int VEC = Tr<T>::VEC;
  constexpr int NB = D / 16;     // 16-wide blocks over the head dim
  constexpr int KS = D / 32;     // K steps over the head dim
  constexpr int NJ = D / DVTA;
  constexpr int LDQ = LY::LDQ, LDB = LY::LDB;

  extern __shared__ __align__(16) unsigned char smem[];
  T* sQt = reinterpret_cast<T*>(smem + LY::oQt);
  T* sKh = reinterpret_cast<T*>(smem + LY::oKh);
  T* sEb = reinterpret_cast<T*>(smem + LY::oEb);
  T* sdO = reinterpret_cast<T*>(smem + LY::odO);
  T* sdSt = reinterpret_cast<T*>(smem + LY::oBig);          // dS' transposed [j][i], row-major
  float* sDb = reinterpret_cast<float*>(smem + LY::oBig);
  T* sV = reinterpret_cast<T*>(smem + LY::oV);
  T* sKw = sQt;    // window: raw keys of chunk kt (query side)
  T* sQw = sKh;    // window: raw queries of chunk qc (key side)
  T* sDw = sEb;    // window: dO of chunk qc > c (key side)
  T* sMkT = reinterpret_cast<T*>(smem + LY::oMkT);
  T* sDLm = reinterpret_cast<T*>(smem + LY::oDLm);
  T* sPm = reinterpret_cast<T*>(smem + LY::oPm);
  float* sLse = reinterpret_cast<float*>(smem + LY::oLse);
  float* sDel = reinterpret_cast<float*>(smem + LY::oDel);
  float* sBnd = reinterpret_cast<float*>(smem + LY::oBnd);
  float* sTot = reinterpret_cast<float*>(smem + LY::oTot);

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, r = lane & 15, kg = lane >> 4;
  const bool qrole = w < 4;        // waves 0..3: dq; waves 4..7: dk, dv
  const int wb = w & 3;            // token block of this wave (rows 16*wb .. +16 of the chunk)
  const int L = a.L, NC = (L + C - 1) / C, W = a.W, M = a.M;
  // workgroup -> (chunk, head); consecutive chunks of one head share an XCD
  const int BH = a.B * a.H;
  int bh, c;
  {
    const int bid = blockIdx.x;
    if ((BH & 7) == 0) {
      const int x = bid % 8, y = bid / 8;           // y runs over (head group, chunk)
      c = y % NC;
      bh = (y / NC) * 8 + x;
    } else {
      bh = bid / NC;
      c = bid % NC;
    }
  }
  const int b = bh / a.H, h = bh % a.H;
  const size_t hoff = (size_t)bh * L * D;
  const T* q = reinterpret_cast<const T*>(a.q) + hoff;
  const T* k = reinterpret_cast<const T*>(a.k) + hoff;
  const T* v = reinterpret_cast<const T*>(a.v) + hoff;
  const T* dO = reinterpret_cast<const T*>(a.dO) + hoff;
  const float* g = a.g + (SG ? (size_t)bh * L : hoff);
  const T* Sprev = reinterpret_cast<const T*>(a.chunk_states) + ((size_t)bh * NC + c) * D * D;
  const T* dSpT = wsdS + ((size_t)bh * NC + c) * D * D;     // dS' transposed [j][i]
  const T* mk = reinterpret_cast<const T*>(a.meta_k) + (size_t)h * M * D;
  const T* mv = a.meta_v ? reinterpret_cast<const T*>(a.meta_v) + (size_t)h * M * D : nullptr;
  const float sl2 = a.scale * LOG2E;
  const float mix = a.mix, scale = a.scale;
  const int t0 = c * C;
  const int u = 16 * wb + r;        // this lane's token within the chunk
  const int tok = t0 + u;


  // Register image of a [C][D] chunk tile: NVT 16-byte vectors per thread.  Rows past the
  // sequence end are loaded clamped (no branch around the load) and zeroed when stored.
  constexpr int NVT = C * (D / VEC) / NTHR_CK;
  auto fetch_rows = [&](V16 (&dst)[NVT], const T* src, int row0) {
#pragma unroll
    for (int e = 0; e < NVT; ++e) {
      const int idx = tid + e * NTHR_CK, t = idx / (D / VEC), cv = idx % (D / VEC);
      dst[e] = ldg16(src + (size_t)min(row0 + t, L - 1) * D + cv * VEC);
    }
  };
  auto put_rows = [&](T* dst, const V16 (&src)[NVT], int row0) {
#pragma unroll
    for (int e = 0; e < NVT; ++e) {
      const int idx = tid + e * NTHR_CK, t = idx / (D / VEC), cv = idx % (D / VEC);
      *reinterpret_cast<V16*>(dst + t * LDQ + cv * VEC) = row0 + t < L ? src[e] : zero16();
    }
  };

  // S_prev rows of the dq waves' inter-chunk product, two K steps ahead: the first two go out
  // last among the staging loads (so nothing in the staging phase waits for them) and arrive
  // during it; each step of the product then issues the rows of the step two ahead.
  auto load_s = [&](frag (&dst)[NB], int ks) {
#pragma unroll
    for (int x = 0; x < NB; ++x) dst[x] = ldg_frag<T>(Sprev + (size_t)(16 * x + r) * D + 32 * ks + 8 * kg);
  };
  frag fs0[NB], fs1[NB];

  // ---------------------------------------------------------------- staging
  // Every load of the staging phase is issued before anything waits on one: no load sits
  // in a branch with its use, so the compiler places no wait between them (each such wait
  // would cost a full memory round trip before the next loads go out).
  {
    // lse / delta of this chunk and the next two (rows clamped into the sequence)
    const int lrow = min(t0 + min(tid, 3 * C - 1), L - 1);
    const float rls = a.lse[(size_t)bh * L + lrow], rdl = a.ws_delta[(size_t)bh * L + lrow];
    // boundary term of dg for this thread's column, per d_v tile (the sweep writes zero for
    // the last chunk); summed when stored
    float bndp[NJ];
#pragma unroll
    for (int j = 0; j < NJ; ++j) bndp[j] = wsbnd[(((size_t)bh * NC + c) * NJ + j) * D + tid % D];
    // meta keys, raw, rows clamped (any valid address when there are none)
    constexpr int NMK = D * 16 / NTHR_CK;          // meta-key elements per thread
    const T* mkp = M > 0 ? mk : q;
    T rmk[NMK];
#pragma unroll
    for (int e = 0; e < NMK; ++e) {
      const int idx = tid + e * NTHR_CK, d = idx / 16, m = idx % 16;
      rmk[e] = mkp[(size_t)min(m, max(M - 1, 0)) * D + d];
    }
    constexpr int NVS = D * (D / VEC) / NTHR_CK;   // dS' vectors per thread
    V16 rds[NVS];
#pragma unroll
    for (int e = 0; e < NVS; ++e) {
      const int idx = tid + e * NTHR_CK, j = idx / (D / VEC), cv = idx % (D / VEC);
      rds[e] = ldg16(dSpT + (size_t)j * D + cv * VEC);
    }
    V16 rdo[NVT], rv[NVT];
    fetch_rows(rdo, dO, t0);
    fetch_rows(rv, v, t0);
    const bool has_strip = w < D / 16;             // wave w folds the gates of columns 16w .. 16w+15
    std::conditional_t<FEAT, GateStripLog<T>, GateStrip<T>> gs;
    if constexpr (FEAT) {
      if (has_strip) gs.template load<SG>(a.lq + hoff, a.lk + hoff, g, D, t0, L, 16 * w + 4 * kg, r);
    } else {
      if (has_strip) gs.template load<SG>(q, k, g, D, t0, L, 16 * w + 4 * kg, r);
    }
    if (qrole) {
      load_s(fs0, 0);
      if (KS > 1) load_s(fs1, 1);
    }
    put_rows(sdO, rdo, t0);
    put_rows(sV, rv, t0);
#pragma unroll
    for (int e = 0; e < NMK; ++e) {
      const int idx = tid + e * NTHR_CK, d = idx / 16, m = idx % 16;
      put_elem(sMkT + d * LY::LDM + m, m < M ? Tr<T>::to_f(rmk[e]) : 0.f);
    }
    if (tid < 3 * C) {
      const bool ok = t0 + tid < L;
      sLse[tid] = ok ? rls * LOG2E : 0.f;
      sDel[tid] = ok ? rdl : 0.f;
    }
    if (tid < D) {
      float bnd = 0.f;
#pragma unroll
      for (int j = 0; j < NJ; ++j) bnd += bndp[j];
      sBnd[tid] = bnd;
    }
    // chunk-local gate prefix b: q~ = q e^b, k^ = k e^-b, e^b
    if (has_strip) gs.fold(sQt, sKh, sEb, LDQ, 16 * w + 4 * kg, r);
#pragma unroll
    for (int e = 0; e < NVS; ++e) {
      const int idx = tid + e * NTHR_CK, j = idx / (D / VEC), cv = idx % (D / VEC);
      *reinterpret_cast<V16*>(sdSt + j * LDQ + cv * VEC) = rds[e];
    }
    __syncthreads();
  }

  // ------------------------------------------------------ GLA gradients
  // Q role: acc0 = dq~.  K role: acc0 = dk^, acc1 = dv.
  f32x4 acc0[NB], acc1[NB];
#pragma unroll
  for (int x = 0; x < NB; ++x) { acc0[x] = f32x4{0, 0, 0, 0}; acc1[x] = acc0[x]; }
  if (qrole) {
    // (the S_prev rows of the first two K steps were issued with the staging loads)
    frag fo[KS];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) fo[ks] = ld_frag(sdO, LDQ, u, 32 * ks + 8 * kg);
    // dA^T blocks (keys of block sb <= wb, queries of block wb), then dq~ += dA k^
    f32x4 blk[4];
#pragma unroll
    for (int sb = 0; sb < 4; ++sb) {
      blk[sb] = f32x4{0, 0, 0, 0};
      if (sb <= wb) {
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) mma32(blk[sb], ld_frag(sV, LDQ, 16 * sb + r, 32 * ks + 8 * kg), fo[ks]);
        mfma_drain();
        if (sb == wb)
#pragma unroll
          for (int i = 0; i < 4; ++i)
            if (4 * kg + i > r) blk[sb][i] = 0.f;
      }
    }
#pragma unroll
    for (int p = 0; p < 2; ++p)
      if (2 * p <= wb) {
        frag op;
        pack_acc(op, blk[2 * p], blk[2 * p + 1]);
#pragma unroll
        for (int x = 0; x < NB; ++x)
          mma32(acc0[x], ld_frag_tr(sKh, LDQ, 32 * p + 4 * kg, 32 * p + 16 + 4 * kg, 16 * x, lane), op);
      }
    // dq~ += dO S_prev^T
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      frag (&cur)[NB] = (ks & 1) ? fs1 : fs0;
#pragma unroll
      for (int x = 0; x < NB; ++x) mma32(acc0[x], cur[x], fo[ks]);
      if (ks + 2 < KS) load_s(cur, ks + 2);
    }
  } else {
    frag fvu[KS], fkh[KS];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      fvu[ks] = ld_frag(sV, LDQ, u, 32 * ks + 8 * kg);
      fkh[ks] = ld_frag(sKh, LDQ, u, 32 * ks + 8 * kg);
    }
    // A blocks (queries of block tb >= wb, keys of block wb): dv += A^T dO
    f32x4 blk[4];
#pragma unroll
    for (int tb = 0; tb < 4; ++tb) {
      blk[tb] = f32x4{0, 0, 0, 0};
      if (tb >= wb) {
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) mma32(blk[tb], ld_frag(sQt, LDQ, 16 * tb + r, 32 * ks + 8 * kg), fkh[ks]);
        mfma_drain();
        if (tb == wb)
#pragma unroll
          for (int i = 0; i < 4; ++i)
            if (4 * kg + i < r) blk[tb][i] = 0.f;
      }
    }
#pragma unroll
    for (int p = 0; p < 2; ++p)
      if (2 * p + 1 >= wb) {
        frag op;
        pack_acc(op, blk[2 * p], blk[2 * p + 1]);
#pragma unroll
        for (int x = 0; x < NB; ++x)
          mma32(acc1[x], ld_frag_tr(sdO, LDQ, 32 * p + 4 * kg, 32 * p + 16 + 4 * kg, 16 * x, lane), op);
      }
    // dA blocks (queries tb >= wb, keys of block wb): dk^ += dA^T q~
#pragma unroll
    for (int tb = 0; tb < 4; ++tb) {
      blk[tb] = f32x4{0, 0, 0, 0};
      if (tb >= wb) {
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) mma32(blk[tb], ld_frag(sdO, LDQ, 16 * tb + r, 32 * ks + 8 * kg), fvu[ks]);
        mfma_drain();
        if (tb == wb)
#pragma unroll
          for (int i = 0; i < 4; ++i)
            if (4 * kg + i < r) blk[tb][i] = 0.f;
      }
    }
#pragma unroll
    for (int p = 0; p < 2; ++p)
      if (2 * p + 1 >= wb) {
        frag op;
        pack_acc(op, blk[2 * p], blk[2 * p + 1]);
#pragma unroll
        for (int x = 0; x < NB; ++x)
          mma32(acc0[x], ld_frag_tr(sQt, LDQ, 32 * p + 4 * kg, 32 * p + 16 + 4 * kg, 16 * x, lane), op);
      }
    // inter-chunk: dk^ += V dS'^T (dS' read down the columns of its transpose) ; dv += k^ dS'
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
#pragma unroll
      for (int x = 0; x < NB; ++x) {
        mma32(acc0[x], ld_frag_tr(sdSt, LDQ, 32 * ks + 8 * kg, 32 * ks + 8 * kg + 4, 16 * x, lane), fvu[ks]);
        mma32(acc1[x], ld_frag(sdSt, LDQ, 16 * x + r, 32 * ks + 8 * kg), fkh[ks]);
      }
    }
  }
  mfma_drain();
  // this lane's window operands: Q role raw q and dO of its query, K role raw k and v of its key
  frag fa[KS], fb[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    fa[ks] = ldg_row_frag<T>(qrole ? q : k, D, tok, 32 * ks + 8 * kg, L);
    fb[ks] = ld_frag(qrole ? sdO : sV, LDQ, u, 32 * ks + 8 * kg);
  }
  // window tiles of the first iteration (raw keys and queries of this chunk; its values and dO are staged)
  V16 pk[NVT], pv[NVT], pq[NVT], pd[NVT];
  fetch_rows(pk, k, t0);
  fetch_rows(pq, q, t0);
  __syncthreads();   // every wave is done with dS': its region now holds the per-token gate gradient

  // gate gradient terms d b_u = q~ dq~ - k^ dk^, then dq = dq~ e^b, dk = dk^ e^-b.  The dq waves
  // hand q~ dq~ over through LDS; the dk/dv waves (same token rows, same lane layout) form d b,
  // take its suffix sums over their 16 tokens in registers and over later blocks through the
  // block totals, add the boundary term and store dg.
  if (qrole) {
#pragma unroll
    for (int x = 0; x < NB; ++x) {
      const int i = 16 * x + 4 * kg;
      const f32x4 qd = lds4(sQt + u * LDQ + i) * acc0[x];
      *reinterpret_cast<f32x4*>(sDb + u * LDB + i) = qd;
      if constexpr (FEAT) {   // dlq = q~ dq~; the window part of dq starts from zero
        if (tok < L) *reinterpret_cast<f32x4*>(a.dlq + hoff + (size_t)tok * D + i) = qd;
        acc0[x] = f32x4{0, 0, 0, 0};
      } else {
        acc0[x] *= lds4(sEb + u * LDQ + i);
      }
    }
  }
  __syncthreads();
  f32x4 db[NB];
  if (!qrole) {
#pragma unroll
    for (int x = 0; x < NB; ++x) {
      const int i = 16 * x + 4 * kg;
      const f32x4 kd = lds4(sKh + u * LDQ + i) * acc0[x];
      db[x] = *reinterpret_cast<const f32x4*>(sDb + u * LDB + i) - kd;
      if constexpr (FEAT) {   // dlk = k^ dk^; the window part of dk starts from zero
        if (tok < L) *reinterpret_cast<f32x4*>(a.dlk + hoff + (size_t)tok * D + i) = kd;
        acc0[x] = f32x4{0, 0, 0, 0};
#pragma unroll
        for (int e = 0; e < 4; ++e) db[x][e] = row_suffix16(db[x][e]);
      } else {
        const f32x4 eb = lds4(sEb + u * LDQ + i);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          acc0[x][e] *= __builtin_amdgcn_rcpf(eb[e]);
          db[x][e] = row_suffix16(db[x][e]);
        }
      }
      if (r == 0) *reinterpret_cast<f32x4*>(sTot + wb * D + i) = db[x];
    }
  }
  __syncthreads();
  if (!qrole) {
    float dsum = 0.f;   // scalar gate: the token's gradient is the sum over the key dimensions
#pragma unroll
    for (int x = 0; x < NB; ++x) {
      const int i = 16 * x + 4 * kg;
      f32x4 carry = *reinterpret_cast<const f32x4*>(sBnd + i);
      for (int b2 = wb + 1; b2 < 4; ++b2) carry += *reinterpret_cast<const f32x4*>(sTot + b2 * D + i);
      const f32x4 dgv = db[x] + carry;
      if constexpr (SG)
        dsum += (dgv[0] + dgv[1]) + (dgv[2] + dgv[3]);
      else if (tok < L)
        *reinterpret_cast<f32x4*>(a.dg + hoff + (size_t)tok * D + i) = dgv;
    }
    if constexpr (SG) {
      dsum = xor_sum(xor_sum(dsum, 16), 32);   // the four column groups of the token
      if (kg == 0 && tok < L) a.dg[(size_t)bh * L + tok] = dsum;
    }
  }
  // (the first window iteration begins with a barrier: d b, q~, k^, e^b are then dead)

  // ----------------------------------------------------------- anchor window
  const bool tvalid = tok < L;
  const float lse2 = sLse[u], delq = sDel[u];
  if (qrole && M > 0) {
    // meta keys (always visible); absent meta values read as zero rows (no branch around the product)
    const T* mvp = mv ? mv : mk;
    const int mvrows = mv ? M : 0;
    f32x4 x = f32x4{0, 0, 0, 0}, dp = f32x4{0, 0, 0, 0};
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      mma32(x, ld_frag_tr(sMkT, LY::LDM, 32 * ks + 8 * kg, 32 * ks + 8 * kg + 4, 0, lane), fa[ks]);
      mma32(dp, ldg_row_frag<T>(mvp, D, r, 32 * ks + 8 * kg, mvrows), fb[ks]);
    }
    mfma_drain();
    f32x4 dl;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int m = 4 * kg + i;
      const float p = (m < M && tvalid) ? fast_exp2(x[i] * sl2 - lse2) : 0.f;
      dl[i] = p * (mix * dp[i] - delq) * scale;
      put_elem(sDLm + m * LY::LDC + u, dl[i]);
      put_elem(sPm + m * LY::LDC + u, p * mix);
    }
    frag op;
    pack_acc(op, dl, f32x4{0, 0, 0, 0});
#pragma unroll
    for (int x2 = 0; x2 < NB; ++x2) mma32(acc0[x2], ld_frag_perm(sMkT, LY::LDM, 16 * x2 + r, 0, 0, kg), op);
  }
  const int kt_lo = max(0, t0 - W + 1) / C;
  const int qc_hi = min(NC - 1, (t0 + C - 1 + W - 1) / C);
  const int n_q = c - kt_lo + 1, n_k = qc_hi - c + 1;
  const int n_it = max(n_q, n_k);
  const int lo = t0 + 16 * wb;                     // first query (Q role) or key (K role) of this wave
  for (int it = 0; it < n_it; ++it) {
    __syncthreads();   // the previous tiles' readers are done
    if (it < n_q) {
      put_rows(sKw, pk, (c - it) * C);
      if (it > 0) put_rows(sV, pv, (c - it) * C);
    }
    if (it < n_k) {
      put_rows(sQw, pq, (c + it) * C);
      if (it > 0) put_rows(sDw, pd, (c + it) * C);
    }
    // next iteration's tiles load while this one is processed
    if (it + 1 < n_q) {
      fetch_rows(pk, k, (c - it - 1) * C);
      fetch_rows(pv, v, (c - it - 1) * C);
    }
    if (it + 1 < n_k) {
      fetch_rows(pq, q, (c + it + 1) * C);
      fetch_rows(pd, dO, (c + it + 1) * C);
    }
    __syncthreads();
    if (qrole) {
      if (it < n_q) {
        // query side: keys of chunk kt, dq += dl K, two 16-key blocks at a time
        const int kbase = (c - it) * C;
#pragma unroll
        for (int p = 0; p < 2; ++p) {
          f32x4 dl[2];
          bool vis[2];
#pragma unroll
          for (int h2 = 0; h2 < 2; ++h2) {
            const int s0 = kbase + 16 * (2 * p + h2);
            vis[h2] = (s0 <= lo + 15) && (s0 + 15 >= lo - W + 1);
          }
          // both blocks of the pair are formed when either is visible (the mask zeroes the
          // other), so their products interleave with one drain
          if (!(vis[0] || vis[1])) continue;
          f32x4 xs[2], dps[2];
#pragma unroll
          for (int h2 = 0; h2 < 2; ++h2) { xs[h2] = f32x4{0, 0, 0, 0}; dps[h2] = xs[h2]; }
#pragma unroll
          for (int ks = 0; ks < KS; ++ks)
#pragma unroll
            for (int h2 = 0; h2 < 2; ++h2) {
              const int kb = 2 * p + h2;
              mma32(xs[h2], ld_frag(sKw, LDQ, 16 * kb + r, 32 * ks + 8 * kg), fa[ks]);
              mma32(dps[h2], ld_frag(sV, LDQ, 16 * kb + r, 32 * ks + 8 * kg), fb[ks]);
            }
          mfma_drain();
#pragma unroll
          for (int h2 = 0; h2 < 2; ++h2) {
            const int kb = 2 * p + h2, s0 = kbase + 16 * kb;
            const f32x4 x = xs[h2], dp = dps[h2];
            // blocks wholly inside the band (every key at or before every query, within the
            // window, queries inside the sequence) need no per-element mask
            const bool full = vis[h2] && s0 + 15 <= lo && lo + 15 - s0 < W && lo + 15 < L;
            if (full) {
#pragma unroll
              for (int i = 0; i < 4; ++i) dl[h2][i] = fast_exp2(x[i] * sl2 - lse2) * (mix * dp[i] - delq) * scale;
            } else {
#pragma unroll
              for (int i = 0; i < 4; ++i) {
                const int s2 = s0 + 4 * kg + i;
                const bool ok = vis[h2] && tvalid && s2 <= tok && s2 > tok - W;
                const float pr = ok ? fast_exp2(x[i] * sl2 - lse2) : 0.f;
                dl[h2][i] = pr * (mix * dp[i] - delq) * scale;
              }
            }
          }
          {
            frag op;
            pack_acc(op, dl[0], dl[1]);
#pragma unroll
            for (int x = 0; x < NB; ++x)
              mma32(acc0[x], ld_frag_tr(sKw, LDQ, 32 * p + 4 * kg, 32 * p + 16 + 4 * kg, 16 * x, lane), op);
          }
        }
      }
    } else {
      if (it < n_k) {
        // key side: queries of chunk qc, dk += dl^T Q, dv += (mix P)^T dO, two 16-query blocks at a time
        const int qc = c + it, qbase = qc * C;
        const T* dOr = it == 0 ? sdO : sDw;
#pragma unroll
        for (int p = 0; p < 2; ++p) {
          f32x4 dl[2], pp[2];
          bool vis[2];
#pragma unroll
          for (int h2 = 0; h2 < 2; ++h2) {
            const int q0 = qbase + 16 * (2 * p + h2);
            vis[h2] = (q0 + 15 >= lo) && (q0 <= lo + 15 + W - 1);
          }
          if (!(vis[0] || vis[1])) continue;
          f32x4 xs[2], dps[2];
#pragma unroll
          for (int h2 = 0; h2 < 2; ++h2) { xs[h2] = f32x4{0, 0, 0, 0}; dps[h2] = xs[h2]; }
#pragma unroll
          for (int ks = 0; ks < KS; ++ks)
#pragma unroll
            for (int h2 = 0; h2 < 2; ++h2) {
              const int tb = 2 * p + h2;
              mma32(xs[h2], ld_frag(sQw, LDQ, 16 * tb + r, 32 * ks + 8 * kg), fa[ks]);
              mma32(dps[h2], ld_frag(dOr, LDQ, 16 * tb + r, 32 * ks + 8 * kg), fb[ks]);
            }
          mfma_drain();
#pragma unroll
          for (int h2 = 0; h2 < 2; ++h2) {
            const int tb = 2 * p + h2, q0 = qbase + 16 * tb;
            const f32x4 x = xs[h2], dp = dps[h2];
            const f32x4 lse4 = lds4(sLse + it * C + 16 * tb + 4 * kg);
            const f32x4 del4 = lds4(sDel + it * C + 16 * tb + 4 * kg);
            // every query of the block at or after every key of this wave, within the window,
            // inside the sequence: no per-element mask
            const bool full = vis[h2] && q0 >= lo + 15 && q0 + 15 - lo < W && q0 + 15 < L;
            if (full) {
#pragma unroll
              for (int i = 0; i < 4; ++i) {
                const float pr = fast_exp2(x[i] * sl2 - lse4[i]);
                pp[h2][i] = pr * mix;
                dl[h2][i] = pr * (mix * dp[i] - del4[i]) * scale;
              }
            } else {
#pragma unroll
              for (int i = 0; i < 4; ++i) {
                const int t = q0 + 4 * kg + i;
                const bool ok = vis[h2] && t < L && tok <= t && tok > t - W;
                const float pr = ok ? fast_exp2(x[i] * sl2 - lse4[i]) : 0.f;
                pp[h2][i] = pr * mix;
                dl[h2][i] = pr * (mix * dp[i] - del4[i]) * scale;
              }
            }
          }
          {
            frag opl, opp;
            pack_acc(opl, dl[0], dl[1]);
            pack_acc(opp, pp[0], pp[1]);
#pragma unroll
            for (int x = 0; x < NB; ++x) {
              mma32(acc0[x], ld_frag_tr(sQw, LDQ, 32 * p + 4 * kg, 32 * p + 16 + 4 * kg, 16 * x, lane), opl);
              mma32(acc1[x], ld_frag_tr(dOr, LDQ, 32 * p + 4 * kg, 32 * p + 16 + 4 * kg, 16 * x, lane), opp);
            }
          }
        }
      }
      // meta partial sums over this chunk's queries: dmk^T = q^T dl_meta, dmv^T = (mix dO)^T p_meta
      if (it == 0 && M > 0) {
        float* dst = a.ws_dmeta + (((size_t)b * NC + c) * a.H + h) * M * 2 * D;
#pragma unroll
        for (int xb = 0; xb < NB / 4; ++xb) {
          const int d0 = 16 * (wb * (NB / 4) + xb);
          f32x4 xk = f32x4{0, 0, 0, 0}, xv = f32x4{0, 0, 0, 0};
#pragma unroll
          for (int ks = 0; ks < C / 32; ++ks) {
            mma32(xk, ld_frag_tr(sQw, LDQ, 32 * ks + 8 * kg, 32 * ks + 8 * kg + 4, d0, lane),
                  ld_frag(sDLm, LY::LDC, r, 32 * ks + 8 * kg));
            mma32(xv, ld_frag_tr(sdO, LDQ, 32 * ks + 8 * kg, 32 * ks + 8 * kg + 4, d0, lane),
                  ld_frag(sPm, LY::LDC, r, 32 * ks + 8 * kg));
          }
          mfma_drain();
          if (r < M)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              dst[(size_t)r * 2 * D + d0 + 4 * kg + i] = xk[i];
              dst[(size_t)r * 2 * D + D + d0 + 4 * kg + i] = xv[i];
            }
        }
      }
    }
  }

  // ------------------------------------------------------------------ store
  mfma_drain();
  if (tvalid) {
    const size_t o = hoff + (size_t)tok * D;
    if (qrole) {
#pragma unroll
      for (int x = 0; x < NB; ++x)
        stg4(reinterpret_cast<T*>(a.dq) + o + 16 * x + 4 * kg, acc0[x][0], acc0[x][1], acc0[x][2], acc0[x][3]);
    } else {
#pragma unroll
      for (int x = 0; x < NB; ++x) {
        stg4(reinterpret_cast<T*>(a.dk) + o + 16 * x + 4 * kg, acc0[x][0], acc0[x][1], acc0[x][2], acc0[x][3]);
        stg4(reinterpret_cast<T*>(a.dv) + o + 16 * x + 4 * kg, acc1[x][0], acc1[x][1], acc1[x][2], acc1[x][3]);
      }
    }
  }
}

// ------------------------------------------------------------ meta reduce
// Two-level deterministic sum of the per-(batch, chunk) meta partials
// part[slot][H*M*2D]: level 1 folds each run of `per` slots into its first
// slot (in place), level 2 sums the run heads in order.
__global__ __launch_bounds__(NTHR) void dmeta_fold_kernel(float* __restrict__ part, int slots, int n, int per) {
  const int e = blockIdx.x * NTHR + threadIdx.x;
  if (e >= n) return;
  const int s0 = blockIdx.y * per, s1 = min(slots, s0 + per);
  float acc = 0.f;
  for (int s = s0; s < s1; ++s) acc += part[(size_t)s * n + e];
  if (s0 < slots) part[(size_t)s0 * n + e] = acc;
}

__global__ __launch_bounds__(NTHR) void dmeta_kernel(const float* __restrict__ part, float* __restrict__ dmk,
                                                      float* __restrict__ dmv, int slots, int per, int n, int D) {
  const int e = blockIdx.x * NTHR + threadIdx.x;   // over H*M*2D
  if (e >= n) return;
  float acc = 0.f;
  for (int s = 0; s < slots; s += per) acc += part[(size_t)s * n + e];
  const int hm = e / (2 * D), col = e % (2 * D);
  if (col < D) dmk[(size_t)hm * D + col] = acc;
  else if (dmv != nullptr) dmv[(size_t)hm * D + col - D] = acc;
}

__global__ void fill_zero_kernel(float* p, size_t n) {
  const size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = 0.f;
}

template <typename K>
hipError_t set_lds(K kern, size_t bytes) {
  return hipFuncSetAttribute(reinterpret_cast<const void*>(kern), hipFuncAttributeMaxDynamicSharedMemorySize,
                             (int)bytes);
}

template <typename T, int D>
hipError_t launch_bwd_t(const BwdArgs& args, hipStream_t st) {
  BwdArgs a = args;
  const int BH = a.B * a.H;
  const int NC = (a.L + C - 1) / C;
  const WsLayout wl = ws_layout(a.B, a.H, a.L, a.M, D, std::is_same<T, bf16_t>::value ? 1 : 0);
  unsigned char* ws = reinterpret_cast<unsigned char*>(a.workspace);
  a.ws_delta = reinterpret_cast<float*>(ws + wl.delta);
  a.ws_dmeta = reinterpret_cast<float*>(ws + wl.dmeta);
  T* wsdS = reinterpret_cast<T*>(ws + wl.dS);
  float* wsbnd = reinterpret_cast<float*>(ws + wl.bnd);
  hipError_t e;
  if (a.L == 0) {
    if (a.M > 0) {
      const size_t n = (size_t)a.H * a.M * D;
      hipLaunchKernelGGL(fill_zero_kernel, dim3((n + 255) / 256), dim3(256), 0, st, a.dmeta_k, n);
      if (a.dmeta_v) hipLaunchKernelGGL(fill_zero_kernel, dim3((n + 255) / 256), dim3(256), 0, st, a.dmeta_v, n);
    }
    return hipGetLastError();
  }
  auto mark = [&](int i) {
    if (a.stage_events != nullptr) (void)hipEventRecord(a.stage_events[i], st);
  };
  mark(0);
  // the state-gradient sweep also forms the window row dots delta_t from the dO rows it streams
  {
    const bool feat = a.lq != nullptr;
    const int NS = sweep_segments(a.B, a.H, a.L, D);
    SweepArgs sw{feat ? (const void*)a.lq : a.q, a.dO, a.g, a.chunk_states, wsdS, wsbnd, nullptr, nullptr,
                 a.B, a.H, a.L, NS, (NC + NS - 1) / NS, nullptr, nullptr, nullptr, a.gate, feat ? 1 : 0, a.o_swa,
                 a.ws_delta, a.mix};
    if (NS > 1) {
      const size_t mat = (size_t)a.B * a.H * NS * D * D * sizeof(float);
      sw.seg_in = reinterpret_cast<float*>(ws + wl.seg);
      sw.seg_fin = reinterpret_cast<float*>(ws + wl.seg + mat);
      sw.seg_gtot = reinterpret_cast<float*>(ws + wl.seg + 2 * mat);
    }
    if ((e = launch_sweep(sw, std::is_same<T, bf16_t>::value ? 1 : 0, D, true, st)) != hipSuccess) return e;
  }
  mark(1);
  {
    using LY = CkLayout<T, D>;
    static bool attr[3] = {false, false, false};   // idempotent; a race only repeats the same call
    const int variant = a.lq != nullptr ? 2 : a.gate ? 1 : 0;   // log features: per-dimension gates only
    auto kern = variant == 2 ? chunk_kernel<T, D, false, true>
              : variant == 1 ? chunk_kernel<T, D, true, false> : chunk_kernel<T, D, false, false>;
    if (!attr[variant]) {
      if ((e = set_lds(kern, LY::bytes)) != hipSuccess) return e;
      attr[variant] = true;
    }
    hipLaunchKernelGGL(kern, dim3(BH * NC), dim3(NTHR_CK), LY::bytes, st, a, (const T*)wsdS, (const float*)wsbnd);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  mark(2);
  if (a.M > 0) {
    const int n = a.H * a.M * 2 * D;
    const int slots = a.B * NC;
    const int runs = slots < 32 ? slots : 32;
    const int per = (slots + runs - 1) / runs;
    hipLaunchKernelGGL(dmeta_fold_kernel, dim3((n + NTHR - 1) / NTHR, runs), dim3(NTHR), 0, st,
                       a.ws_dmeta, slots, n, per);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    hipLaunchKernelGGL(dmeta_kernel, dim3((n + NTHR - 1) / NTHR), dim3(NTHR), 0, st,
                       (const float*)a.ws_dmeta, a.dmeta_k, a.dmeta_v, slots, per, n, D);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  mark(3);
  return hipSuccess;
}

}  // namespace

size_t bwd_workspace_bytes(int B, int H, int L, int M, int D, int dtype) {
  return ws_layout(B, H, L, M, D, dtype).total;
}

hipError_t launch_bwd(const BwdArgs& a, int dtype, int D, hipStream_t st) {
  if (dtype == 1) {
    if (D == 128) return launch_bwd_t<bf16_t, 128>(a, st);
    if (D == 64) return launch_bwd_t<bf16_t, 64>(a, st);
  } else if (dtype == 0) {
    if (D == 64) return launch_bwd_t<float, 64>(a, st);
  }
  return hipErrorInvalidValue;
}

}  // namespace lz
