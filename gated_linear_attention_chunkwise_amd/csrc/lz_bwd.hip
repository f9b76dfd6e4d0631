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
//   dmeta_sum_kernel
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
  size_t delta, dS, bnd, dmeta, seg, disp, total;
  // recompute (lse, o_swa or chunk_states not given): the forward's workspace (its chunk
  // states at its end), lse and o_swa, after `total`
  size_t rc_fwd, rc_lse, rc_oswa, rc_total;
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
  w.disp = off;  // strong-gate dispatch: masks, list
  off += dispatch_bytes(B, H, L, D);
  w.total = off;
  w.rc_fwd = off;
  off += round_up(fwd_workspace_bytes(B, H, L, D, dtype), 256);
  w.rc_lse = off;
  off += round_up(sizeof(float) * (size_t)B * H * L, 256);
  w.rc_oswa = off;
  off += round_up(esz * (size_t)B * H * L * D, 256);
  w.rc_total = off;
  return w;
}

// ------------------------------------------------------------ chunk kernel
template <typename T, int D, bool STRONG = false>
struct CkLayout {
  static constexpr int PAD = Tr<T>::PAD;
  static constexpr int LDQ = D + PAD;    // row-major [C][D] and [D][D] tiles
  static constexpr int LDB = D + 4;      // fp32 gate-gradient rows
  static constexpr int LDC = C + PAD;    // [16][C] meta tiles
  static constexpr int LDM = 16 + PAD;   // [D][16] meta keys transposed
  static constexpr size_t tile = sizeof(T) * C * LDQ;
  static constexpr int NT = STRONG ? 4 : 5;   // [C][D] tiles (the sub-block path keeps no e^b)
  static constexpr size_t oQt = 0;            // q~ (sub-block path: raw q); window: key tile of an earlier chunk
  static constexpr size_t oKh = tile;         // k^ (sub-block path: keys folded to their block end);
                                              // window: query tile of a later chunk
  static constexpr size_t oEb = 2 * tile;     // fast path: e^b; window: dO tile of a later chunk
  static constexpr size_t odO = (NT - 2) * tile;   // dO of this chunk
  static constexpr size_t oV = (NT - 1) * tile;    // v of this chunk; window: value tile of an earlier chunk
  static constexpr size_t oBig = NT * tile;   // dS'^T [D][D] | d b [C][LDB] fp32
  static constexpr size_t bigBytes = sizeof(T) * D * LDQ > sizeof(float) * C * LDB ? sizeof(T) * D * LDQ
                                                                                   : sizeof(float) * C * LDB;
  static constexpr size_t oBnd = oBig + bigBytes;                    // boundary term of dg [D]
  static constexpr size_t oTot = oBnd + sizeof(float) * D;           // per-block column totals of d b [4][D]
  // window-phase tiles; on the fast path they share their region with S_prev [D][D] (row-major),
  // staged once for the dq waves' inter-chunk product and dead after the GLA part
  static constexpr size_t oWin = oTot + sizeof(float) * 4 * D;
  static constexpr size_t oSp = oWin;                                // fast path: S_prev
  static constexpr size_t oMkT = oWin;                               // meta keys^T [D][16]
  static constexpr size_t oDLm = oMkT + sizeof(T) * D * LDM;         // dl_meta^T [16][C]
  static constexpr size_t oPm = oDLm + sizeof(T) * 16 * LDC;         // mix * p_meta^T [16][C]
  static constexpr size_t oLse = oPm + sizeof(T) * 16 * LDC;         // lse of 3 query chunks (log2 units)
  static constexpr size_t oDel = oLse + sizeof(float) * 3 * C;       // delta of 3 query chunks
  static constexpr size_t win_end = oDel + sizeof(float) * 3 * C;
  static constexpr size_t sp_end = oSp + sizeof(T) * D * LDQ;
  static constexpr size_t fast_end = STRONG || win_end > sp_end ? win_end : sp_end;
  // sub-block path: fp32 block-local gate prefixes [C][LDBF] (the window's dO tile of a later
  // chunk afterwards), the 16-token block totals [4][D], the strips' largest in-block decays [D/16][4]
  static constexpr int LDBF = D + 4;
  static constexpr size_t oB = fast_end;
  static constexpr size_t oBT = oB + sizeof(float) * C * LDBF;
  static constexpr size_t oSpan = oBT + sizeof(float) * 4 * D;
  static constexpr size_t bytes = STRONG ? oSpan + sizeof(float) * 4 * (D / 16) : fast_end;
  static constexpr size_t oDw = STRONG ? oB : oEb;                  // window: dO tile of a later chunk
  static_assert(sizeof(float) * C * LDBF >= tile, "dO tile fits the prefix area");
  static_assert(bytes <= 160 * 1024, "LDS budget exceeded");
};

__device__ __forceinline__ void set_elem(bf16x8& f, int e, float x) { f[e] = (__bf16)x; }
__device__ __forceinline__ void set_elem(f32x8& f, int e, float x) { f[e] = x; }
// The value an operand of type T holds for x (bf16 rounding, or none).
template <typename T>
__device__ __forceinline__ float rnd_op(float x) {
  if constexpr (std::is_same<T, bf16_t>::value)
    return (float)(__bf16)x;
  else
    return x;
}
// One term q_t k_s e^(b_t - b_s) of a pairwise score (x = b_t - b_s), raw or log features.
template <bool FEAT>
__device__ __forceinline__ float pair_term(float qv, float kv, float x) {
  if constexpr (FEAT)
    return __expf(qv + kv + x);
  else
    return qv * kv * __expf(x);
}


// One workgroup per (b, h, chunk), eight waves in two roles over the four
// 16-token blocks of the chunk: waves 0..3 accumulate dq (GLA and the window
// seen from the query side), waves 4..7 accumulate dk and dv (GLA and the
// window seen from the key side).  Each side forms the score tiles it needs
// once for all output columns (dA and the window scores are formed on both
// sides; split by output columns, every wave would form every tile).
// Accumulators are kept transposed: acc[x][e] belongs to token 16*wb + r of
// the chunk and column 16*x + 4*kg + e.
// SG: one log-gate per head and token (g, dg [B,H,L]).
// FEAT: the GLA branch reads fp32 log features lq, lk (q~ = exp(lq + b), k^ = exp(lk - b)) and
// its q / k gradients leave as dlq = q~ dq~, dlk = k^ dk^; dq, dk keep the window part only.
// STRONG: the GLA part by 16-token blocks, for chunks whose gates are too strong for the
// chunk-start factoring (see out_chunk in lz_fwd.hip): the score of query t (block tb) against key
// s (block sb <= tb) is formed from q e^(b_t - rho_sb) and k e^(rho_sb - b_s), rho_sb = b at the
// last token of block sb; a diagonal block whose own decay exceeds the factoring's range is
// formed pairwise.
// Every pair's operand values are the same on the query side (dq, q-terms of d b) and the key
// side (dk, dv, k-terms of d b), so the chunk-local sums of d b cancel as on the fast path.  The
// inter-chunk terms use k e^(gamma - b) against the stored state gradient, gamma = Gamma in the
// columns the sweep stored undecayed and 0 elsewhere.
// Without STRONG, a chunk flagged by the sweep is appended to the dispatch list and left.
template <typename T, int D, bool SG, bool FEAT, bool STRONG>
__device__ __forceinline__ void chunk_body(const BwdArgs& a, const T* __restrict__ wsdS,
                                           const float* __restrict__ wsbnd, int bh, int c, unsigned char* smem,
                                           int tid) {
  using LY = CkLayout<T, D, STRONG>;
  using frag = typename Tr<T>::frag;
  constexpr int VEC = Tr<T>::VEC;
  constexpr int NB = D / 16;     // 16-wide blocks over the head dim
  constexpr int KS = D / 32;     // K steps over the head dim
  constexpr int NJ = D / DVTA;
  constexpr int LDQ = LY::LDQ, LDB = LY::LDB, LDBF = LY::LDBF;

  T* sQt = reinterpret_cast<T*>(smem + LY::oQt);
  T* sKh = reinterpret_cast<T*>(smem + LY::oKh);
  T* sEb = reinterpret_cast<T*>(smem + LY::oEb);
  T* sdO = reinterpret_cast<T*>(smem + LY::odO);
  T* sdSt = reinterpret_cast<T*>(smem + LY::oBig);          // dS' transposed [j][i], row-major
  float* sDb = reinterpret_cast<float*>(smem + LY::oBig);
  T* sV = reinterpret_cast<T*>(smem + LY::oV);
  T* sKw = sQt;    // window: raw keys of chunk kt (query side)
  T* sQw = sKh;    // window: raw queries of chunk qc (key side)
  T* sDw = reinterpret_cast<T*>(smem + LY::oDw);    // window: dO of chunk qc > c (key side)
  T* sMkT = reinterpret_cast<T*>(smem + LY::oMkT);
  T* sDLm = reinterpret_cast<T*>(smem + LY::oDLm);
  T* sPm = reinterpret_cast<T*>(smem + LY::oPm);
  float* sLse = reinterpret_cast<float*>(smem + LY::oLse);
  float* sDel = reinterpret_cast<float*>(smem + LY::oDel);
  float* sBnd = reinterpret_cast<float*>(smem + LY::oBnd);
  float* sTot = reinterpret_cast<float*>(smem + LY::oTot);
  T* sSp = reinterpret_cast<T*>(smem + LY::oSp);                 // fast path only
  float* sB = reinterpret_cast<float*>(smem + LY::oB);         // STRONG only
  float* sBT = reinterpret_cast<float*>(smem + LY::oBT);       // STRONG only
  float* sSpan = reinterpret_cast<float*>(smem + LY::oSpan);   // STRONG only

  const int lane = tid & 63, w = tid >> 6, r = lane & 15, kg = lane >> 4;
  const bool qrole = w < 4;        // waves 0..3: dq; waves 4..7: dk, dv
  const int wb = w & 3;            // token block of this wave (rows 16*wb .. +16 of the chunk)
  const int L = a.L, NC = (L + C - 1) / C, W = a.W, M = a.M;
  // the sweep's strong-column masks of this chunk (bit i: column i was stored undecayed)
  uint64_t sm0, sm1 = 0;
  {
    const uint64_t* mp = reinterpret_cast<const uint64_t*>(a.strong + ((size_t)bh * NC + c) * (D / 16));
    sm0 = mp[0];
    if constexpr (D == 128) sm1 = mp[1];
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

  // Sub-block path: S_prev rows of the dq waves' inter-chunk product, two K steps ahead: the first
  // two go out last among the staging loads (so nothing in the staging phase waits for them) and
  // arrive during it; each step of the product then issues the rows of the step two ahead.  (The
  // fast path stages S_prev in LDS once for all four dq waves.)
  auto load_s = [&](frag (&dst)[NB], int ks) {
#pragma unroll
    for (int x = 0; x < NB; ++x) dst[x] = ldg_frag<T>(Sprev + (size_t)(16 * x + r) * D + 32 * ks + 8 * kg);
  };
  frag fs0[NB], fs1[NB];

  // fast path: the window phase's lse / delta rows and raw meta keys (one 16-byte vector of
  // meta_k [16][D] per dq lane, rows clamped; any valid address when there are none) come with
  // the staging loads and wait in the dq waves' registers until the hand-over, when S_prev's LDS
  // region is free
  constexpr int NMV = 16 * (D / VEC);
  static_assert(NMV <= 4 * 64, "one meta-key vector per dq lane");
  float wls = 0.f, wdl = 0.f;
  V16 wmk = zero16();

  // ---------------------------------------------------------------- staging
  // Every load of the staging phase is issued before anything waits on one: no load sits
  // in a branch with its use, so the compiler places no wait between them (each such wait
  // would cost a full memory round trip before the next loads go out).
  {
    constexpr int NMK = D * 16 / NTHR_CK;          // meta-key elements per thread
    // issued in the order of their use: the gate strips' q, k, g (the fold goes first), dO and v,
    // then the rest, so that the fold runs while the later loads are still in flight
    const bool has_strip = w < D / 16;             // wave w folds the gates of columns 16w .. 16w+15
    std::conditional_t<FEAT, GateStripLog<T>, GateStrip<T>> gs;
    if constexpr (FEAT) {
      if (has_strip) gs.template load<SG>(a.lq + hoff, a.lk + hoff, g, D, t0, L, 16 * w + 4 * kg, r);
    } else {
      if (has_strip) gs.template load<SG>(q, k, g, D, t0, L, 16 * w + 4 * kg, r);
    }
    V16 rdo[NVT], rv[NVT];
    fetch_rows(rdo, dO, t0);
    fetch_rows(rv, v, t0);
    // sub-block path: lse / delta of this chunk and the next two (rows clamped into the sequence)
    // and the raw meta keys (rows clamped; any valid address when there are none)
    float rls = 0.f, rdl = 0.f;
    T rmk[NMK];
    if constexpr (STRONG) {
      const int lrow = min(t0 + min(tid, 3 * C - 1), L - 1);
      rls = a.lse[(size_t)bh * L + lrow];
      rdl = a.ws_delta[(size_t)bh * L + lrow];
      const T* mkp = M > 0 ? mk : q;
#pragma unroll
      for (int e = 0; e < NMK; ++e) {
        const int idx = tid + e * NTHR_CK, d = idx / 16, m = idx % 16;
        rmk[e] = mkp[(size_t)min(m, max(M - 1, 0)) * D + d];
      }
    }
    // boundary term of dg for this thread's column, per d_v tile (the sweep writes zero for
    // the last chunk); summed when stored
    float bndp[NJ];
#pragma unroll
    for (int j = 0; j < NJ; ++j) bndp[j] = wsbnd[(((size_t)bh * NC + c) * NJ + j) * D + tid % D];
    constexpr int NVS = D * (D / VEC) / NTHR_CK;   // [D][D] vectors per thread
    V16 rds[NVS];
#pragma unroll
    for (int e = 0; e < NVS; ++e) {
      const int idx = tid + e * NTHR_CK, j = idx / (D / VEC), cv = idx % (D / VEC);
      rds[e] = ldg16(dSpT + (size_t)j * D + cv * VEC);
    }
    if constexpr (!STRONG) {
      if (qrole) {
        const int lrow = min(t0 + min(tid, 3 * C - 1), L - 1);
        wls = a.lse[(size_t)bh * L + lrow];
        wdl = a.ws_delta[(size_t)bh * L + lrow];
        const int mi = min(tid, NMV - 1), m = mi % 16, cv = mi / 16;
        wmk = ldg16((M > 0 ? mk : q) + (size_t)min(m, max(M - 1, 0)) * D + cv * VEC);
      }
    }
    // fast path: S_prev once for all four dq waves (the sub-block path loads fragments per wave)
    V16 rsp[STRONG ? 1 : NVS];
    if constexpr (!STRONG) {
#pragma unroll
      for (int e = 0; e < NVS; ++e) {
        const int idx = tid + e * NTHR_CK, i = idx / (D / VEC), cv = idx % (D / VEC);
        rsp[e] = ldg16(Sprev + (size_t)i * D + cv * VEC);
      }
    }
    if constexpr (STRONG) {
      if (qrole) {
        load_s(fs0, 0);
        if (KS > 1) load_s(fs1, 1);
      }
    }
    if constexpr (!STRONG) {
      if ((sm0 | sm1) != 0) {   // the sub-block launch takes this chunk
        if (tid == 0) a.list[atomicAdd(a.list_count, 1)] = bh * NC + c;
        return;
      }
    }
    // chunk-local gate prefix b: q~ = q e^b, k^ = k e^-b, e^b (sub-block path: b, rho, raw q and
    // keys folded to the end of their block)
    if (has_strip) {
      if constexpr (STRONG)
        gs.fold_strong(sQt, sKh, LDQ, sB, LDBF, sBT, D, sSpan + 4 * w, 16 * w + 4 * kg, r, lane);
      else
        gs.fold(sQt, sKh, sEb, LDQ, 16 * w + 4 * kg, r);
    }
    put_rows(sdO, rdo, t0);
    put_rows(sV, rv, t0);
    if constexpr (STRONG) {
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
    }
    if (tid < D) {
      float bnd = 0.f;
#pragma unroll
      for (int j = 0; j < NJ; ++j) bnd += bndp[j];
      sBnd[tid] = bnd;
    }
#pragma unroll
    for (int e = 0; e < NVS; ++e) {
      const int idx = tid + e * NTHR_CK, j = idx / (D / VEC), cv = idx % (D / VEC);
      *reinterpret_cast<V16*>(sdSt + j * LDQ + cv * VEC) = rds[e];
      if constexpr (!STRONG) *reinterpret_cast<V16*>(sSp + j * LDQ + cv * VEC) = rsp[e];
    }
    __syncthreads();
  }

  // ------------------------------------------------------ GLA gradients
  // Q role: acc0 = dq~.  K role: acc0 = dk^, acc1 = dv.
  f32x4 acc0[NB], acc1[NB];
#pragma unroll
  for (int x = 0; x < NB; ++x) { acc0[x] = f32x4{0, 0, 0, 0}; acc1[x] = acc0[x]; }
  f32x4 dbs[NB];   // sub-block path: this lane's gate-gradient terms (q side or k side)
  if constexpr (STRONG) {
    // Exponents come from block-local sums only (sB: P, the inclusive prefix inside each 16-token
    // block; sBT: the block totals T), never as differences of chunk-cumulative sums, so that
    // each is as accurate as its own size.  Relative to the end of key block j, query t of block
    // i > j has exponent b_t - rho_j = P_t + T_{j+1} + .. + T_{i-1}; key s of block j has
    // rho_j - b_s = T_j - P_s.  The pairwise form sums the gates between key and query directly.
    // Diagonal blocks formed pairwise: those whose own decay exceeds the factoring's range (bf16)
    // or its accurate range (fp32); the same decision in every wave.
    constexpr float kPairSpan = std::is_same<T, float>::value ? 16.f : kStrongGate;
    int prm = 0;   // bit kb: diagonal block kb is formed pairwise
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
      float m = 0.f;
      for (int w2 = 0; w2 < D / 16; ++w2) m = fmaxf(m, sSpan[4 * w2 + kb]);
      if (m > kPairSpan) prm |= 1 << kb;
    }
    const bool prw = (prm >> wb) & 1;   // this wave's diagonal block
    // raw GLA operands (log features) of chunk row `row`, columns col .. col+3; rows past the
    // end give zero operands (log features: -inf)
    auto qraw4 = [&](int row, int col) -> f32x4 {
      if constexpr (FEAT) {
        if (t0 + row >= L) return f32x4{-INFINITY, -INFINITY, -INFINITY, -INFINITY};
        return ld4f(a.lq + hoff + (size_t)(t0 + row) * D + col);
      } else {
        return ld4f(sQt + row * LDQ + col);   // the raw-q tile (zero rows past the end)
      }
    };
    auto qraw1 = [&](int row, int col) -> float {
      if constexpr (FEAT)
        return t0 + row < L ? a.lq[hoff + (size_t)(t0 + row) * D + col] : -INFINITY;
      else
        return Tr<T>::to_f(sQt[row * LDQ + col]);
    };
    auto kraw4 = [&](int row, int col) -> f32x4 {
      if constexpr (FEAT) {
        if (t0 + row >= L) return f32x4{-INFINITY, -INFINITY, -INFINITY, -INFINITY};
        return ld4f(a.lk + hoff + (size_t)(t0 + row) * D + col);
      } else {
        if (t0 + row >= L) return f32x4{0, 0, 0, 0};
        return ld4f(k + (size_t)(t0 + row) * D + col);
      }
    };
    // the log-gates of chunk row `row` (zero past the end; a scalar gate broadcast)
    auto graw4 = [&](int row, int col) -> f32x4 {
      if (t0 + row >= L) return f32x4{0, 0, 0, 0};
      if constexpr (SG) {
        const float x = g[t0 + row];
        return f32x4{x, x, x, x};
      } else {
        return ld4f(g + (size_t)(t0 + row) * D + col);
      }
    };
    // T_{j0} + .. + T_{j1} (zero when j0 > j1), four columns or one
    auto bsum4 = [&](int j0, int j1, int col) {
      f32x4 z = f32x4{0, 0, 0, 0};
      for (int m = j0; m <= j1; ++m) z += ld4f(sBT + m * D + col);
      return z;
    };
    auto bsum1 = [&](int j0, int j1, int col) {
      float z = 0.f;
      for (int m = j0; m <= j1; ++m) z += sBT[m * D + col];
      return z;
    };
#pragma unroll
    for (int x = 0; x < NB; ++x) dbs[x] = f32x4{0, 0, 0, 0};
    if (qrole) {
      frag fo[KS];
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) fo[ks] = ld_frag(sdO, LDQ, u, 32 * ks + 8 * kg);
      // inter-chunk first (the prefetched S_prev rows are then free): Y = dO S_prev^T, the
      // gradient of q~ = q e^b, b_t = T_0 + .. + T_{wb-1} + P_t
      f32x4 Y[NB];
#pragma unroll
      for (int x = 0; x < NB; ++x) Y[x] = f32x4{0, 0, 0, 0};
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        frag (&cur)[NB] = (ks & 1) ? fs1 : fs0;
#pragma unroll
        for (int x = 0; x < NB; ++x) mma32(Y[x], cur[x], fo[ks]);
        if (ks + 2 < KS) load_s(cur, ks + 2);
      }
#pragma unroll
      for (int x = 0; x < NB; ++x) {
        const int col = 16 * x + 4 * kg;
        const f32x4 bt = bsum4(0, wb - 1, col) + ld4f(sB + u * LDBF + col), qv = qraw4(u, col);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          dbs[x][e] += rnd_op<T>(gate_op<FEAT>(qv[e], bt[e])) * Y[x][e];
          if constexpr (!FEAT) acc0[x][e] += __expf(bt[e]) * Y[x][e];
        }
      }
      // dA^T blocks (keys of block sb <= wb, queries of block wb)
      f32x4 blk[4];
#pragma unroll
      for (int sb = 0; sb < 4; ++sb) {
        blk[sb] = f32x4{0, 0, 0, 0};
        if (sb <= wb) {
#pragma unroll
          for (int ks = 0; ks < KS; ++ks) mma32(blk[sb], ld_frag(sV, LDQ, 16 * sb + r, 32 * ks + 8 * kg), fo[ks]);
          if (sb == wb)
#pragma unroll
            for (int i = 0; i < 4; ++i)
              if (4 * kg + i > r) blk[sb][i] = 0.f;
        }
      }
      // acc0: raw dq.  Per key block: X = dA k'' (k'' = k e^(rho_sb - b)), then the query factor
      // e^(b_t - rho_sb) turns it into dq and the operand value q e^(b_t - rho_sb) into d b terms
#pragma unroll
      for (int sb = 0; sb < 4; ++sb) {
        if (sb > wb) continue;
        if (sb == wb && prw) {
          // pairwise: e^(g_{s+1} + .. + g_t), the sum formed going back from the query;
          // dA[this query][key 16 sb + s2] sits in lane r + 16 (s2 / 4), slot s2 % 4
#pragma unroll
          for (int x = 0; x < NB; ++x) {
            const int col = 16 * x + 4 * kg;
            const f32x4 qv = qraw4(u, col);
            f32x4 run = f32x4{0, 0, 0, 0};
#pragma unroll 1
            for (int s2 = 15; s2 >= 0; --s2) {
              if (s2 < r) run += graw4(16 * sb + s2 + 1, col);   // keys after the query carry dA = 0
              const float dAv = __shfl(blk[sb][s2 & 3], r + 16 * (s2 >> 2), WAVE);
              const f32x4 kv = kraw4(16 * sb + s2, col);
#pragma unroll
              for (int e = 0; e < 4; ++e) {
                dbs[x][e] += dAv * pair_term<FEAT>(qv[e], kv[e], run[e]);
                if constexpr (!FEAT) acc0[x][e] += dAv * (kv[e] * __expf(run[e]));
              }
            }
          }
        } else {
          f32x4 X[NB];
#pragma unroll
          for (int x = 0; x < NB; ++x) X[x] = f32x4{0, 0, 0, 0};
          frag op;
          pack_acc(op, blk[sb], f32x4{0, 0, 0, 0});
#pragma unroll
          for (int x = 0; x < NB; ++x)
            mma32(X[x], ld_frag_tr(sKh, LDQ, 16 * sb + 4 * kg, 16 * sb + 4 * kg, 16 * x, lane), op);
#pragma unroll
          for (int x = 0; x < NB; ++x) {
            const int col = 16 * x + 4 * kg;
            // b_t - rho_sb: P_t + T_{sb+1} + .. + T_{wb-1} below the diagonal, P_t - T_wb on it
            const f32x4 pt = ld4f(sB + u * LDBF + col), qv = qraw4(u, col);
            const f32x4 xb = sb < wb ? pt + bsum4(sb + 1, wb - 1, col) : pt - ld4f(sBT + wb * D + col);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              dbs[x][e] += rnd_op<T>(gate_op<FEAT>(qv[e], xb[e])) * X[x][e];
              if constexpr (!FEAT) acc0[x][e] += __expf(xb[e]) * X[x][e];
            }
          }
        }
      }
    } else {
      // inter-chunk with k e^(gamma - b) against the stored state gradient (gamma = Gamma in the
      // columns stored undecayed, 0 in the others): Gamma - b_s = (T_wb - P_s) + T_{wb+1} + .. + T_3,
      // -b_s = -(T_0 + .. + T_{wb-1} + P_s); dk part V dS^T, dv += k e^(gamma - b) dS
      auto kexp4 = [&](int col) {
        const f32x4 ps = ld4f(sB + u * LDBF + col);
        const f32x4 ks = ld4f(sBT + wb * D + col) - ps + bsum4(wb + 1, 3, col);
        const f32x4 kw = -(bsum4(0, wb - 1, col) + ps);
        f32x4 z;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int cc = col + e;
          z[e] = ((cc < 64 ? sm0 >> cc : sm1 >> (cc - 64)) & 1ull) ? ks[e] : kw[e];
        }
        return z;
      };
      // inter-chunk dv first, while no other accumulator is live: dv += k e^(gamma - b) dS, the key
      // operand formed one K step at a time
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        frag fki;
        const int col = 32 * ks + 8 * kg;
#pragma unroll
        for (int h2 = 0; h2 < 2; ++h2) {
          const f32x4 xk = kexp4(col + 4 * h2), kv = kraw4(u, col + 4 * h2);
#pragma unroll
          for (int e = 0; e < 4; ++e) set_elem(fki, 4 * h2 + e, gate_op<FEAT>(kv[e], xk[e]));
        }
#pragma unroll
        for (int x = 0; x < NB; ++x) mma32(acc1[x], ld_frag(sdSt, LDQ, 16 * x + r, 32 * ks + 8 * kg), fki);
      }
      frag fkh[KS];
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) fkh[ks] = ld_frag(sKh, LDQ, u, 32 * ks + 8 * kg);
      // exponent of query row `row` (block tb >= wb) against this key block's end: b_t - rho_wb
      auto qexp1 = [&](int row, int col) {
        const int tb = row >> 4;
        const float pt = sB[row * LDBF + col];
        return tb > wb ? pt + bsum1(wb + 1, tb - 1, col) : pt - sBT[wb * D + col];
      };
      auto qop_row = [&](int row, int ks) {
        frag f;
        const int col = 32 * ks + 8 * kg, tb = row >> 4;
#pragma unroll
        for (int h2 = 0; h2 < 2; ++h2) {
          const int c4 = col + 4 * h2;
          const f32x4 pt = ld4f(sB + row * LDBF + c4), qv = qraw4(row, c4);
          const f32x4 xb = tb > wb ? pt + bsum4(wb + 1, tb - 1, c4) : pt - ld4f(sBT + wb * D + c4);
#pragma unroll
          for (int e = 0; e < 4; ++e) set_elem(f, 4 * h2 + e, gate_op<FEAT>(qv[e], xb[e]));
        }
        return f;
      };
      // A blocks (queries of block tb >= wb, keys of block wb): dv += A^T dO
      f32x4 blk[4];
#pragma unroll
      for (int tb = 0; tb < 4; ++tb) {
        blk[tb] = f32x4{0, 0, 0, 0};
        if (tb >= wb) {
          if (tb == wb && prw) {
            // pairwise: this key against queries 16 tb + 4 kg + i, every column (P_t - P_s: the
            // same block)
#pragma unroll 1
            for (int f = 0; f < D; f += 4) {
              const f32x4 bs = ld4f(sB + u * LDBF + f), kv = kraw4(u, f);
#pragma unroll
              for (int i = 0; i < 4; ++i) {
                const int tr = 16 * tb + 4 * kg + i;
                const f32x4 bt = ld4f(sB + tr * LDBF + f), qv = qraw4(tr, f);
#pragma unroll
                for (int e = 0; e < 4; ++e) blk[tb][i] += pair_term<FEAT>(qv[e], kv[e], fminf(bt[e] - bs[e], 0.f));
              }
            }
          } else {
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) mma32(blk[tb], qop_row(16 * tb + r, ks), fkh[ks]);
          }
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
      // dA blocks (queries tb >= wb, keys of block wb)
#pragma unroll
      for (int tb = 0; tb < 4; ++tb) {
        blk[tb] = f32x4{0, 0, 0, 0};
        if (tb >= wb) {
#pragma unroll
          for (int ks = 0; ks < KS; ++ks)
            mma32(blk[tb], ld_frag(sdO, LDQ, 16 * tb + r, 32 * ks + 8 * kg), ld_frag(sV, LDQ, u, 32 * ks + 8 * kg));
          if (tb == wb)
#pragma unroll
            for (int i = 0; i < 4; ++i)
              if (4 * kg + i < r) blk[tb][i] = 0.f;
        }
      }
      // dk'' += dA^T q' over the other blocks (q' of queries before this key block is zero)
#pragma unroll
      for (int p = 0; p < 2; ++p)
        if (2 * p + 1 >= wb) {
          f32x4 b0 = blk[2 * p], b1 = blk[2 * p + 1];
          if (prw) {
            if (2 * p == wb) b0 = f32x4{0, 0, 0, 0};
            if (2 * p + 1 == wb) b1 = f32x4{0, 0, 0, 0};
          }
          frag op;
          pack_acc(op, b0, b1);
#pragma unroll
          for (int x = 0; x < NB; ++x) {
            const int col = 16 * x + r;
            frag qa;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
              const int row = 32 * p + (e < 4 ? 0 : 16) + 4 * kg + (e & 3);
              const bool use = row >= 16 * wb && !(prw && (row >> 4) == wb);
              set_elem(qa, e, use ? gate_op<FEAT>(qraw1(row, col), qexp1(row, col)) : 0.f);
            }
            mma32(acc0[x], qa, op);
            __builtin_amdgcn_sched_barrier(0);   // one operand's loads at a time (register pressure)
          }
        }
      // intra-chunk k side: terms of d b from k'', then acc0 turns from dk'' into the raw dk,
      // dk = dk'' e^(T_wb - P_s) (at most 1); log features keep no GLA part in dk
#pragma unroll
      for (int x = 0; x < NB; ++x) {
        const int col = 16 * x + 4 * kg;
        const f32x4 kpp = ld4f(sKh + u * LDQ + col);
        const f32x4 xs = ld4f(sBT + wb * D + col) - ld4f(sB + u * LDBF + col);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          dbs[x][e] += kpp[e] * acc0[x][e];
          acc0[x][e] = FEAT ? 0.f : __expf(xs[e]) * acc0[x][e];
        }
      }
      if (prw) {
        // pairwise diagonal block (its dA was left out above): dk and the k-side terms directly, e^(g_{s+1} + .. + g_t) with
        // the sum formed going forward from the key; dA[query 16 wb + t2][this key] sits in lane
        // r + 16 (t2 / 4), slot t2 % 4
        const f32x4 dAq = blk[wb];
#pragma unroll
        for (int x = 0; x < NB; ++x) {
          const int col = 16 * x + 4 * kg;
          const f32x4 kv = kraw4(u, col);
          f32x4 run = f32x4{0, 0, 0, 0};
#pragma unroll 1
          for (int t2 = 0; t2 < 16; ++t2) {
            if (t2 > r) run += graw4(16 * wb + t2, col);   // queries before the key carry dA = 0
            const float dAv = __shfl(dAq[t2 & 3], r + 16 * (t2 >> 2), WAVE);
            const f32x4 qv = qraw4(16 * wb + t2, col);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              dbs[x][e] += dAv * pair_term<FEAT>(qv[e], kv[e], run[e]);
              if constexpr (!FEAT) acc0[x][e] += dAv * (qv[e] * __expf(run[e]));
            }
          }
        }
      }
      // inter-chunk dk (the dv part went first): V dS^T, one 16-column block at a time, straight
      // into d b and dk.  This key's raw values come in once, packed (their loads would otherwise
      // be hoisted out of the loop in fp32 and spill).
      using R4 = decltype(ld4raw(static_cast<const T*>(nullptr)));
      R4 kr[NB];
      const bool kin = t0 + u < L;
#pragma unroll
      for (int x = 0; x < NB; ++x) kr[x] = ld4raw(k + (size_t)min(t0 + u, L - 1) * D + 16 * x + 4 * kg);
#pragma unroll
      for (int x = 0; x < NB; ++x) {
        f32x4 y = f32x4{0, 0, 0, 0};
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
          mma32(y, ld_frag_tr(sdSt, LDQ, 32 * ks + 8 * kg, 32 * ks + 8 * kg + 4, 16 * x, lane),
                ld_frag(sV, LDQ, u, 32 * ks + 8 * kg));
        const int col = 16 * x + 4 * kg;
        f32x4 kv;
        if constexpr (FEAT) {
          kv = kraw4(u, col);
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e) kv[e] = kin ? (float)kr[x][e] : 0.f;
        }
        const f32x4 xk = kexp4(col);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          dbs[x][e] += rnd_op<T>(gate_op<FEAT>(kv[e], xk[e])) * y[e];
          if constexpr (!FEAT) acc0[x][e] += __expf(xk[e]) * y[e];
        }
      }
    }
  } else if (qrole) {
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
    for (int ks = 0; ks < KS; ++ks)
#pragma unroll
      for (int x = 0; x < NB; ++x) mma32(acc0[x], ld_frag(sSp, LDQ, 16 * x + r, 32 * ks + 8 * kg), fo[ks]);
  } else {
    frag fvu[KS], fkh[KS];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      fvu[ks] = ld_frag(sV, LDQ, u, 32 * ks + 8 * kg);
      fkh[ks] = ld_frag(sKh, LDQ, u, 32 * ks + 8 * kg);
    }
    // (the intra-chunk dv product, A^T dO, waits for the hand-over below)
    f32x4 blk[4];
    // dA blocks (queries tb >= wb, keys of block wb): dk^ += dA^T q~
#pragma unroll
    for (int tb = 0; tb < 4; ++tb) {
      blk[tb] = f32x4{0, 0, 0, 0};
      if (tb >= wb) {
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) mma32(blk[tb], ld_frag(sdO, LDQ, 16 * tb + r, 32 * ks + 8 * kg), fvu[ks]);
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
      f32x4 qd;
      if constexpr (STRONG)
        qd = dbs[x];   // (acc0 already holds the raw dq)
      else
        qd = ld4f(sQt + u * LDQ + i) * acc0[x];
      *reinterpret_cast<f32x4*>(sDb + u * LDB + i) = qd;
      if constexpr (FEAT) {   // dlq = q~ dq~; the window part of dq starts from zero
        if (tok < L) *reinterpret_cast<f32x4*>(a.dlq + hoff + (size_t)tok * D + i) = qd;
        acc0[x] = f32x4{0, 0, 0, 0};
      } else if constexpr (!STRONG) {
        acc0[x] *= ld4f(sEb + u * LDQ + i);
      }
    }
  }
  if constexpr (!STRONG) {
    if (!qrole) {
      // intra-chunk dv += A^T dO (A blocks: queries of block tb >= wb, keys of block wb), while the
      // dq waves hand their terms over (q~, k^ and dO stay in LDS until the window phase)
      frag fkh[KS];
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) fkh[ks] = ld_frag(sKh, LDQ, u, 32 * ks + 8 * kg);
      f32x4 blk[4];
#pragma unroll
      for (int tb = 0; tb < 4; ++tb) {
        blk[tb] = f32x4{0, 0, 0, 0};
        if (tb >= wb) {
#pragma unroll
          for (int ks = 0; ks < KS; ++ks) mma32(blk[tb], ld_frag(sQt, LDQ, 16 * tb + r, 32 * ks + 8 * kg), fkh[ks]);
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
    }
  }
  __syncthreads();
  if constexpr (!STRONG) {
    if (qrole) {   // the window phase's tiles (S_prev is dead; the next barrier publishes them)
      if (tid < NMV) {   // consecutive lanes, consecutive meta rows: adjacent LDS halfwords
        const int m = tid % 16, cv = tid / 16;
#pragma unroll
        for (int e = 0; e < VEC; ++e)
          put_elem(sMkT + (cv * VEC + e) * LY::LDM + m, m < M ? v16_get(wmk, e, (T*)nullptr) : 0.f);
      }
      if (tid < 3 * C) {
        const bool ok = t0 + tid < L;
        sLse[tid] = ok ? wls * LOG2E : 0.f;
        sDel[tid] = ok ? wdl : 0.f;
      }
    }
  }
  f32x4 db[NB];
  if (!qrole) {
#pragma unroll
    for (int x = 0; x < NB; ++x) {
      const int i = 16 * x + 4 * kg;
      f32x4 kd;
      if constexpr (STRONG)
        kd = dbs[x];   // (acc0 already holds the raw dk)
      else
        kd = ld4f(sKh + u * LDQ + i) * acc0[x];
      db[x] = *reinterpret_cast<const f32x4*>(sDb + u * LDB + i) - kd;
      if constexpr (FEAT || STRONG) {   // dlk = k^ dk^; the window part of dk starts from zero
        if constexpr (FEAT) {
          if (tok < L) *reinterpret_cast<f32x4*>(a.dlk + hoff + (size_t)tok * D + i) = kd;
          acc0[x] = f32x4{0, 0, 0, 0};
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) db[x][e] = row_suffix16(db[x][e]);
      } else {
        const f32x4 eb = ld4f(sEb + u * LDQ + i);
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
    if constexpr (STRONG) {
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
    } else {
      // the boundary term plus the totals of the later blocks: every total is read and weighted
      // by an exact 0 or 1 (a loop over wb + 1 .. 3, or a branch per block, would wait on each
      // read), and all column blocks are summed before any store (the sub-block kernel, at its
      // register limit, keeps the loop above)
      const float w1 = wb < 1 ? 1.f : 0.f, w2 = wb < 2 ? 1.f : 0.f, w3 = wb < 3 ? 1.f : 0.f;
#pragma unroll
      for (int x = 0; x < NB; ++x) {
        const int i = 16 * x + 4 * kg;
        f32x4 carry = *reinterpret_cast<const f32x4*>(sBnd + i);
        carry += w1 * *reinterpret_cast<const f32x4*>(sTot + D + i);
        carry += w2 * *reinterpret_cast<const f32x4*>(sTot + 2 * D + i);
        carry += w3 * *reinterpret_cast<const f32x4*>(sTot + 3 * D + i);
        db[x] += carry;
      }
      // (raw per-dimension gates: dg goes to its own rows of the gate-gradient area, which every
      // other wave has read by now, and leaves as whole rows in the window's first iteration)
#pragma unroll
      for (int x = 0; x < NB; ++x) {
        const int i = 16 * x + 4 * kg;
        if constexpr (SG)
          dsum += (db[x][0] + db[x][1]) + (db[x][2] + db[x][3]);
        else if constexpr (!FEAT)
          *reinterpret_cast<f32x4*>(sDb + u * LDB + i) = db[x];
        else if (tok < L)
          *reinterpret_cast<f32x4*>(a.dg + hoff + (size_t)tok * D + i) = db[x];
      }
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
    // meta keys (always visible) and, when given, meta values
    f32x4 x = f32x4{0, 0, 0, 0}, dp = f32x4{0, 0, 0, 0};
    if constexpr (STRONG) {
      // absent meta values read as zero rows (no branch around the product)
      const T* mvp = mv ? mv : mk;
      const int mvrows = mv ? M : 0;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        mma32(x, ld_frag_tr(sMkT, LY::LDM, 32 * ks + 8 * kg, 32 * ks + 8 * kg + 4, 0, lane), fa[ks]);
        mma32(dp, ldg_row_frag<T>(mvp, D, r, 32 * ks + 8 * kg, mvrows), fb[ks]);
      }
    } else {
#pragma unroll
      for (int ks = 0; ks < KS; ++ks)
        mma32(x, ld_frag_tr(sMkT, LY::LDM, 32 * ks + 8 * kg, 32 * ks + 8 * kg + 4, 0, lane), fa[ks]);
      if (mv != nullptr) {
        // meta values (absent ones add nothing to dp); rows clamped and zeroed past M, with no
        // branch around the loads (each such branch ends in a wait for every load in flight)
        frag fmv[KS];
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
          fmv[ks] = ldg_frag<T>(mv + (size_t)min(r, M - 1) * D + 32 * ks + 8 * kg);
          if (r >= M) fmv[ks] = zero_frag<T>();
        }
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) mma32(dp, fmv[ks], fb[ks]);
      }
    }
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
  // lse / delta of query chunk c + it sit in slot it % 3: the staging phase filled the first
  // three, a window reaching further refills a slot once its previous chunk is done
  float nls = 0.f, ndl = 0.f;
  for (int it = 0; it < n_it; ++it) {
    __syncthreads();   // the previous tiles' readers are done
    if constexpr (!STRONG && !SG && !FEAT) {
      if (it == 0) {
        // dg of this chunk from the gate-gradient area: 16 bytes a lane, whole rows
        constexpr int NDG = C * D / 4 / NTHR_CK;
#pragma unroll
        for (int e = 0; e < NDG; ++e) {
          const int idx = tid + e * NTHR_CK, row = idx / (D / 4), c4 = idx % (D / 4);
          if (t0 + row < L)
            *reinterpret_cast<f32x4*>(a.dg + hoff + (size_t)(t0 + row) * D + 4 * c4) =
                *reinterpret_cast<const f32x4*>(sDb + row * LDB + 4 * c4);
        }
      }
    }
    if (it < n_q) {
      put_rows(sKw, pk, (c - it) * C);
      if (it > 0) put_rows(sV, pv, (c - it) * C);
    }
    if (it < n_k) {
      put_rows(sQw, pq, (c + it) * C);
      if (it > 0) put_rows(sDw, pd, (c + it) * C);
      if (it >= 3 && tid < C) {
        const bool ok = (c + it) * C + tid < L;
        sLse[(it % 3) * C + tid] = ok ? nls * LOG2E : 0.f;
        sDel[(it % 3) * C + tid] = ok ? ndl : 0.f;
      }
    }
    // next iteration's tiles load while this one is processed
    if (it + 1 < n_q) {
      fetch_rows(pk, k, (c - it - 1) * C);
      fetch_rows(pv, v, (c - it - 1) * C);
    }
    if (it + 1 < n_k) {
      fetch_rows(pq, q, (c + it + 1) * C);
      fetch_rows(pd, dO, (c + it + 1) * C);
      if (it + 1 >= 3 && tid < C) {
        const int row = min((c + it + 1) * C + tid, L - 1);
        nls = a.lse[(size_t)bh * L + row];
        ndl = a.ws_delta[(size_t)bh * L + row];
      }
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
#pragma unroll
          for (int h2 = 0; h2 < 2; ++h2) {
            const int tb = 2 * p + h2, q0 = qbase + 16 * tb;
            const f32x4 x = xs[h2], dp = dps[h2];
            const f32x4 lse4 = ld4f(sLse + (it % 3) * C + 16 * tb + 4 * kg);
            const f32x4 del4 = ld4f(sDel + (it % 3) * C + 16 * tb + 4 * kg);
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
      // (the latter only with meta values: each partial holds M rows of MW columns)
      if (it == 0 && M > 0) {
        const int MW = mv != nullptr ? 2 * D : D;
        float* dst = a.ws_dmeta + (((size_t)b * NC + c) * a.H + h) * M * MW;
#pragma unroll
        for (int xb = 0; xb < NB / 4; ++xb) {
          const int d0 = 16 * (wb * (NB / 4) + xb);
          f32x4 xk = f32x4{0, 0, 0, 0}, xv = f32x4{0, 0, 0, 0};
#pragma unroll
          for (int ks = 0; ks < C / 32; ++ks)
            mma32(xk, ld_frag_tr(sQw, LDQ, 32 * ks + 8 * kg, 32 * ks + 8 * kg + 4, d0, lane),
                  ld_frag(sDLm, LY::LDC, r, 32 * ks + 8 * kg));
          if (mv != nullptr) {
#pragma unroll
            for (int ks = 0; ks < C / 32; ++ks)
              mma32(xv, ld_frag_tr(sdO, LDQ, 32 * ks + 8 * kg, 32 * ks + 8 * kg + 4, d0, lane),
                    ld_frag(sPm, LY::LDC, r, 32 * ks + 8 * kg));
          }
          if (r < M) {
            *reinterpret_cast<f32x4*>(dst + (size_t)r * MW + d0 + 4 * kg) = xk;
            if (mv != nullptr) *reinterpret_cast<f32x4*>(dst + (size_t)r * MW + D + d0 + 4 * kg) = xv;
          }
        }
      }
    }
  }

  // ------------------------------------------------------------------ store
  // Fast path: through LDS (every tile is free after the window phase), so that each lane writes
  // 16-byte runs of whole rows (dq to the first tile, dk to the second, dv to the third).  The
  // sub-block path, at its register limit, stores its accumulators directly.
  if constexpr (STRONG) {
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
  } else {
    T* sOq = reinterpret_cast<T*>(smem);
    T* sOk = reinterpret_cast<T*>(smem + LY::tile);
    T* sOv = reinterpret_cast<T*>(smem + 2 * LY::tile);
    __syncthreads();   // the window phase's last readers of the tiles are done
    if (qrole) {
#pragma unroll
      for (int x = 0; x < NB; ++x) st4(sOq + u * LDQ + 16 * x + 4 * kg, acc0[x][0], acc0[x][1], acc0[x][2], acc0[x][3]);
    } else {
#pragma unroll
      for (int x = 0; x < NB; ++x) {
        st4(sOk + u * LDQ + 16 * x + 4 * kg, acc0[x][0], acc0[x][1], acc0[x][2], acc0[x][3]);
        st4(sOv + u * LDQ + 16 * x + 4 * kg, acc1[x][0], acc1[x][1], acc1[x][2], acc1[x][3]);
      }
    }
    __syncthreads();
#pragma unroll
    for (int e = 0; e < NVT; ++e) {
      const int idx = tid + e * NTHR_CK, row = idx / (D / VEC), cv = idx % (D / VEC);
      if (t0 + row < L) {
        const size_t o = hoff + (size_t)(t0 + row) * D + cv * VEC;
        *reinterpret_cast<V16*>(reinterpret_cast<T*>(a.dq) + o) = *reinterpret_cast<const V16*>(sOq + row * LDQ + cv * VEC);
        *reinterpret_cast<V16*>(reinterpret_cast<T*>(a.dk) + o) = *reinterpret_cast<const V16*>(sOk + row * LDQ + cv * VEC);
        *reinterpret_cast<V16*>(reinterpret_cast<T*>(a.dv) + o) = *reinterpret_cast<const V16*>(sOv + row * LDQ + cv * VEC);
      }
    }
  }
}

// The fast path: one workgroup per (b, h, chunk); consecutive chunks of one head share an XCD.
template <typename T, int D, bool SG, bool FEAT>
__global__ __launch_bounds__(NTHR_CK, 1) void chunk_kernel(BwdArgs a, const T* __restrict__ wsdS,
                                                            const float* __restrict__ wsbnd) {
  extern __shared__ __align__(16) unsigned char smem[];
  const int NC = (a.L + C - 1) / C, BH = a.B * a.H;
  int bh, c;
  const int bid = blockIdx.x;
  if ((BH & 7) == 0) {
    const int x = bid % 8, y = bid / 8;           // y runs over (head group, chunk)
    c = y % NC;
    bh = (y / NC) * 8 + x;
  } else {
    bh = bid / NC;
    c = bid % NC;
  }
  chunk_body<T, D, SG, FEAT, false>(a, wsdS, wsbnd, bh, c, smem, threadIdx.x);
}

// The sub-block path over the dispatch list (persistent workgroups; an empty list ends at once).
template <typename T, int D, bool SG, bool FEAT>
__global__ __launch_bounds__(NTHR_CK, 1) void chunk_strong_kernel(BwdArgs a, const T* __restrict__ wsdS,
                                                                   const float* __restrict__ wsbnd) {
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
    chunk_body<T, D, SG, FEAT, true>(a, wsdS, wsbnd, id / NC, id % NC, smem, tid);
  }
}

// ------------------------------------------------------------ meta reduce
// Deterministic sum of the per-(batch, chunk) meta partials part[slot][H*M*MW] (MW = 2D with meta
// values, D without) in one launch: a workgroup takes 64 partial columns; its 16 groups of 64
// threads sum every 16th slot, and the 16 group sums are added in a fixed order.
constexpr int DM_COLS = 64, DM_GROUPS = 16;
__global__ __launch_bounds__(DM_COLS * DM_GROUPS) void dmeta_sum_kernel(const float* __restrict__ part,
                                                                         float* __restrict__ dmk,
                                                                         float* __restrict__ dmv, int slots, int n,
                                                                         int D, int MW) {
  __shared__ float red[DM_GROUPS][DM_COLS];
  const int col = threadIdx.x % DM_COLS, grp = threadIdx.x / DM_COLS;
  const int e = blockIdx.x * DM_COLS + col;
  float acc = 0.f;
  if (e < n) {
#pragma unroll 8
    for (int s = grp; s < slots; s += DM_GROUPS) acc += part[(size_t)s * n + e];
  }
  red[grp][col] = acc;
  __syncthreads();
  if (grp == 0 && e < n) {
    float t = 0.f;
#pragma unroll
    for (int g2 = 0; g2 < DM_GROUPS; ++g2) t += red[g2][col];
    const int hm = e / MW, c2 = e % MW;
    if (c2 < D) dmk[(size_t)hm * D + c2] = t;
    else if (dmv != nullptr) dmv[(size_t)hm * D + c2 - D] = t;
  }
}

__global__ void fill_zero_kernel(float* p, size_t n) {
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
constexpr int kStrongGridBwd = 256;

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
  const StrongDispatch sd = dispatch_layout(ws + wl.disp, a.B, a.H, a.L, D);
  a.strong = sd.mask;
  a.list = sd.list;
  a.list_count = sd.count;
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
  if (a.lse == nullptr || a.o_swa == nullptr || a.chunk_states == nullptr) {
    // the saved forward tensors were not kept: the forward kernels recompute all three into the
    // workspace (o itself is not written)
    FwdArgs f{};
    f.q = a.q; f.k = a.k; f.v = a.v; f.g = a.g; f.meta_k = a.meta_k; f.meta_v = a.meta_v;
    f.o = nullptr;
    f.lse = reinterpret_cast<float*>(ws + wl.rc_lse);
    f.o_swa = ws + wl.rc_oswa;
    f.chunk_states = nullptr;
    f.state_out = nullptr;
    f.workspace = ws + wl.rc_fwd;
    f.B = a.B; f.H = a.H; f.L = a.L; f.W = a.W; f.M = a.M;
    f.scale = a.scale; f.mix = a.mix; f.gate = a.gate;
    f.lq = a.lq; f.lk = a.lk;
    if ((e = launch_fwd(f, std::is_same<T, bf16_t>::value ? 1 : 0, D, st)) != hipSuccess) return e;
    a.lse = f.lse;
    a.o_swa = f.o_swa;
    a.chunk_states = ws + wl.rc_fwd + fwd_aux_bytes(a.B, a.H, a.L, D);
  }
  // the state-gradient sweep also forms the window row dots delta_t from the dO rows it streams
  {
    const bool feat = a.lq != nullptr;
    const int NS = sweep_segments(a.B, a.H, a.L, D);
    SweepArgs sw{feat ? (const void*)a.lq : a.q, a.dO, a.g, a.chunk_states, wsdS, wsbnd, nullptr, nullptr,
                 a.B, a.H, a.L, NS, (NC + NS - 1) / NS, nullptr, nullptr, nullptr, a.gate, feat ? 1 : 0, a.o_swa,
                 a.ws_delta, a.mix, sd.mask, sd.count};
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
    using LY = CkLayout<T, D, false>;
    using LS = CkLayout<T, D, true>;
    const int variant = a.lq != nullptr ? 2 : a.gate ? 1 : 0;   // log features: per-dimension gates only
    auto kern = variant == 2 ? chunk_kernel<T, D, false, true>
              : variant == 1 ? chunk_kernel<T, D, true, false> : chunk_kernel<T, D, false, false>;
    auto skern = variant == 2 ? chunk_strong_kernel<T, D, false, true>
               : variant == 1 ? chunk_strong_kernel<T, D, true, false> : chunk_strong_kernel<T, D, false, false>;
    if ((e = set_lds(kern, LY::bytes)) != hipSuccess) return e;
    if ((e = set_lds(skern, LS::bytes)) != hipSuccess) return e;
    hipLaunchKernelGGL(kern, dim3(BH * NC), dim3(NTHR_CK), LY::bytes, st, a, (const T*)wsdS, (const float*)wsbnd);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    hipLaunchKernelGGL(skern, dim3(min(BH * NC, kStrongGridBwd)), dim3(NTHR_CK), LS::bytes, st, a, (const T*)wsdS,
                       (const float*)wsbnd);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  mark(2);
  if (a.M > 0) {
    const int MW = a.meta_v != nullptr ? 2 * D : D;
    const int n = a.H * a.M * MW;
    const int slots = a.B * NC;
    hipLaunchKernelGGL(dmeta_sum_kernel, dim3((n + DM_COLS - 1) / DM_COLS), dim3(DM_COLS * DM_GROUPS), 0, st,
                       (const float*)a.ws_dmeta, a.dmeta_k, a.dmeta_v, slots, n, D, MW);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  mark(3);
  return hipSuccess;
}

}  // namespace

size_t bwd_workspace_bytes(int B, int H, int L, int M, int D, int dtype) {
  return ws_layout(B, H, L, M, D, dtype).total;
}

size_t bwd_recompute_workspace_bytes(int B, int H, int L, int M, int D, int dtype) {
  return L > 0 ? ws_layout(B, H, L, M, D, dtype).rc_total : 0;
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
