// lz_sweep.hip -- the sequential chunk sweeps of the GLA branch on gfx950.
//
// The GLA state (gist.science explainer of "Lizard: An Efficient
// Linearization Framework for Large Language Models", English page §2.A,
// state update with a per-key-dimension gate) and its gradient both follow,
// chunk by chunk, with b the chunk-local inclusive prefix of the log-gates
// and Gamma its value at the chunk end (English page §2.C: gates handled in
// log space, only chunk-local sums exponentiated):
//
//   forward,  chunks ascending:   S_{c+1} = diag(e^Gamma) S_c + (k e^{Gamma-b})^T v
//             stores S_c (the state entering chunk c) in the operand dtype,
//             row-major [d_k][d_v], and the final state in fp32;
//   backward, chunks descending:  dS_{c-1} = diag(e^Gamma) dS_c + (q e^b)^T dO
//             where dS_c is the gradient w.r.t. the state after chunk c;
//             stores dS'_c = diag(e^Gamma) dS_c transposed ([d_v][d_k]) (rows i whose
//             Gamma_i is below -kStrongGate keep dS_c undecayed: e^Gamma may underflow
//             there) and the boundary term of the gate gradient,
//             rowsum(S_{c+1} (.) dS_c), per 64-wide d_v tile.
//   Both directions also publish, per chunk, which key columns have a chunk total
//   below -kStrongGate (the dispatch of the chunk kernels' sub-block path).
//
// Element (i, j) of the carried matrix evolves independently of every other,
// so the sweep is tiled over blocks of 64 rows (d_k): one workgroup per
// (b, h, row block) carries its rows over every column in fp32 registers
// through all chunks (four waves per 64 x 64 tile), with the inputs of the
// next chunks in flight (three forward, two backward) while one is
// processed (none of them depends on the carried matrix).  The gate prefix
// runs inside rows of 16 lanes (DPP), with no LDS round trip or barrier.
// With few heads both directions also split the chunks into sequence segments
// that sweep in parallel: a reduce pass carries every segment but the one swept
// first from zero, a scan over the segments forms what enters each of them, and
// the sweep proper then starts every segment from it.
#include <algorithm>
#include <type_traits>

#include "lz_common.hpp"
#include "lz_kernels.hpp"

namespace lz {
namespace {

constexpr int TT = 64;          // tile edge over d_k and d_v
constexpr int NTHR_SW = 256;

template <typename T, int D>
struct SwLayout {
  static constexpr int LDA = TT + Tr<T>::PAD;
  static constexpr int LDB = D + Tr<T>::PAD;
  static constexpr size_t oA = 0;                                   // [C][TT]  gate-folded q or k (i tile)
  static constexpr size_t oB = oA + sizeof(T) * CHUNK * LDA;        // [C][D]   v or dO (every j)
  static constexpr size_t oS = oB + sizeof(T) * CHUNK * LDB;        // [TT][D]  state rows (backward);
                                                                    // forward: the chunk state on its way out
  static constexpr int LDT = TT + Tr<T>::PAD;
  static constexpr size_t oT = oS + sizeof(T) * TT * LDB;     // backward: dS' on its way out [D][TT]
  static constexpr size_t oDec = oT + sizeof(T) * D * LDT;    // e^Gamma of the 64 rows
  static constexpr size_t oFac = oDec + sizeof(float) * TT;    // backward: factor of the stored dS
  static constexpr size_t bytes = oFac + sizeof(float) * TT;
  static_assert(bytes <= 160 * 1024, "LDS budget");
};

// Four values of column c0 + (lane & 15), rows r0 .. r0+3, of a row-major LDS tile.
__device__ __forceinline__ f32x4 col4(const bf16_t* tile, int ld, int r0, int c0, int lane) {
  const bf16x4 x = tr4(tile, ld, r0, c0, lane);
  return f32x4{(float)x[0], (float)x[1], (float)x[2], (float)x[3]};
}
__device__ __forceinline__ f32x4 col4(const float* tile, int ld, int r0, int c0, int lane) {
  const int c = c0 + (lane & 15);
  return f32x4{tile[r0 * ld + c], tile[(r0 + 1) * ld + c], tile[(r0 + 2) * ld + c], tile[(r0 + 3) * ld + c]};
}

// Inputs of one chunk held in registers while the previous chunk is processed.  Every
// value is kept as loaded (no conversion, no broadcast) until the chunk is processed: a
// use right after a load in a branch makes the compiler wait for it there, and that
// wait (vmcnt counts in issue order) also drains every chunk already in flight.
template <int NV, typename RA>
struct SwStage {
  RA ra[4];      // q or k (or fp32 log features): tokens 4*tg+u, four columns, as loaded
  f32x4 rg[4];   // log-gates, same positions (scalar gates: component 0 only)
  V16 rb[NV];    // v or dO tile, 16-byte vectors
  V16 rs[NV];    // state tile (backward)
  V16 ro[NV];    // o_swa rows (backward row dots)
};

// REDUCE: carry a segment from a zero state (gradient) and keep only its final state
// (gradient at the segment's first chunk boundary) and gate total; no chunk outputs.
// SG: one log-gate per head and token (g [B,H,L]), broadcast over the key dimensions.
// FEAT: a_src holds fp32 log features l (of phi(k) forward, phi(q) backward); the gate is
// absorbed in log space, exp(l + c), instead of scaling a raw operand by exp(c).
template <typename T, int D, bool REV, bool REDUCE, bool SG, bool FEAT>
__global__ __launch_bounds__(NTHR_SW * (D / TT)) void sweep_kernel(SweepArgs a) {
  using LY = SwLayout<T, D>;
  // chunks of inputs in flight: three forward (two measured the same at the train shape; four
  // spill), two backward (its stages also carry state rows and o_swa)
  constexpr int DEPTH = REV ? 2 : 3;
  constexpr int NTI = D / TT;                      // tiles per edge
  constexpr int NTHR = NTHR_SW * NTI;              // four waves per 64 x 64 tile of the row block
  constexpr int VEC = Tr<T>::VEC;
  constexpr int NV = CHUNK * (D / VEC) / NTHR;     // 16-byte vectors per thread of a [64][D] tile
  static_assert(NV % NTI == 0, "the row-dot slots split evenly over the row blocks");
  constexpr int LDA = LY::LDA, LDB = LY::LDB;

  extern __shared__ __align__(16) unsigned char smem[];
  T* sA = reinterpret_cast<T*>(smem + LY::oA);
  T* sB = reinterpret_cast<T*>(smem + LY::oB);
  T* sS = reinterpret_cast<T*>(smem + LY::oS);
  T* sT = reinterpret_cast<T*>(smem + LY::oT);
  float* sDec = reinterpret_cast<float*>(smem + LY::oDec);
  float* sFac = reinterpret_cast<float*>(smem + LY::oFac);

  // One workgroup carries a block of 64 rows (i) of the state over every column (j): four waves
  // per 64 x 64 tile (wave w of tile jt), so the i tile's gate-folded q or k is formed once and
  // the v or dO rows are loaded once for all tiles of the row block.
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, r = lane & 15, kg = lane >> 4;
  const int jt = wave >> 2, w = wave & 3;
  // workgroup -> (b*h, segment, i tile); the row blocks and segments of one head share an XCD
  const int BH = a.B * a.H;
  const int NSL = REDUCE ? a.NS - 1 : a.NS;        // segments launched (a reduce skips the one swept first)
  const int PER = NTI * NSL;
  int bh, it, seg;
  {
    const int bid = blockIdx.x;
    int y2;
    if ((BH & 7) == 0) {
      const int x = bid % 8, y = bid / 8;
      bh = (y / PER) * 8 + x;
      y2 = y % PER;
    } else {
      bh = bid / PER;
      y2 = bid % PER;
    }
    seg = y2 / NTI + (REV && REDUCE ? 1 : 0);   // the reverse reduce skips the first segment
    it = y2 % NTI;
  }
  const int i0 = it * TT, j0 = jt * TT;
  const int L = a.L, NC = (L + CHUNK - 1) / CHUNK;
  const int c_begin = seg * a.SC, c_end = min(NC, c_begin + a.SC), NCs = c_end - c_begin;
  const size_t hoff = (size_t)bh * L * D;
  using AT = std::conditional_t<FEAT, float, T>;
  const AT* asrc = reinterpret_cast<const AT*>(a.a_src) + hoff;
  const T* bsrc = reinterpret_cast<const T*>(a.b_src) + hoff;
  // backward: the row blocks of a head also form the window row dots of each chunk, the block of
  // state rows i0.. taking the token rows of its own register slots u with u % NTI == it
  const bool dots = REV && !REDUCE && a.delta != nullptr;
  const T* osrc = reinterpret_cast<const T*>(dots ? a.o_swa : a.b_src) + hoff;   // (unused without dots)
  const float* g = a.g + (SG ? (size_t)bh * L : hoff);
  const T* states = reinterpret_cast<const T*>(a.states) + (size_t)bh * NC * D * D;
  T* out = reinterpret_cast<T*>(a.out) + (size_t)bh * NC * D * D;

  // gate scan map: wave w owns columns 16w .. 16w+15 of the tile; a row of 16
  // lanes (column group cg = kg) holds tokens 4*tg .. 4*tg+3, tg = lane & 15,
  // so the prefix over tokens is an in-row scan
  const int tg = r, cg = kg;
  const int acol = i0 + 16 * w + 4 * cg;
  using RA = decltype(ld4raw(static_cast<const AT*>(nullptr)));
  // No bounds branches: rows past the sequence end are loaded clamped onto its last row (and
  // the state after the last chunk onto the last state) and masked when the chunk is processed.
  auto load = [&](SwStage<NV, RA>& s, int c) {
    const int t0 = c * CHUNK;
    // Only the waves of the first column tile use q or k and the gates; the others read one
    // fixed line instead, so that every wave issues the same loads (a wave that skipped them
    // would, by the reasoning above, make the compiler's waits shallower for all).
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int t = jt == 0 ? min(t0 + 4 * tg + u, L - 1) : 0;
      const size_t o = jt == 0 ? (size_t)t * D + acol : 0;
      s.ra[u] = ld4raw(asrc + o);
      if constexpr (SG)
        s.rg[u][0] = g[t];
      else
        s.rg[u] = ld4raw(g + o);
    }
#pragma unroll
    for (int u = 0; u < NV; ++u) {
      const int idx = tid + u * NTHR, row = idx / (D / VEC), cv = idx % (D / VEC);
      s.rb[u] = ldg16(bsrc + (size_t)min(t0 + row, L - 1) * D + cv * VEC);
    }
    if constexpr (REV && !REDUCE) {
      const int cn = min(c + 1, NC - 1);
#pragma unroll
      for (int u = 0; u < NV; ++u) {
        const int idx = tid + u * NTHR, row = idx / (D / VEC), cv = idx % (D / VEC);
        s.rs[u] = ldg16(states + ((size_t)cn * D + i0 + row) * D + cv * VEC);
      }
      // the token rows of slots u = it, it + NTI, ... (slot u / NTI holds slot u's row)
#pragma unroll
      for (int m = 0; m < NV / NTI; ++m) {
        const int idx = tid + (m * NTI + it) * NTHR, row = idx / (D / VEC), cv = idx % (D / VEC);
        s.ro[m] = ldg16(osrc + (size_t)min(t0 + row, L - 1) * D + cv * VEC);
      }
    }
  };

  // carried tile: forward acc[ib][e] = S[i0+16ib+r][j0+16w+4kg+e];
  //               backward acc[jb][e] = dS[i0+16w+4kg+e][j0+16jb+r]
  f32x4 acc[4];
#pragma unroll
  for (int x = 0; x < 4; ++x) acc[x] = f32x4{0, 0, 0, 0};
  if constexpr (REV && !REDUCE) {
    // the gradient entering this segment from the later ones (the reverse segment scan)
    if (a.NS > 1) {   // (its wait taken here, as for the forward's entering state below)
      const float* si = a.seg_in + ((size_t)bh * a.NS + seg) * D * D;
#pragma unroll
      for (int jb = 0; jb < 4; ++jb)
#pragma unroll
        for (int e = 0; e < 4; ++e) acc[jb][e] = si[(size_t)(i0 + 16 * w + 4 * kg + e) * D + j0 + 16 * jb + r];
#pragma unroll
      for (int jb = 0; jb < 4; ++jb)
        asm volatile("" ::"v"(acc[jb][0]), "v"(acc[jb][1]), "v"(acc[jb][2]), "v"(acc[jb][3]));
    }
  }
  if constexpr (!REV && !REDUCE) {
    // the state entering this segment: from the segment scan, or the carried state of a
    // continuation for a single segment
    const float* si = a.NS > 1 ? a.seg_in + ((size_t)bh * a.NS + seg) * D * D
                               : (a.state_in != nullptr ? a.state_in + (size_t)bh * D * D : nullptr);
    if (si != nullptr)
#pragma unroll
      for (int ib = 0; ib < 4; ++ib)
        acc[ib] = *reinterpret_cast<const f32x4*>(si + (size_t)(i0 + 16 * ib + r) * D + j0 + 16 * w + 4 * kg);
    // take the wait for these loads here, before any chunk is in flight: otherwise the loop
    // (whose first step stores the carried tile) inherits a possibly pending load into the
    // carried registers and waits on it at every step, draining the chunks in flight
#pragma unroll
    for (int ib = 0; ib < 4; ++ib) asm volatile("" ::"v"(acc[ib][0]), "v"(acc[ib][1]), "v"(acc[ib][2]), "v"(acc[ib][3]));
  }
  f32x4 gsum = f32x4{0, 0, 0, 0};   // reduce: gate total of this lane's four key columns
  if constexpr (!REDUCE)
    if (a.list_count != nullptr && blockIdx.x == 0 && tid == 0) *a.list_count = 0;

  auto chunk_of = [&](int n) { return REV ? c_end - 1 - n : c_begin + n; };
  // backward: dS' of chunk cs from its LDS tile to HBM as whole row runs, 16 bytes a lane (the
  // tile is written after one barrier and read after the next)
  auto flush_dS = [&](int cs) {
#pragma unroll
    for (int u = 0; u < NV; ++u) {
      const int idx = tid + u * NTHR, row = idx / (TT / VEC), cv = idx % (TT / VEC);
      *reinterpret_cast<V16*>(out + ((size_t)cs * D + row) * D + i0 + cv * VEC) =
          *reinterpret_cast<const V16*>(sT + row * LY::LDT + cv * VEC);
    }
  };
  const int nlast = max(NCs - 1, 0);
  auto process = [&](SwStage<NV, RA>& s, int n) {
    const int c = chunk_of(n);
    if constexpr (!REV && !REDUCE) {
      // state entering chunk c, to LDS (its readers of the previous chunk passed the last barrier)
#pragma unroll
      for (int ib = 0; ib < 4; ++ib)
        st4(sS + (16 * ib + r) * LDB + j0 + 16 * w + 4 * kg, acc[ib][0], acc[ib][1], acc[ib][2], acc[ib][3]);
    }
    __syncthreads();   // the previous chunk's operand reads are done
    if constexpr (REV && !REDUCE) {
      if (n > 0) flush_dS(c + 1);   // the chunk processed last (descending order)
    }
    if constexpr (!REV && !REDUCE) {
      // ... and out as whole rows, 16 bytes a lane
#pragma unroll
      for (int u = 0; u < NV; ++u) {
        const int idx = tid + u * NTHR, row = idx / (D / VEC), cv = idx % (D / VEC);
        *reinterpret_cast<V16*>(out + ((size_t)c * D + i0 + row) * D + cv * VEC) =
            *reinterpret_cast<const V16*>(sS + row * LDB + cv * VEC);
      }
    }
#pragma unroll
    for (int u = 0; u < NV; ++u) {
      const int idx = tid + u * NTHR, row = idx / (D / VEC), cv = idx % (D / VEC);
      *reinterpret_cast<V16*>(sB + row * LDB + cv * VEC) = c * CHUNK + row < L ? s.rb[u] : zero16();
      if constexpr (REV && !REDUCE) *reinterpret_cast<V16*>(sS + row * LDB + cv * VEC) = c + 1 < NC ? s.rs[u] : zero16();
    }
    if (REV && dots) {
      // delta_t = mix * dO_t . o_swa_t, formed before this stage's registers take the next chunk;
      // a row's D/VEC vectors sit in consecutive lanes
      const int t0 = c * CHUNK;
#pragma unroll
      for (int u = 0; u < NV; ++u) {
        if (u % NTI != it) continue;
        const int idx = tid + u * NTHR, row = idx / (D / VEC), cv = idx % (D / VEC);
        float dot = 0.f;
#pragma unroll
        for (int e = 0; e < VEC; ++e)
          dot += v16_get(s.rb[u], e, (T*)nullptr) * v16_get(s.ro[u / NTI], e, (T*)nullptr);
        dot = group_sum<D / VEC>(dot);
        if (cv == 0 && t0 + row < L) a.delta[(size_t)bh * L + t0 + row] = a.mix * dot;
      }
    }
    if (jt == 0) {
      // rows past the end: no decay, and a zero operand (log features: -inf)
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const bool okr = c * CHUNK + 4 * tg + u < L;
        if constexpr (SG) {
          const float x = okr ? s.rg[u][0] : 0.f;
          s.rg[u] = f32x4{x, x, x, x};
        } else if (!okr) {
          s.rg[u] = f32x4{0, 0, 0, 0};
        }
      }
      // chunk-local inclusive prefix b of the gates and the chunk total Gamma; the forward also
      // forms Gamma - b (the keys' decay to the chunk end) directly as the exclusive suffix of the
      // gates, not as the difference of two chunk-long sums, so it is as accurate as its own size
      f32x4 sx[4];   // forward: exclusive suffix inside the lane
      if constexpr (!REV) {
        sx[3] = f32x4{0, 0, 0, 0};
#pragma unroll
        for (int u = 2; u >= 0; --u) sx[u] = sx[u + 1] + s.rg[u + 1];
      }
#pragma unroll
      for (int u = 1; u < 4; ++u) s.rg[u] += s.rg[u - 1];
      f32x4 excl, tot, esx;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float own = s.rg[3][e];
        excl[e] = row_scan16(own) - own;
        tot[e] = row_sum16(own);
        if constexpr (!REV) esx[e] = dpp_row<0x101>(row_suffix16(own));   // later lanes of the row
      }
      // a column is strong when its chunk total is below -kStrongGate: there the chunk kernels
      // take the sub-block path, and the backward stores the state gradient undecayed (e^Gamma
      // may underflow); the one comparison below decides both, so they always agree
      bool strongc[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) strongc[e] = tot[e] < -kStrongGate;
      if (tg == 0)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float dec = __expf(tot[e]);
          sDec[16 * w + 4 * cg + e] = dec;
          if constexpr (REV) sFac[16 * w + 4 * cg + e] = strongc[e] ? 1.f : dec;
        }
      if constexpr (!REDUCE) {
        if (a.strong != nullptr) {
          // 16 columns of this wave: bit 4*cg + e (every lane of a row holds the row's totals)
          unsigned m16 = 0;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const unsigned long long bal = __ballot(strongc[e]);
#pragma unroll
            for (int g4 = 0; g4 < 4; ++g4) m16 |= (unsigned)((bal >> (16 * g4)) & 1ull) << (4 * g4 + e);
          }
          if (lane == 0) a.strong[((size_t)bh * NC + c) * (D / 16) + it * 4 + w] = (uint16_t)m16;
        }
      }
      if constexpr (REDUCE) gsum += tot;
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        f32x4 x;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float ex = REV ? s.rg[u][e] + excl[e] : sx[u][e] + esx[e];
          const bool okr = c * CHUNK + 4 * tg + u < L;
          const float av = okr ? (float)s.ra[u][e] : (FEAT ? -INFINITY : 0.f);
          x[e] = FEAT ? __expf(av + ex) : av * __expf(ex);
        }
        st4(sA + (4 * tg + u) * LDA + 16 * w + 4 * cg, x[0], x[1], x[2], x[3]);
      }
    }
    // unconditional for the same reason as the first loads (the last rounds repeat the last chunk)
    load(s, chunk_of(min(n + DEPTH, nlast)));
    __syncthreads();

    if constexpr (REV) {
      // boundary rowsum over this j tile, decay, store dS' transposed (a reduce only decays)
      if constexpr (!REDUCE) {
        f32x4 rsum = f32x4{0, 0, 0, 0};
#pragma unroll
        for (int jb = 0; jb < 4; ++jb) rsum += col4(sS, LDB, 16 * w + 4 * kg, j0 + 16 * jb, lane) * acc[jb];
#pragma unroll
        for (int e = 0; e < 4; ++e) rsum[e] = row_sum16(rsum[e]);
        if (r == 0)
          stg4(a.bnd + (((size_t)bh * NC + c) * NTI + jt) * D + i0 + 16 * w + 4 * kg, rsum[0], rsum[1], rsum[2],
               rsum[3]);
      }
      f32x4 dec, fac;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        dec[e] = sDec[16 * w + 4 * kg + e];
        fac[e] = sFac[16 * w + 4 * kg + e];
      }
#pragma unroll
      for (int jb = 0; jb < 4; ++jb) {
        if constexpr (!REDUCE) {
          // dS' = e^Gamma dS, or dS itself in the strong columns (fac = 1)
          const f32x4 y = acc[jb] * fac;
          st4(sT + (j0 + 16 * jb + r) * LY::LDT + 16 * w + 4 * kg, y[0], y[1], y[2], y[3]);
        }
        acc[jb] *= dec;
      }
      // + (q e^b)^T dO
#pragma unroll
      for (int ks = 0; ks < CHUNK / 32; ++ks) {
        const auto fa = ld_frag_tr(sA, LDA, 32 * ks + 8 * kg, 32 * ks + 8 * kg + 4, 16 * w, lane);
#pragma unroll
        for (int jb = 0; jb < 4; ++jb)
          mma32(acc[jb], fa, ld_frag_tr(sB, LDB, 32 * ks + 8 * kg, 32 * ks + 8 * kg + 4, j0 + 16 * jb, lane));
      }
    } else {
#pragma unroll
      for (int ib = 0; ib < 4; ++ib) acc[ib] *= sDec[16 * ib + r];
      // + (k e^{Gamma-b})^T v, computed transposed so each lane holds four consecutive d_v entries
#pragma unroll
      for (int ks = 0; ks < CHUNK / 32; ++ks) {
        const auto fb = ld_frag_tr(sB, LDB, 32 * ks + 8 * kg, 32 * ks + 8 * kg + 4, j0 + 16 * w, lane);
#pragma unroll
        for (int ib = 0; ib < 4; ++ib)
          mma32(acc[ib], fb, ld_frag_tr(sA, LDA, 32 * ks + 8 * kg, 32 * ks + 8 * kg + 4, 16 * ib, lane));
      }
    }
  };

  // DEPTH chunks of inputs in flight, stage i serving the steps n with n % DEPTH == i
  SwStage<NV, RA> s0, s1, s2;
  // The first stages load unconditionally (a short segment repeats its last chunk; every row
  // is clamped into the sequence): a stage skipped on some path would make the compiler
  // assume, at the loop head, that its registers were loaded just before and wait for them.
  load(s0, chunk_of(0));
  load(s1, chunk_of(min(1, nlast)));
  if constexpr (DEPTH > 2) load(s2, chunk_of(min(2, nlast)));
  // Full rounds, then the tail: with the tail's conditions inside the loop, its control flow
  // would hold a path back to the loop head after one stage only, along which the next
  // stage's loads look recent, and the compiler would wait for them (and for every chunk
  // in flight) at each step.
  int n0 = 0;
  for (; n0 + DEPTH <= NCs; n0 += DEPTH) {
    process(s0, n0);
    process(s1, n0 + 1);
    if constexpr (DEPTH > 2) process(s2, n0 + 2);
  }
  if (n0 < NCs) process(s0, n0);
  if (DEPTH > 2 && n0 + 1 < NCs) process(s1, n0 + 1);
  if constexpr (REV && !REDUCE) {
    if (NCs > 0) {
      __syncthreads();
      flush_dS(chunk_of(NCs - 1));
    }
  }
  if constexpr (REDUCE) {
    const size_t sb = (size_t)bh * a.NS + seg;
    float* sf = a.seg_fin + sb * D * D;
    if constexpr (REV) {
#pragma unroll
      for (int jb = 0; jb < 4; ++jb)
#pragma unroll
        for (int e = 0; e < 4; ++e) sf[(size_t)(i0 + 16 * w + 4 * kg + e) * D + j0 + 16 * jb + r] = acc[jb][e];
    } else {
#pragma unroll
      for (int ib = 0; ib < 4; ++ib)
        stg4(sf + (size_t)(i0 + 16 * ib + r) * D + j0 + 16 * w + 4 * kg, acc[ib][0], acc[ib][1], acc[ib][2],
             acc[ib][3]);
    }
    if (jt == 0 && tg == 0)
      *reinterpret_cast<f32x4*>(a.seg_gtot + sb * D + acol) = gsum;
  } else if constexpr (!REV) {
    if (a.state_out != nullptr && seg == a.NS - 1) {
      float* so = a.state_out + (size_t)bh * D * D;
#pragma unroll
      for (int ib = 0; ib < 4; ++ib)
        stg4(so + (size_t)(i0 + 16 * ib + r) * D + j0 + 16 * w + 4 * kg, acc[ib][0], acc[ib][1], acc[ib][2],
             acc[ib][3]);
    }
  }
}

// The state entering each segment: seg_in[0] = state_in (or zero),
// seg_in[s+1] = diag(e^{gtot[s]}) seg_in[s] + seg_fin[s].  Reverse (state gradients):
// seg_in[NS-1] = 0, seg_in[s-1] = diag(e^{gtot[s]}) seg_in[s] + seg_fin[s].  One thread
// per (b*h, i, j).
__global__ __launch_bounds__(256) void seg_scan_kernel(SweepArgs a, int D, int rev) {
  const int per = D * D / 256;
  const int bh = blockIdx.x / per, e = (blockIdx.x % per) * 256 + threadIdx.x, i = e / D;
  const int NS = a.NS;
  const size_t base = (size_t)bh * NS;
  if (rev) {
    float S = 0.f;
    a.seg_in[(base + NS - 1) * D * D + e] = S;
    for (int s = NS - 1; s > 0; --s) {
      S = __expf(a.seg_gtot[(base + s) * D + i]) * S + a.seg_fin[(base + s) * D * D + e];
      a.seg_in[(base + s - 1) * D * D + e] = S;
    }
    return;
  }
  float S = a.state_in != nullptr ? a.state_in[(size_t)bh * D * D + e] : 0.f;
  a.seg_in[base * D * D + e] = S;
  for (int s = 0; s + 1 < NS; ++s) {
    S = __expf(a.seg_gtot[(base + s) * D + i]) * S + a.seg_fin[(base + s) * D * D + e];
    a.seg_in[(base + s + 1) * D * D + e] = S;
  }
}

template <typename T, int D, bool REV, bool SG, bool FEAT>
hipError_t launch_sweep_g(const SweepArgs& a, hipStream_t st) {
  using LY = SwLayout<T, D>;
  const int blocks = D / TT;                    // 64-row blocks of the state
  const int nthr = NTHR_SW * (D / TT);
  // (the fp32 layout exceeds the default 64 KB of dynamic LDS; set on every launch, which is cheap
  // and keeps no state on the host)
  hipError_t e;
  if ((e = hipFuncSetAttribute(reinterpret_cast<const void*>(sweep_kernel<T, D, REV, true, SG, FEAT>),
                               hipFuncAttributeMaxDynamicSharedMemorySize, (int)LY::bytes)) != hipSuccess)
    return e;
  if ((e = hipFuncSetAttribute(reinterpret_cast<const void*>(sweep_kernel<T, D, REV, false, SG, FEAT>),
                               hipFuncAttributeMaxDynamicSharedMemorySize, (int)LY::bytes)) != hipSuccess)
    return e;
  if (a.NS > 1) {   // segments: reduce (all but the first to be swept), scan, then the sweep
    hipLaunchKernelGGL((sweep_kernel<T, D, REV, true, SG, FEAT>), dim3(a.B * a.H * blocks * (a.NS - 1)),
                       dim3(nthr), LY::bytes, st, a);
    hipLaunchKernelGGL(seg_scan_kernel, dim3(a.B * a.H * (D * D / 256)), dim3(256), 0, st, a, D, REV ? 1 : 0);
  }
  hipLaunchKernelGGL((sweep_kernel<T, D, REV, false, SG, FEAT>), dim3(a.B * a.H * blocks * a.NS), dim3(nthr),
                     LY::bytes, st, a);
  return hipGetLastError();
}

template <typename T, int D, bool REV>
hipError_t launch_sweep_t(const SweepArgs& a, hipStream_t st) {
  // log features are taken with per-dimension gates only
  if (a.feat) return a.gate ? hipErrorInvalidValue : launch_sweep_g<T, D, REV, false, true>(a, st);
  return a.gate ? launch_sweep_g<T, D, REV, true, false>(a, st) : launch_sweep_g<T, D, REV, false, false>(a, st);
}

template <bool REV>
hipError_t launch_sweep_dir(const SweepArgs& a, int dtype, int D, hipStream_t st) {
  if (dtype == 1) {
    if (D == 128) return launch_sweep_t<bf16_t, 128, REV>(a, st);
    if (D == 64) return launch_sweep_t<bf16_t, 64, REV>(a, st);
  } else if (dtype == 0) {
    if (D == 64) return launch_sweep_t<float, 64, REV>(a, st);
  }
  return hipErrorInvalidValue;
}

}  // namespace

int sweep_segments(int B, int H, int L, int D) {
  const int NC = (L + CHUNK - 1) / CHUNK;
  const double base = (double)B * H * (D / TT);             // workgroups of one segment
  if (base >= 256) return 1;                                 // one per CU or more already
  // aim at ~256 workgroups, one per CU: the sweep streams at the same rate with more
  // (measured with 512 and 1024 on the 64K prefill), while every further segment adds
  // reduce work (reads of k, v and the gates)
  int ns = (int)((256 + base - 1) / base);
  ns = std::min(ns, NC / 16);                                // segments of at least 16 chunks
  if (ns <= 1) return 1;
  const int sc = (NC + ns - 1) / ns;
  return (NC + sc - 1) / sc;                                 // no empty segment
}

hipError_t launch_sweep(const SweepArgs& a, int dtype, int D, bool reverse, hipStream_t st) {
  return reverse ? launch_sweep_dir<true>(a, dtype, D, st) : launch_sweep_dir<false>(a, dtype, D, st);
}

}  // namespace lz
