// lz_common.hpp -- device helpers shared by the gfx950 kernels.
//
// Matrix-core convention used everywhere: one 16x16 output block per
// v_mfma_f32_16x16x32_bf16 (bf16 operands) or per eight v_mfma_f32_16x16x4_f32
// (fp32 operands), reduced over a K block of 32.  For both operand types a
// lane l of the 64-wide wave supplies, for row (A) or column (B) r = l & 15,
// the eight K values of "slot group" kg = l >> 4; the accumulator lane l
// holds C[4*kg + i][l & 15], i = 0..3.
//
// The K order inside a block is free as long as A and B agree, which lets an
// accumulator be fed back as an operand: a score tile computed transposed
// (keys as rows) leaves lane l with scores of query l & 15 against keys
// 16*kb + 4*kg + i; two such key blocks (kb0, kb1) form one K=32 operand
// whose slot s maps to key 16*kb_{s/4} + 4*kg + (s % 4).  The matching
// operand on the other side is then read with ld_frag_perm().
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace lz {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));

constexpr int WAVE = 64;
constexpr int CHUNK = 64;   // tokens per chunk of the chunkwise form

struct bf16_t { uint16_t bits; };   // storage tag for bf16 tensors in global memory

__device__ __forceinline__ float bf2f(uint16_t h) { return __uint_as_float(uint32_t(h) << 16); }
__device__ __forceinline__ uint16_t f2bf(float f) {
  __bf16 b = (__bf16)f;                 // round to nearest even (v_cvt_pk_bf16_f32 on gfx950)
  return __builtin_bit_cast(uint16_t, b);
}

// ---------------------------------------------------------------- type traits
template <typename T> struct Tr;

template <> struct Tr<float> {
  using frag = f32x8;
  static constexpr int PAD = 4;      // row padding in LDS (elements): 16 bytes
  static constexpr int VEC = 4;      // elements per 16-byte vector
  __device__ static float to_f(float x) { return x; }
  __device__ static float from_f(float x) { return x; }
};

template <> struct Tr<bf16_t> {
  using frag = bf16x8;
  static constexpr int PAD = 8;
  static constexpr int VEC = 8;
  __device__ static float to_f(bf16_t x) { return bf2f(x.bits); }
  __device__ static bf16_t from_f(float x) { return bf16_t{f2bf(x)}; }
};

// ------------------------------------------------------------------ MFMA core
__device__ __forceinline__ void mma32(f32x4& acc, const bf16x8& a, const bf16x8& b) {
  acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, acc, 0, 0, 0);
}
__device__ __forceinline__ void mma32(f32x4& acc, const f32x8& a, const f32x8& b) {
#pragma unroll
  for (int s = 0; s < 8; ++s) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a[s], b[s], acc, 0, 0, 0);
}

// Eight consecutive K values of row `row` of an LDS tile stored [row][k].
__device__ __forceinline__ bf16x8 ld_frag(const bf16_t* base, int ld, int row, int k) {
  return *reinterpret_cast<const bf16x8*>(base + row * ld + k);
}
__device__ __forceinline__ f32x8 ld_frag(const float* base, int ld, int row, int k) {
  const f32x4* p = reinterpret_cast<const f32x4*>(base + row * ld + k);
  f32x4 a = p[0], b = p[1];
  return f32x8{a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
}

// Operand matching an accumulator-fed operand over key blocks (kb0, kb1):
// slots 0..3 <- base[row][16*kb0 + 4*kg .. +4], slots 4..7 <- base[row][16*kb1 + 4*kg .. +4].
__device__ __forceinline__ bf16x8 ld_frag_perm(const bf16_t* base, int ld, int row, int kb0, int kb1, int kg) {
  const bf16x4 a = *reinterpret_cast<const bf16x4*>(base + row * ld + 16 * kb0 + 4 * kg);
  const bf16x4 b = *reinterpret_cast<const bf16x4*>(base + row * ld + 16 * kb1 + 4 * kg);
  return bf16x8{a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
}
__device__ __forceinline__ f32x8 ld_frag_perm(const float* base, int ld, int row, int kb0, int kb1, int kg) {
  const f32x4 a = *reinterpret_cast<const f32x4*>(base + row * ld + 16 * kb0 + 4 * kg);
  const f32x4 b = *reinterpret_cast<const f32x4*>(base + row * ld + 16 * kb1 + 4 * kg);
  return f32x8{a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
}

// Operand whose row/column index runs along the COLUMNS of a row-major LDS
// tile and whose K index runs down its ROWS (a transposed read).  Lane l
// gets tile[ra + e][c0 + (l & 15)] in slots e = 0..3 and
// tile[rb + e][c0 + (l & 15)] in slots 4..7, where ra / rb are chosen per
// 16-lane group by the caller (ra = k0 + 8*kg, rb = ra + 4 for the plain K
// order; ra = 16*kb0 + 4*kg, rb = 16*kb1 + 4*kg for the accumulator-fed
// order).  bf16 uses the gfx950 LDS transpose read: within a 16-lane group,
// lane k addresses row r + k/4, columns c0 + 4*(k%4) .. +4, and lane j
// receives the four values of column c0 + j from rows r .. r+3 (layout
// established with an in-bounds probe).  fp32 reads the four values directly.
typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4;
__device__ __forceinline__ bf16x4 tr4(const bf16_t* tile, int ld, int r, int c0, int lane) {
  const int k = lane & 15;
  const bf16_t* p = tile + (r + (k >> 2)) * ld + c0 + 4 * (k & 3);
  return __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(p));
}
__device__ __forceinline__ bf16x8 ld_frag_tr(const bf16_t* tile, int ld, int ra, int rb, int c0, int lane) {
  const bf16x4 a = tr4(tile, ld, ra, c0, lane);
  const bf16x4 b = tr4(tile, ld, rb, c0, lane);
  return bf16x8{a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
}
__device__ __forceinline__ f32x8 ld_frag_tr(const float* tile, int ld, int ra, int rb, int c0, int lane) {
  const int c = c0 + (lane & 15);
  f32x8 f;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    f[e] = tile[(ra + e) * ld + c];
    f[4 + e] = tile[(rb + e) * ld + c];
  }
  return f;
}

// Accumulators of key blocks kb0, kb1 as an operand (slot order as above).
__device__ __forceinline__ void pack_acc(bf16x8& out, const f32x4& a, const f32x4& b) {
  out = bf16x8{(__bf16)a[0], (__bf16)a[1], (__bf16)a[2], (__bf16)a[3],
               (__bf16)b[0], (__bf16)b[1], (__bf16)b[2], (__bf16)b[3]};
}
__device__ __forceinline__ void pack_acc(f32x8& out, const f32x4& a, const f32x4& b) {
  out = f32x8{a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
}

// Four consecutive values from an accumulator to an LDS row (8 or 16 bytes).
__device__ __forceinline__ void st4(bf16_t* p, float a, float b, float c, float d) {
  *reinterpret_cast<bf16x4*>(p) = bf16x4{(__bf16)a, (__bf16)b, (__bf16)c, (__bf16)d};
}
__device__ __forceinline__ void st4(float* p, float a, float b, float c, float d) {
  *reinterpret_cast<f32x4*>(p) = f32x4{a, b, c, d};
}

// ------------------------------------------------------- 16-byte global I/O
struct alignas(16) V16 { uint32_t w[4]; };

template <typename T>
__device__ __forceinline__ V16 ldg16(const T* p) { return *reinterpret_cast<const V16*>(p); }
template <typename T>
__device__ __forceinline__ void stg16(T* p, const V16& v) { *reinterpret_cast<V16*>(p) = v; }
__device__ __forceinline__ V16 zero16() { return V16{{0u, 0u, 0u, 0u}}; }

// Element e of a 16-byte vector of T, as float.
__device__ __forceinline__ float v16_get(const V16& v, int e, float*) { return __uint_as_float(v.w[e]); }
__device__ __forceinline__ float v16_get(const V16& v, int e, bf16_t*) {
  return bf2f(uint16_t((v.w[e >> 1] >> (16 * (e & 1))) & 0xFFFFu));
}

// ------------------------------------------------------------- wave reductions
// Reductions over lane pairs (l, l ^ m).  For m = 16 and m = 32 they use the gfx950 row
// swap instead of the LDS permute path: swapping a register with a copy of itself (the odd
// 16-lane rows, or the upper 32 lanes, of one copy trading places with the even rows, or the
// lower 32 lanes, of the other) leaves each lane holding its own value in one copy and its
// partner's in the other, so max and sum of the two copies are the pair's max and sum.
__device__ __forceinline__ void swap_pair(float x, int m, float& a, float& b) {
  const unsigned u = __float_as_uint(x);
  if (m == 16) {
    const auto r = __builtin_amdgcn_permlane16_swap(u, u, false, false);
    a = __uint_as_float(r[0]);
    b = __uint_as_float(r[1]);
  } else {
    const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
    a = __uint_as_float(r[0]);
    b = __uint_as_float(r[1]);
  }
}
__device__ __forceinline__ float xor_max(float x, int m) {
  if (m == 16 || m == 32) {
    float a, b;
    swap_pair(x, m, a, b);
    return fmaxf(a, b);
  }
  return fmaxf(x, __shfl_xor(x, m, WAVE));
}
__device__ __forceinline__ float xor_sum(float x, int m) {
  if (m == 16 || m == 32) {
    float a, b;
    swap_pair(x, m, a, b);
    return a + b;
  }
  return x + __shfl_xor(x, m, WAVE);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Cross-lane moves inside rows of 16 lanes through DPP (no LDS traffic).
// CTRL 0x110 + n: shift right by n within the row (zero fill);
// CTRL 0x120 + n: rotate right by n within the row.
template <int CTRL>
__device__ __forceinline__ float dpp_row(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL, 0xF, 0xF, true));
}
// Inclusive prefix sum over the 16 lanes of each row.
__device__ __forceinline__ float row_scan16(float x) {
  x += dpp_row<0x111>(x);
  x += dpp_row<0x112>(x);
  x += dpp_row<0x114>(x);
  x += dpp_row<0x118>(x);
  return x;
}
// Suffix sum over the 16 lanes of each row: lane r gets the sum of lanes r .. 15.
__device__ __forceinline__ float row_suffix16(float x) {
  x += dpp_row<0x101>(x);
  x += dpp_row<0x102>(x);
  x += dpp_row<0x104>(x);
  x += dpp_row<0x108>(x);
  return x;
}
// Sum over the 16 lanes of each row, returned in every lane of the row.
__device__ __forceinline__ float row_sum16(float x) {
  x += dpp_row<0x128>(x);
  x += dpp_row<0x124>(x);
  x += dpp_row<0x122>(x);
  x += dpp_row<0x121>(x);
  return x;
}
// Max over the 16 lanes of each row, returned in every lane of the row.
__device__ __forceinline__ float row_max16(float x) {
  x = fmaxf(x, dpp_row<0x128>(x));
  x = fmaxf(x, dpp_row<0x124>(x));
  x = fmaxf(x, dpp_row<0x122>(x));
  x = fmaxf(x, dpp_row<0x121>(x));
  return x;
}
// Max / sum over the whole wave, returned in every lane: rows by DPP, then the row swaps.
__device__ __forceinline__ float wave_max(float x) { return xor_max(xor_max(row_max16(x), 16), 32); }
__device__ __forceinline__ float wave_sum(float x) { return xor_sum(xor_sum(row_sum16(x), 16), 32); }
// Sum over aligned groups of N consecutive lanes, returned in every lane of the group.
template <int N>
__device__ __forceinline__ float group_sum(float x);
template <>
__device__ __forceinline__ float group_sum<8>(float x) {
  x += dpp_row<0x141>(x);   // half-row mirror: lane i of 8 pairs with lane 7-i
  x += dpp_row<0xB1>(x);    // quad permute [1,0,3,2]
  x += dpp_row<0x4E>(x);    // quad permute [2,3,0,1]
  return x;
}
template <>
__device__ __forceinline__ float group_sum<16>(float x) { return row_sum16(x); }
template <>
__device__ __forceinline__ float group_sum<32>(float x) { return xor_sum(row_sum16(x), 16); }

constexpr float LOG2E = 1.4426950408889634f;

// ------------------------------------------------------ operand / store helpers
// Eight consecutive K values straight from global memory (row-major tensor).
template <typename T>
__device__ __forceinline__ typename Tr<T>::frag ldg_frag(const T* p);
template <>
__device__ __forceinline__ bf16x8 ldg_frag<bf16_t>(const bf16_t* p) {
  return *reinterpret_cast<const bf16x8*>(p);
}
template <>
__device__ __forceinline__ f32x8 ldg_frag<float>(const float* p) {
  const f32x4 a = *reinterpret_cast<const f32x4*>(p);
  const f32x4 b = *reinterpret_cast<const f32x4*>(p + 4);
  return f32x8{a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
}
template <typename T>
__device__ __forceinline__ typename Tr<T>::frag zero_frag() {
  typename Tr<T>::frag f;
#pragma unroll
  for (int i = 0; i < 8; ++i) f[i] = 0;
  return f;
}

__device__ __forceinline__ void put_elem(float* p, float x) { *p = x; }
__device__ __forceinline__ void put_elem(bf16_t* p, float x) { p->bits = f2bf(x); }
__device__ __forceinline__ void put_bits(float* p, const V16& v, int e) { *p = __uint_as_float(v.w[e]); }
__device__ __forceinline__ void put_bits(bf16_t* p, const V16& v, int e) {
  p->bits = uint16_t((v.w[e >> 1] >> (16 * (e & 1))) & 0xFFFFu);
}

// Four consecutive floats to global memory in T.
__device__ __forceinline__ void stg4(float* p, float a, float b, float c, float d) {
  *reinterpret_cast<f32x4*>(p) = f32x4{a, b, c, d};
}
__device__ __forceinline__ void stg4(bf16_t* p, float a, float b, float c, float d) {
  *reinterpret_cast<bf16x4*>(p) = bf16x4{(__bf16)a, (__bf16)b, (__bf16)c, (__bf16)d};
}

// VEC consecutive elements (one 16-byte vector) built from floats.
__device__ __forceinline__ void st_vec(float* p, const float* x) {
  *reinterpret_cast<f32x4*>(p) = f32x4{x[0], x[1], x[2], x[3]};
}
__device__ __forceinline__ void st_vec(bf16_t* p, const float* x) {
  *reinterpret_cast<bf16x8*>(p) = bf16x8{(__bf16)x[0], (__bf16)x[1], (__bf16)x[2], (__bf16)x[3],
                                         (__bf16)x[4], (__bf16)x[5], (__bf16)x[6], (__bf16)x[7]};
}

// Operand from global row `row` (columns col..col+7) or zero past the last row.
template <typename T>
__device__ __forceinline__ typename Tr<T>::frag ldg_row_frag(const T* base, int ld, int row, int col, int nrows) {
  return row < nrows ? ldg_frag<T>(base + (size_t)row * ld + col) : zero_frag<T>();
}

// Four consecutive elements (LDS or global) as floats.
__device__ __forceinline__ f32x4 ld4f(const float* p) { return *reinterpret_cast<const f32x4*>(p); }
__device__ __forceinline__ f32x4 ld4f(const bf16_t* p) {
  const bf16x4 x = *reinterpret_cast<const bf16x4*>(p);
  return f32x4{(float)x[0], (float)x[1], (float)x[2], (float)x[3]};
}

// ------------------------------------------------------- gate absorbed into an operand
// The gate meets a GLA operand as src * e^x (raw q or k) or e^(src + x) (log features src); x is
// a difference of chunk-local cumulative log-gates.  Every kernel that must reproduce another's
// operand value bit for bit forms it through this one function.
template <bool FEAT>
__device__ __forceinline__ float gate_op(float src, float x) {
  if constexpr (FEAT)
    return __expf(src + x);
  else
    return src * __expf(x);
}

// ------------------------------------------------------- chunk-local gate prefix
// Thread map of a CHUNK x D tile: column group cg (VEC dims), tokens
// tg*TPT .. +TPT.  Computes the chunk-local inclusive prefix b of the
// log-gates held in rg (overwritten with b) and the chunk total Gamma.
template <int D, int VEC, int NT>
struct ScanMap {
  static constexpr int VPR = D / VEC;
  static constexpr int NTG = NT / VPR;
  static constexpr int TPT = CHUNK / NTG;
  static constexpr int GV = VEC / 4;
};

template <int D, int VEC, int NT, int TPT_, int GV_>
__device__ __forceinline__ void chunk_prefix(f32x4 (&rg)[TPT_][GV_], f32x4 (&tot)[GV_], float* sScan, int cg,
                                             int tg) {
  using SM = ScanMap<D, VEC, NT>;
  static_assert(SM::TPT == TPT_ && SM::GV == GV_, "scan map");
#pragma unroll
  for (int u = 1; u < SM::TPT; ++u)
#pragma unroll
    for (int e = 0; e < SM::GV; ++e) rg[u][e] += rg[u - 1][e];
#pragma unroll
  for (int e = 0; e < SM::GV; ++e)
    *reinterpret_cast<f32x4*>(sScan + tg * D + cg * VEC + 4 * e) = rg[SM::TPT - 1][e];
  __syncthreads();
  f32x4 excl[SM::GV];
#pragma unroll
  for (int e = 0; e < SM::GV; ++e) { excl[e] = f32x4{0, 0, 0, 0}; tot[e] = f32x4{0, 0, 0, 0}; }
  for (int p = 0; p < SM::NTG; ++p) {
#pragma unroll
    for (int e = 0; e < SM::GV; ++e) {
      const f32x4 x = *reinterpret_cast<const f32x4*>(sScan + p * D + cg * VEC + 4 * e);
      tot[e] += x;
      if (p < tg) excl[e] += x;
    }
  }
#pragma unroll
  for (int u = 0; u < SM::TPT; ++u)
#pragma unroll
    for (int e = 0; e < SM::GV; ++e) rg[u][e] += excl[e];
}

// ------------------------------------------------- gate prefix in column strips
// Block-local sums of a strip (see GateStrip below) for the sub-block form.  The 16 tokens of a
// 16-token block sit in four consecutive lanes of a row (tg & ~3 .. tg | 3, four tokens each).
// g[u] is replaced by P, the inclusive prefix of the log-gates inside the token's block; S[u]
// gets the exclusive suffix inside the block and T the block total.  Each is a sum of at most 16
// gates, so its rounding error is relative to its own size: exponents formed from them stay
// accurate however far the chunk-cumulative sum has fallen.
__device__ __forceinline__ void block_sums(f32x4 (&g)[4], f32x4 (&S)[4], f32x4& T, int lane) {
  f32x4 pin[4], sin[4];
  pin[0] = g[0];
#pragma unroll
  for (int u = 1; u < 4; ++u) pin[u] = pin[u - 1] + g[u];
  sin[3] = f32x4{0, 0, 0, 0};
#pragma unroll
  for (int u = 2; u >= 0; --u) sin[u] = sin[u + 1] + g[u + 1];
  const int q0 = lane & ~3, qi = lane & 3;
  f32x4 ep = f32x4{0, 0, 0, 0}, es = ep, tot = ep;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    f32x4 o;
#pragma unroll
    for (int e = 0; e < 4; ++e) o[e] = __shfl(pin[3][e], q0 + j, WAVE);
    tot += o;
    if (j < qi) ep += o;
    if (j > qi) es += o;
  }
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    g[u] = pin[u] + ep;
    S[u] = sin[u] + es;
  }
  T = tot;
}

// One wave handles a strip of 16 columns of a chunk: lane (tg = lane & 15,
// cg = lane >> 4) holds tokens 4*tg .. 4*tg+3 of columns col .. col+3 with
// col = 16*strip + 4*cg, so the chunk-local prefix over tokens is an
// in-thread sum plus a scan inside the 16-lane row (DPP): no LDS round trip,
// no barrier.
__device__ __forceinline__ bf16x4 ld4raw(const bf16_t* p) { return *reinterpret_cast<const bf16x4*>(p); }
__device__ __forceinline__ f32x4 ld4raw(const float* p) { return *reinterpret_cast<const f32x4*>(p); }

template <typename T>
struct GateStrip {
  using R4 = decltype(ld4raw(static_cast<const T*>(nullptr)));
  R4 q[4], k[4];   // raw q and k
  f32x4 g[4];      // log-gates, then the inclusive prefix b

  // SG: gp holds one gate per token (broadcast over the columns); else one per (token, column)
  template <bool SG>
  __device__ __forceinline__ void load(const T* qp, const T* kp, const float* gp, int D, int t0, int L, int col,
                                       int tg) {
    auto gate4 = [&](int t, size_t o) {
      if constexpr (SG) {
        const float x = gp[t];
        return f32x4{x, x, x, x};
      } else {
        return ld4raw(gp + o);
      }
    };
    if (t0 + CHUNK <= L) {
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int t = t0 + 4 * tg + u;
        const size_t o = (size_t)t * D + col;
        q[u] = ld4raw(qp + o);
        k[u] = ld4raw(kp + o);
        g[u] = gate4(t, o);
      }
    } else {
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int t = t0 + 4 * tg + u;
        const size_t o = (size_t)t * D + col;
        q[u] = t < L ? ld4raw(qp + o) : R4{};
        k[u] = t < L ? ld4raw(kp + o) : R4{};
        g[u] = t < L ? gate4(t, o) : f32x4{0, 0, 0, 0};
      }
    }
  }

  // q e^b, k e^-b and (if sEb) e^b into rows 4*tg+u, columns lcol .. lcol+3 of LDS tiles
  __device__ __forceinline__ void fold(T* sQt, T* sKh, T* sEb, int ldq, int lcol, int tg) {
#pragma unroll
    for (int u = 1; u < 4; ++u) g[u] += g[u - 1];
    f32x4 excl;
#pragma unroll
    for (int e = 0; e < 4; ++e) excl[e] = row_scan16(g[3][e]) - g[3][e];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      f32x4 eb, qt, kh;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float b = g[u][e] + excl[e];
        eb[e] = __expf(b);
        qt[e] = (float)q[u][e] * eb[e];
        kh[e] = (float)k[u][e] * __expf(-b);
      }
      const int row = (4 * tg + u) * ldq + lcol;
      st4(sQt + row, qt[0], qt[1], qt[2], qt[3]);
      st4(sKh + row, kh[0], kh[1], kh[2], kh[3]);
      if (sEb != nullptr) st4(sEb + row, eb[0], eb[1], eb[2], eb[3]);
    }
  }

  // Sub-block form (gates too strong for the chunk-start factoring): the block-local prefixes P to
  // sB, the block totals T to sBT (row kb), the keys folded to the end of their own block,
  // k e^S (S the block-local suffix, so at most |k|), to sKh, the raw q to sQr; sSpan[kb] gets
  // the largest decay inside block kb, -T, over the strip's 16 columns.
  __device__ __forceinline__ void fold_strong(T* sQr, T* sKh, int ldq, float* sB, int ldb, float* sBT, int D,
                                              float* sSpan, int lcol, int tg, int lane) {
    f32x4 S[4], Tb;
    block_sums(g, S, Tb, lane);
    float m = fmaxf(fmaxf(-Tb[0], -Tb[1]), fmaxf(-Tb[2], -Tb[3]));
    m = xor_max(xor_max(m, 16), 32);
    if ((lane & 51) == 0) sSpan[tg >> 2] = m;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int row = 4 * tg + u;
      *reinterpret_cast<f32x4*>(sB + row * ldb + lcol) = g[u];
      f32x4 kh;
#pragma unroll
      for (int e = 0; e < 4; ++e) kh[e] = gate_op<false>((float)k[u][e], S[u][e]);
      st4(sKh + row * ldq + lcol, kh[0], kh[1], kh[2], kh[3]);
      st4(sQr + row * ldq + lcol, (float)q[u][0], (float)q[u][1], (float)q[u][2], (float)q[u][3]);
    }
    if ((tg & 3) == 0) *reinterpret_cast<f32x4*>(sBT + (tg >> 2) * D + lcol) = Tb;
  }
};

// The same strip for log features lq, lk (fp32) of the GLA branch: the gate is absorbed in log
// space, q~ = exp(lq + b), k^ = exp(lk - b).  Rows past the sequence end are loaded clamped and
// given l = -inf at the fold, so their q~, k^ are exactly zero as in the raw form.
template <typename T>
struct GateStripLog {
  f32x4 q[4], k[4];   // log features
  f32x4 g[4];         // log-gates, then the inclusive prefix b
  int nvalid;         // rows of this strip inside the sequence

  template <bool SG>
  __device__ __forceinline__ void load(const float* qp, const float* kp, const float* gp, int D, int t0, int L,
                                       int col, int tg) {
    static_assert(!SG, "log features are taken with per-dimension gates");
    nvalid = L - t0 - 4 * tg;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const size_t o = (size_t)min(t0 + 4 * tg + u, L - 1) * D + col;
      q[u] = ld4raw(qp + o);
      k[u] = ld4raw(kp + o);
      g[u] = ld4raw(gp + o);
    }
#pragma unroll
    for (int u = 0; u < 4; ++u)
      if (u >= nvalid) g[u] = f32x4{0, 0, 0, 0};   // no decay past the end (b stays finite)
  }

  __device__ __forceinline__ void fold(T* sQt, T* sKh, T* sEb, int ldq, int lcol, int tg) {
#pragma unroll
    for (int u = 1; u < 4; ++u) g[u] += g[u - 1];
    f32x4 excl;
#pragma unroll
    for (int e = 0; e < 4; ++e) excl[e] = row_scan16(g[3][e]) - g[3][e];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const bool ok = u < nvalid;
      f32x4 eb, qt, kh;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float b = g[u][e] + excl[e];
        eb[e] = __expf(b);
        qt[e] = __expf((ok ? q[u][e] : -INFINITY) + b);
        kh[e] = __expf((ok ? k[u][e] : -INFINITY) - b);
      }
      const int row = (4 * tg + u) * ldq + lcol;
      st4(sQt + row, qt[0], qt[1], qt[2], qt[3]);
      st4(sKh + row, kh[0], kh[1], kh[2], kh[3]);
      if (sEb != nullptr) st4(sEb + row, eb[0], eb[1], eb[2], eb[3]);
    }
  }

  // Sub-block form as for GateStrip (the log-feature queries are read where they are used).
  __device__ __forceinline__ void fold_strong(T*, T* sKh, int ldq, float* sB, int ldb, float* sBT, int D,
                                              float* sSpan, int lcol, int tg, int lane) {
    f32x4 S[4], Tb;
    block_sums(g, S, Tb, lane);
    float m = fmaxf(fmaxf(-Tb[0], -Tb[1]), fmaxf(-Tb[2], -Tb[3]));
    m = xor_max(xor_max(m, 16), 32);
    if ((lane & 51) == 0) sSpan[tg >> 2] = m;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int row = 4 * tg + u;
      const bool ok = u < nvalid;
      *reinterpret_cast<f32x4*>(sB + row * ldb + lcol) = g[u];
      f32x4 kh;
#pragma unroll
      for (int e = 0; e < 4; ++e) kh[e] = gate_op<true>(ok ? k[u][e] : -INFINITY, S[u][e]);
      st4(sKh + row * ldq + lcol, kh[0], kh[1], kh[2], kh[3]);
    }
    if ((tg & 3) == 0) *reinterpret_cast<f32x4*>(sBT + (tg >> 2) * D + lcol) = Tb;
  }
};

}  // namespace lz
