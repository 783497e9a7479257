// Device-side helpers for the gfx950 kernels: matrix-core operand types, the
// code-word layout (record layout v2) and codebook lookups.
//
// Operand layouts of v_mfma_f32_16x16x32_f16 (wave64), used everywhere:
//   A (16 x 32): lane l holds row l%16, k = 8*(l/16) .. +7   (8 fp16)
//   B (32 x 16): lane l holds column l%16, k = 8*(l/16) .. +7
//   D (16 x 16): lane l holds column l%16, rows 4*(l/16) + i, i = 0..3
// Which actual coordinate/token sits in each k slot is a free choice as long
// as A and B agree; the choices below make every pack and unpack lane-local.
#pragma once

#include <hip/hip_runtime.h>
#include <cstdint>

#include "tq_internal.h"

namespace tq {

typedef _Float16 h8 __attribute__((ext_vector_type(8)));
typedef float f4 __attribute__((ext_vector_type(4)));
typedef uint32_t u4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ f4 mfma(const h8& a, const h8& b, const f4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

// v_mfma_f32_32x32x16_f16 (wave64):
//   A (32 x 16): lane l holds row l%32, k = 8*(l/32) .. +7
//   B (16 x 32): lane l holds column l%32, k = 8*(l/32) .. +7
//   D (32 x 32): lane l holds column l%32, rows 8 j + 4*(l/32) + i at acc[4 j + i]
typedef float f16v __attribute__((ext_vector_type(16)));
__device__ __forceinline__ f16v mfma32(const h8& a, const h8& b, const f16v& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f4 quarter(const f16v& v, int j) {
  return f4{v[4 * j], v[4 * j + 1], v[4 * j + 2], v[4 * j + 3]};
}

__device__ __forceinline__ h8 as_h8(const u4& v) { return __builtin_bit_cast(h8, v); }
__device__ __forceinline__ u4 as_u4(const h8& v) { return __builtin_bit_cast(u4, v); }

__device__ __forceinline__ uint32_t perm(uint32_t hi, uint32_t lo, uint32_t sel) {
  return __builtin_amdgcn_perm(hi, lo, sel);
}

// ---- code words ---------------------------------------------------------------
// A group of b 32-bit words holds the b-bit codes of 8 "slots" s = 0..7 of 4
// byte lanes i = 0..3 each (32 codes).  The byte lane i of every word belongs
// to code (s, i).  Within a byte lane:
//   b = 1: bit s of word 0
//   b = 2: bits 2(s%4).. of word s/4
//   b = 4: bits 4(s%2).. of word s/2
//   b = 3: s < 6: bits 3(s%2).. of word s/2;
//          s = 6: code bits 0,1 at bits 6,7 of word 0, code bit 2 at bit 6 of word 2
//          s = 7: code bits 0,1 at bits 6,7 of word 1, code bit 2 at bit 7 of word 2
// so that the 4 codes of a slot come out as one byte-per-code selector word
// ("sel4") in one or two ALU operations.

// OR the selector word x (code of byte lane i in byte i) into slot S.
template <int B, int S>
__device__ __forceinline__ void put_sel4(uint32_t (&w)[B], uint32_t x) {
  if constexpr (B == 1) {
    w[0] |= x << S;
  } else if constexpr (B == 2) {
    w[S / 4] |= x << (2 * (S % 4));
  } else if constexpr (B == 4) {
    w[S / 2] |= x << (4 * (S % 2));
  } else {
    static_assert(B == 3, "bits must be 1..4");
    if constexpr (S < 6) {
      w[S / 2] |= x << (3 * (S % 2));
    } else if constexpr (S == 6) {
      w[0] |= (x & 0x03030303u) << 6;
      w[2] |= (x & 0x04040404u) << 4;
    } else {
      w[1] |= (x & 0x03030303u) << 6;
      w[2] |= (x & 0x04040404u) << 5;
    }
  }
}

// Extract the selector word of slot S.
template <int B, int S>
__device__ __forceinline__ uint32_t get_sel4(const uint32_t (&w)[B]) {
  if constexpr (B == 1) {
    return (w[0] >> S) & 0x01010101u;
  } else if constexpr (B == 2) {
    return (w[S / 4] >> (2 * (S % 4))) & 0x03030303u;
  } else if constexpr (B == 4) {
    return (w[S / 2] >> (4 * (S % 2))) & 0x0F0F0F0Fu;
  } else {
    if constexpr (S < 6) {
      return (w[S / 2] >> (3 * (S % 2))) & 0x07070707u;
    } else if constexpr (S == 6) {
      return ((w[0] >> 6) & 0x03030303u) | ((w[2] >> 4) & 0x04040404u);
    } else {
      return ((w[1] >> 6) & 0x03030303u) | ((w[2] >> 5) & 0x04040404u);
    }
  }
}

// Field mask (all bits) of slot S in word W, byte lane I.
template <int B, int S, int W, int I>
__device__ __forceinline__ constexpr uint32_t field_mask() {
  uint32_t m = 0;
  if constexpr (B == 1) {
    if (W == 0) m = 1u << S;
  } else if constexpr (B == 2) {
    if (W == S / 4) m = 3u << (2 * (S % 4));
  } else if constexpr (B == 4) {
    if (W == S / 2) m = 15u << (4 * (S % 2));
  } else {
    if (S < 6) {
      if (W == S / 2) m = 7u << (3 * (S % 2));
    } else if (S == 6) {
      if (W == 0) m = 3u << 6;
      if (W == 2) m = 1u << 6;
    } else {
      if (W == 1) m = 3u << 6;
      if (W == 2) m = 1u << 7;
    }
  }
  return m << (8 * I);
}

// Field mask of (slot s, word w, byte lane i) for b-bit codes (runtime form).
__device__ __forceinline__ uint32_t field_mask_rt(int b, int s, int w, int i) {
  uint32_t m = 0;
  if (b == 1) {
    if (w == 0) m = 1u << s;
  } else if (b == 2) {
    if (w == s / 4) m = 3u << (2 * (s % 4));
  } else if (b == 4) {
    if (w == s / 2) m = 15u << (4 * (s % 2));
  } else {
    if (s < 6) {
      if (w == s / 2) m = 7u << (3 * (s % 2));
    } else if (s == 6) {
      if (w == 0) m = 3u << 6;
      if (w == 2) m = 1u << 6;
    } else {
      if (w == 1) m = 3u << 6;
      if (w == 2) m = 1u << 7;
    }
  }
  return m << (8 * i);
}

// Decode a selector word into 4 fp16 centroids: two registers holding
// (c[code0], c[code1]) and (c[code2], c[code3]).  tlo/thi hold the low/high
// bytes of the fp16 centroid table (entry v at byte v).
template <int B>
__device__ __forceinline__ void decode4(uint32_t sel, const uint32_t (&tlo)[4], const uint32_t (&thi)[4],
                                        uint32_t& p01, uint32_t& p23) {
  uint32_t lo, hi;
  if constexpr (B <= 3) {
    lo = perm(tlo[1], tlo[0], sel);
    hi = perm(thi[1], thi[0], sel);
  } else {
    // The codebook is symmetric (c[v] = -c[15 - v], exactly: the loaded
    // centroids are symmetrised), so only its positive half (entries 8..15,
    // tlo/thi[2..3]) is read: code v >= 8 is c[v], code v < 8 is -c[15 - v],
    // whose magnitude index 7 - v is (v & 7) ^ 7 and whose sign is the top
    // bit of the high byte.
    const uint32_t neg = (~sel >> 3) & 0x01010101u;  // 1 in the bytes of codes < 8
    const uint32_t mag = (sel & 0x07070707u) ^ (neg * 7u);
    lo = perm(tlo[3], tlo[2], mag);
    hi = perm(thi[3], thi[2], mag) | (neg << 7);
  }
  p01 = perm(hi, lo, 0x05010400u);
  p23 = perm(hi, lo, 0x07030602u);
}

// Decode slots S0 and S1 (= S0 + 1) into one 8-element fp16 operand:
// elements 0..3 = slot S0 byte lanes 0..3, elements 4..7 = slot S1.
template <int B, int S0>
__device__ __forceinline__ h8 decode_pair(const uint32_t (&w)[B], const uint32_t (&tlo)[4],
                                          const uint32_t (&thi)[4]) {
  uint32_t r0, r1, r2, r3;
  decode4<B>(get_sel4<B, S0>(w), tlo, thi, r0, r1);
  decode4<B>(get_sel4<B, S0 + 1>(w), tlo, thi, r2, r3);
  return as_h8(u4{r0, r1, r2, r3});
}

// ---- 3-bit code groups decoded through LDS pair tables ----------------------
// A byte lane of a 3-bit group holds the codes of slots 2p and 2p + 1 in bits
// 0-5 of word p (p < 3); slots 6 and 7 keep bits 0-1 in bits 6-7 of words 0
// and 1 and bit 2 in bits 6 and 7 of word 2.  A 64-entry table of fp16 pairs
// turns one 6-bit index into both centroids with one 4-byte LDS read, so a
// pair of codes costs 1.5 ALU operations for p < 3 instead of 3 with byte
// permutes.  The 64 entries of a table sit in distinct LDS banks, so lanes
// only ever share a bank when they read the same entry (a broadcast).
//   t01[e] = (c[e & 7], c[e >> 3])
//   t67[e] = (c[(e & 3) | (e >> 2 & 4)], c[(e >> 2 & 3) | (e >> 3 & 4)]),
//            e = w0 bits 6-7 | w1 bits 6-7 << 2 | w2 bits 6-7 << 4
struct PairTables {
  uint32_t t01[64];
  uint32_t t67[64];
};

// Threads tid = 0..127 each write one entry (the caller synchronises).
__device__ __forceinline__ void fill_pair_tables(PairTables& t, const uint32_t (&tlo)[4], const uint32_t (&thi)[4],
                                                 int tid) {
  auto c16 = [&](uint32_t v) -> uint32_t {  // fp16 bits of centroid v < 8
    const uint32_t lo = (tlo[v >> 2] >> (8 * (v & 3))) & 0xFFu, hi = (thi[v >> 2] >> (8 * (v & 3))) & 0xFFu;
    return lo | hi << 8;
  };
  const uint32_t e = (uint32_t)tid & 63;
  if (tid >= 0 && tid < 64) t.t01[e] = c16(e & 7) | c16(e >> 3) << 16;
  else if (tid >= 64 && tid < 128) t.t67[e] = c16((e & 3) | (e >> 2 & 4)) | c16((e >> 2 & 3) | (e >> 3 & 4)) << 16;
}

// Word whose byte i is the byte address 4 e of pair P's table entry for byte
// lane i.
template <int P>
__device__ __forceinline__ uint32_t pair_addr4(const uint32_t (&w)[3]) {
  if constexpr (P < 3) {
    return (w[P] << 2) & 0xFCFCFCFCu;
  } else {
    return ((w[0] >> 4) & 0x0C0C0C0Cu) | ((w[1] >> 2) & 0x30303030u) | (w[2] & 0xC0C0C0C0u);
  }
}

// The 8 centroids of slots 2P, 2P + 1 as one fp16 operand in pair order:
// element 2 i = slot 2P, byte lane i; element 2 i + 1 = slot 2P + 1, lane i.
template <int P>
__device__ __forceinline__ h8 decode_pair_lds(const uint32_t (&w)[3], const PairTables& t) {
  const uint32_t a = pair_addr4<P>(w);
  const char* base = (const char*)(P < 3 ? t.t01 : t.t67);
  // byte i of a, zero-extended, by one byte permute each (shift-and-mask
  // forms get re-derived from w by the compiler at two operations apiece)
  u4 r;
  r[0] = *(const uint32_t*)(base + perm(0u, a, 0x0C0C0C00u));
  r[1] = *(const uint32_t*)(base + perm(0u, a, 0x0C0C0C01u));
  r[2] = *(const uint32_t*)(base + perm(0u, a, 0x0C0C0C02u));
  r[3] = *(const uint32_t*)(base + perm(0u, a, 0x0C0C0C03u));
  return as_h8(r);
}

// Reorder an operand built in slot order (elements 0-3 = slot 2P lanes 0-3,
// 4-7 = slot 2P + 1) into the pair order of decode_pair_lds.
__device__ __forceinline__ h8 to_pair_order(const h8& x) {
  const u4 v = as_u4(x);
  return as_h8(u4{perm(v[2], v[0], 0x05040100u), perm(v[2], v[0], 0x07060302u), perm(v[3], v[1], 0x05040100u),
                  perm(v[3], v[1], 0x07060302u)});
}

// Lloyd-Max cell of y: idx = #{i : beta_i < y} by binary search over the
// sorted boundaries (beta in registers / kernel arguments).
template <int B>
__device__ __forceinline__ int bucket(float y, const float (&beta)[15]) {
  if constexpr (B == 1) {
    return y > beta[0] ? 1 : 0;
  } else if constexpr (B == 2) {
    const bool m1 = y > beta[1];
    const float t = m1 ? beta[2] : beta[0];
    const bool m0 = y > t;
    return (m1 ? 2 : 0) + (m0 ? 1 : 0);
  } else if constexpr (B == 3) {
    const bool m2 = y > beta[3];
    const float t1 = m2 ? beta[5] : beta[1];
    const bool m1 = y > t1;
    const float t0 = m2 ? (m1 ? beta[6] : beta[4]) : (m1 ? beta[2] : beta[0]);
    const bool m0 = y > t0;
    return (m2 ? 4 : 0) + (m1 ? 2 : 0) + (m0 ? 1 : 0);
  } else {
    // value selects only (a select of two array addresses would force the
    // boundary array into scratch memory)
    const float b0 = beta[0], b1 = beta[1], b2 = beta[2], b3 = beta[3], b4 = beta[4], b5 = beta[5];
    const float b6 = beta[6], b7 = beta[7], b8 = beta[8], b9 = beta[9], b10 = beta[10], b11 = beta[11];
    const float b12 = beta[12], b13 = beta[13], b14 = beta[14];
    const bool m3 = y > b7;
    const float t2 = m3 ? b11 : b3;
    const bool m2 = y > t2;
    const float t1 = m3 ? (m2 ? b13 : b9) : (m2 ? b5 : b1);
    const bool m1 = y > t1;
    const float ta = m1 ? b14 : b12, tb = m1 ? b10 : b8;
    const float tc = m1 ? b6 : b4, te = m1 ? b2 : b0;
    const float t0 = m3 ? (m2 ? ta : tb) : (m2 ? tc : te);
    const bool m0 = y > t0;
    return (m3 ? 8 : 0) + (m2 ? 4 : 0) + (m1 ? 2 : 0) + (m0 ? 1 : 0);
  }
}


// Lloyd-Max cell of y for a codebook symmetric about 0 (c_i = -c_{L-1-i},
// middle boundary 0): with k = #{j : |y| > beta+_j} over the H-1 positive
// boundaries (H = L/2), idx = H + k for y > 0 and H - 1 - k otherwise, i.e.
// idx = k ^ (y > 0 ? H : H-1).  bp[j] = beta_{H + j}.  Compare + add-with-
// carry per boundary, no selects and no branches.
template <int B>
__device__ __forceinline__ int bucket_sym(float y, const float (&bp)[8]) {
  constexpr int H = 1 << (B - 1);
  const float a = fabsf(y);
  int k = 0;
#pragma unroll
  for (int j = 0; j < H - 1; ++j) k += a > bp[j] ? 1 : 0;
  return k ^ (y > 0.f ? H : H - 1);
}

// Split two fp32 values into fp16 high parts (round toward zero) and fp16
// low parts (the exact remainders, rounded): x = hi + lo to ~2^-22 relative.
struct HiLo {
  uint32_t hi, lo;
};
__device__ __forceinline__ HiLo split2(float x0, float x1) {
  const auto h = __builtin_amdgcn_cvt_pkrtz(x0, x1);
  const auto l = __builtin_amdgcn_cvt_pkrtz(x0 - (float)h[0], x1 - (float)h[1]);
  return HiLo{__builtin_bit_cast(uint32_t, h), __builtin_bit_cast(uint32_t, l)};
}

__device__ __forceinline__ float shfl_xor(float v, int mask) { return __shfl_xor(v, mask, 64); }

// 2^x on the hardware exponential unit (one v_exp_f32, no range fix-ups):
// results below the normal fp32 range come out as 0, which softmax weights
// and rescale factors tolerate.
__device__ __forceinline__ float exp2_hw(float x) { return __builtin_amdgcn_exp2f(x); }

// Cross-lane maxima without LDS.  dpp_f<CTRL> reads another lane of the same
// 16-lane row (quad_perm 0xB1 / 0x4E = lane ^ 1 / ^ 2, 0x124 / 0x128 = row
// rotate by 4 / 8).  v_permlane16_swap and v_permlane32_swap exchange whole
// rows: with both operands v, one result holds v of lane l ^ 16 (or l ^ 32)
// where the other holds v of lane l, so their maximum reduces across rows.
template <int CTRL>
__device__ __forceinline__ float dpp_f(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}
// DPP move of src into the lanes of old selected by BANK (bit b = lanes
// 4b .. 4b + 3 of every 16-lane row); lanes left out, or whose source lies
// outside the row, keep old.  CTRL: row_shl:n = 0x100 + n (read lane + n),
// row_shr:n = 0x110 + n (read lane - n).
template <int CTRL, int BANK>
__device__ __forceinline__ uint32_t dpp_into(uint32_t old, uint32_t src) {
  return (uint32_t)__builtin_amdgcn_update_dpp((int)old, (int)src, CTRL, 0xF, BANK, false);
}
template <int CTRL, int BANK>
__device__ __forceinline__ float dpp_into(float old, float src) {
  return __uint_as_float(dpp_into<CTRL, BANK>(__float_as_uint(old), __float_as_uint(src)));
}

__device__ __forceinline__ float max_xor16_32(float v) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}
__device__ __forceinline__ float wave_max(float v) {
  v = fmaxf(v, dpp_f<0xB1>(v));
  v = fmaxf(v, dpp_f<0x4E>(v));
  v = fmaxf(v, dpp_f<0x124>(v));
  v = fmaxf(v, dpp_f<0x128>(v));
  return max_xor16_32(v);
}

// Runtime-slot form of put_sel4 (the switch folds away when s is a constant).
template <int B>
__device__ __forceinline__ void put_sel4_rt(uint32_t (&w)[B], int s, uint32_t x) {
  switch (s) {
    case 0: put_sel4<B, 0>(w, x); break;
    case 1: put_sel4<B, 1>(w, x); break;
    case 2: put_sel4<B, 2>(w, x); break;
    case 3: put_sel4<B, 3>(w, x); break;
    case 4: put_sel4<B, 4>(w, x); break;
    case 5: put_sel4<B, 5>(w, x); break;
    case 6: put_sel4<B, 6>(w, x); break;
    default: put_sel4<B, 7>(w, x); break;
  }
}

// ---- quantisation helpers -----------------------------------------------------

typedef _Float16 h2 __attribute__((ext_vector_type(2)));

// Norms of finite fp32 rows at any magnitude.  e = pow2_exponent(max |x|)
// gives max |x| in [2^(e-1), 2^e) (0 for a zero row); the scaled coordinates
// ldexp(x, -e) are exact and their sum of squares lies in [2^-2, n], so it
// neither overflows nor underflows, and ||x|| = ldexp(sqrt(sum), e).
__device__ __forceinline__ int pow2_exponent(float a) {
  int e = 0;
  frexpf(a, &e);
  return a > 0.f ? e : 0;
}

// One-pass form for block reductions: a partial (e, s) stands for a sum of
// squares s 2^(2e) with s taken over coordinates shifted by 2^-e, e the
// exponent of the partial's largest magnitude (kNoExp for a zero partial, so
// that it never sets the exponent).  Two partials merge exactly at the larger
// exponent; the merged e is that of the whole row's largest magnitude, and
// ||x|| = ldexp(sqrt(s), e).
constexpr int kNoExp = -1000;
__device__ __forceinline__ void norm2_partial(float mx, int& e) { e = mx > 0.f ? pow2_exponent(mx) : kNoExp; }
__device__ __forceinline__ void merge_norm2(int& e, float& s, int e2, float s2) {
  const int E = e > e2 ? e : e2;
  s = ldexpf(s, 2 * (e - E)) + ldexpf(s2, 2 * (e2 - E));
  e = E;
}
__device__ __forceinline__ void wave_norm2(int& e, float& s) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) merge_norm2(e, s, __shfl_xor(e, o, 64), __shfl_xor(s, o, 64));
}

// The fp32 input pre-scale of the matrix-core kernels: the row is brought to
// |x| < 2^13 (fp16 hi/lo operands) by ldexp(x, input_shift(||x||)), an exact
// power-of-two shift that, unlike a multiply by 2^(13 - E), cannot overflow
// for tiny norms.
__device__ __forceinline__ int input_shift(float n) {
  int E = 0;
  frexpf(n, &E);
  return n > 0.f ? 13 - E : 0;
}

// Partial sum of squares of 32 fp16 coordinates (dot2 with fp32 accumulation;
// the fp16 x fp16 products are exact).
__device__ __forceinline__ float sq_norm16(const h8 (&x)[4]) {
  float s[2] = {0.f, 0.f};
#pragma unroll
  for (int kb = 0; kb < 4; ++kb)
#pragma unroll
    for (int e = 0; e < 8; e += 2) {
      const h2 v = {x[kb][e], x[kb][e + 1]};
      s[kb & 1] = __builtin_amdgcn_fdot2(v, v, s[kb & 1], false);
    }
  return s[0] + s[1];
}

// Lloyd-Max cells of 4 coordinates of one token, with the residual, for a
// codebook symmetric about 0 (H = L/2 cells per side, middle boundary 0).
//   a     scaled rotated coordinates, a = sigma y with sigma = 2^8 ||k|| (> 0)
//   bs    the positive boundaries beta_{H+t} scaled by sigma (t < H-1)
//   s16   2^12 / sigma, so that a s16 = 2^12 y (0 for a zero vector)
//   ctab  LDS table of 2^12 c_i at byte offset 4 i
// With k = #{t : |a| > bs_t}, the cell is H + k for a > 0 and H - 1 - k for
// a <= 0 (the same count as #{i : beta_i < y}).  Both come out of one select
// chain on the byte address 4 (H + k), reflected to 4 (H - 1 - k) for
// a <= 0 by an XOR with all ones (a - 1 as an integer is negative exactly
// for a <= 0, since a = -0 cannot come out of an accumulation from +0).
// r_i = 2^12 (y_i - c[idx_i]); g2 += sum r_i^2.  Returns the selector word
// (cell of coordinate i in byte i).
template <int B>
__device__ __forceinline__ uint32_t quantize4(const f4& a, const float (&bs)[8], float s16, const float* ctab,
                                              float (&r)[4], float& g2) {
  constexpr uint32_t H = 1u << (B - 1);
  constexpr uint32_t kMask = 4u * (2u * H - 1u);
  uint32_t ia[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float m = fabsf(a[i]);
    uint32_t ad = 4u * H;
#pragma unroll
    for (uint32_t t = 0; t + 1 < H; ++t) ad = m > bs[t] ? 4u * (H + 1u + t) : ad;
    const uint32_t neg = (uint32_t)((int32_t)(__float_as_uint(a[i]) - 1u) >> 31);
    ia[i] = (ad ^ neg) & kMask;
    const float c = *(const float*)((const char*)ctab + ia[i]);
    r[i] = fmaf(a[i], s16, -c);
    g2 = fmaf(r[i], r[i], g2);
  }
  return (perm(ia[1], ia[0], 0x0C0C0400u) | perm(ia[3], ia[2], 0x04000C0Cu)) >> 2;
}

// quantize4 with the sign handled once for four coordinates, returning the
// NEGATED scaled residual rn = -2^12 (y - c[idx]) (one bit insert and one
// FMA per coordinate; the caller projects rn and reads the sign bits with
// the opposite polarity, sign_bits16_neg).  The select chain gives the byte
// address 4 (H + k) of the positive centroid c[H + k] = c+_k, and
// copysign(c+_k, a) is the signed centroid of a's cell.  The cells H + k are
// reflected to H - 1 - k where a's sign bit is set by one bitop3 on the
// four code bytes, with the sign mask from v_perm's sign-replicating
// selectors.  ns16 = -2^12 / sigma.  A coordinate that is exactly +0 lands
// in cell H (residual -c+_0) instead of H - 1: it lies on the middle
// boundary, where either cell is within the code tolerance, and a token of
// zero norm (all coordinates +0) is set right by its caller.
template <int B>
__device__ __forceinline__ uint32_t quantize4_signs(const f4& a, const float (&bs)[8], float ns16, const float* ctab,
                                                    float (&rn)[4], float& g2) {
  constexpr uint32_t H = 1u << (B - 1);
  uint32_t ad[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float m = fabsf(a[i]);
    uint32_t c = 4u * H;
#pragma unroll
    for (uint32_t t = 0; t + 1 < H; ++t) c = m > bs[t] ? 4u * (H + 1u + t) : c;
    ad[i] = c;
    const float cp = *(const float*)((const char*)ctab + c);
    rn[i] = fmaf(a[i], ns16, __builtin_copysignf(cp, a[i]));
    g2 = fmaf(rn[i], rn[i], g2);
  }
  const uint32_t mag = (perm(ad[1], ad[0], 0x0C0C0400u) | perm(ad[3], ad[2], 0x04000C0Cu)) >> 2;
  const uint32_t neg = perm(__float_as_uint(a[1]), __float_as_uint(a[0]), 0x0C0C0B09u) |
                       perm(__float_as_uint(a[3]), __float_as_uint(a[2]), 0x0B090C0Cu);
  return mag ^ (neg & ((2u * H - 1u) * 0x01010101u));
}

// Code words of a b-bit group whose 32 codes all equal v (v < 2^b).
template <int B>
__device__ __forceinline__ void fill_code_words(uint32_t (&w)[B], uint32_t v) {
  const uint32_t x = v * 0x01010101u;
#pragma unroll
  for (int k = 0; k < B; ++k) w[k] = 0u;
  put_sel4<B, 0>(w, x);
  put_sel4<B, 1>(w, x);
  put_sel4<B, 2>(w, x);
  put_sel4<B, 3>(w, x);
  put_sel4<B, 4>(w, x);
  put_sel4<B, 5>(w, x);
  put_sel4<B, 6>(w, x);
  put_sel4<B, 7>(w, x);
}

// Cells of 4 coordinates without the residual (the value path): a_i are
// scaled rotated coordinates sigma_i y_i and bs[i][t] = beta_{H+t} sigma_i
// the matching scaled positive boundaries (one token per i).  Same select
// chain and reflection as quantize4; returns the selector word.
template <int B>
__device__ __forceinline__ uint32_t cells4(const f4& a, const float (&bs)[4][8]) {
  constexpr uint32_t H = 1u << (B - 1);
  uint32_t ia[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float m = fabsf(a[i]);
    uint32_t ad = H;
#pragma unroll
    for (uint32_t t = 0; t + 1 < H; ++t) ad = m > bs[i][t] ? H + 1u + t : ad;
    const uint32_t neg = (uint32_t)((int32_t)(__float_as_uint(a[i]) - 1u) >> 31);
    ia[i] = (ad ^ neg) & (2u * H - 1u);
  }
  return perm(ia[1], ia[0], 0x0C0C0400u) | perm(ia[3], ia[2], 0x04000C0Cu);
}

// cells4 with the reflection done once for all four coordinates: the select
// chains give the magnitude cells H + k, v_perm's sign-replicating
// selectors give a byte mask of the coordinates whose sign bit is set, one
// bitop3 reflects those cells to H - 1 - k, and zmask (bytes 0xFF for the
// tokens of zero norm, whose coordinates are all +0 and belong to cell
// H - 1) overrides those tokens.  A coordinate that comes out exactly +0 in
// a token of nonzero norm gets cell H rather than H - 1; it lies on the
// middle boundary, where either cell is within the code tolerance.
template <int B>
__device__ __forceinline__ uint32_t cells4_signs(const f4& a, const float (&bs)[4][8], uint32_t zmask) {
  constexpr uint32_t H = 1u << (B - 1);
  uint32_t ad[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float m = fabsf(a[i]);
    uint32_t c = H;
#pragma unroll
    for (uint32_t t = 0; t + 1 < H; ++t) c = m > bs[i][t] ? H + 1u + t : c;
    ad[i] = c;
  }
  const uint32_t mag = perm(ad[1], ad[0], 0x0C0C0400u) | perm(ad[3], ad[2], 0x04000C0Cu);
  const uint32_t neg = perm(__float_as_uint(a[1]), __float_as_uint(a[0]), 0x0C0C0B09u) |
                       perm(__float_as_uint(a[3]), __float_as_uint(a[2]), 0x0B090C0Cu);
  const uint32_t code = mag ^ (neg & ((2u * H - 1u) * 0x01010101u));
  return (code & ~zmask) | ((H - 1u) * 0x01010101u & zmask);
}

// Split x0, x1 into fp16 high parts (round toward zero) and fp16 low parts
// (the remainders, rounded): x = hi + lo to ~2^-22 relative.  m1 must be the
// fp16 value -1 passed in at run time: with a constant the compiler turns
// the remainder into a subtract plus conversions instead of one mixed FMA.
__device__ __forceinline__ HiLo split2m(float x0, float x1, _Float16 m1) {
  const auto h = __builtin_amdgcn_cvt_pkrtz(x0, x1);
  h2 l;
  l[0] = (_Float16)fmaf((float)h[0], (float)m1, x0);
  l[1] = (_Float16)fmaf((float)h[1], (float)m1, x1);
  return HiLo{__builtin_bit_cast(uint32_t, h), __builtin_bit_cast(uint32_t, l)};
}

// QJL sign bits [z >= 0] of 16 projections, bit 4 p + i for z[p][i]:
// v_perm's sign-replicating selectors turn 4 sign bits into byte masks,
// each byte keeps one distinct bit, and a sum of bytes (v_sad_u8 against 0)
// gathers them.  (z = -0 cannot come out of an accumulation from +0.)
__device__ __forceinline__ uint32_t sign_bits16(const f4& z0, const f4& z1, const f4& z2, const f4& z3) {
  auto keep = [](const f4& z, uint32_t bits) {
    const uint32_t m = perm(__float_as_uint(z[1]), __float_as_uint(z[0]), 0x0C0C0B09u) |
                       perm(__float_as_uint(z[3]), __float_as_uint(z[2]), 0x0B090C0Cu);
    return ~m & bits;
  };
  const uint32_t lo =
      __builtin_amdgcn_sad_u8(keep(z1, 0x80402010u), 0u, __builtin_amdgcn_sad_u8(keep(z0, 0x08040201u), 0u, 0u));
  const uint32_t hi =
      __builtin_amdgcn_sad_u8(keep(z3, 0x80402010u), 0u, __builtin_amdgcn_sad_u8(keep(z2, 0x08040201u), 0u, 0u));
  return lo | (hi << 8);
}

// sign_bits16 for the projections zn = -z of a negated residual: bit 4 p + i
// is set where zn[p][i] has its sign bit set, i.e. z > 0 (the same as
// [z >= 0] except at z = 0 exactly, which lies on the sign tolerance).
__device__ __forceinline__ uint32_t sign_bits16_neg(const f4& z0, const f4& z1, const f4& z2, const f4& z3) {
  auto keep = [](const f4& z, uint32_t bits) {
    const uint32_t m = perm(__float_as_uint(z[1]), __float_as_uint(z[0]), 0x0C0C0B09u) |
                       perm(__float_as_uint(z[3]), __float_as_uint(z[2]), 0x0B090C0Cu);
    return m & bits;
  };
  const uint32_t lo =
      __builtin_amdgcn_sad_u8(keep(z1, 0x80402010u), 0u, __builtin_amdgcn_sad_u8(keep(z0, 0x08040201u), 0u, 0u));
  const uint32_t hi =
      __builtin_amdgcn_sad_u8(keep(z3, 0x80402010u), 0u, __builtin_amdgcn_sad_u8(keep(z2, 0x08040201u), 0u, 0u));
  return lo | (hi << 8);
}

// Copy the boundaries out of the kernel-argument block into registers.
__device__ __forceinline__ void load_beta(float (&beta)[15], const CodebookDev& cb) {
#pragma unroll
  for (int i = 0; i < 15; ++i) beta[i] = cb.beta[i];
}

// The positive boundaries beta_{H}, beta_{H+1}, ... of a symmetric codebook.
template <int B>
__device__ __forceinline__ void load_pos_beta(float (&bp)[8], const CodebookDev& cb) {
  constexpr int H = 1 << (B - 1);
#pragma unroll
  for (int j = 0; j < 8; ++j) bp[j] = j < H - 1 ? cb.beta[H + j] : INFINITY;
}

}  // namespace tq
