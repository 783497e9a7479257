// Compression kernels for gfx950: keys (stage 1 + stage 2) and values
// (stage 1), head_dim 128.
//
// Stage 1 (nav.superapi.store "turboquant-pytorch", 主要能力; atskills.one
// "turboquant-pytorch", Stage 1): y = R k / ||k||, idx_j = #{i : beta_i < y_j}.
// Stage 2, keys only (same sections, Stage 2 / 第二阶段; 算法细节: keys need
// QJL, values do not): r = y - c[idx], gamma = ||r||, s = [S r >= 0].
//
// Arithmetic.  The codes must agree with an fp64 evaluation except within
// ~1e-7 of a boundary, so the rotation cannot run in plain fp16/bf16 on the
// matrix cores (a 2^-11 operand error moves y by ~2e-5).  R is split as
// R * 2^8 = R_hi + R_lo with both halves fp16; an fp16 input k is exact, so
// R k = (R_hi k + R_lo k) / 2^8 is two fp16 MFMAs with fp32 accumulation and
// an error near 2^-22 relative.  fp32 inputs are split too (k = k_hi + k_lo,
// three MFMAs).  The QJL projection of the fp32 residual uses the same
// trick: S_hi r_hi + S_lo r_hi + S_hi r_lo.  Only its sign is stored, so the
// power-of-two scalings never need undoing.
//
// Keys are rotated with output coordinates on the MFMA M axis and tokens on
// N: a lane then owns one token and 32 of its coordinates (16 t + 4 q + i),
// and packs them into the token's record without talking to other lanes.
// Values are rotated with tokens on M: a lane owns one coordinate of 32
// tokens of a 128-token block, which is the order the attention kernel
// contracts them in.
#include <type_traits>

#include "tq_device.h"

namespace tq {

struct KeyArgs {
  const void* x;
  uint32_t* rec;
  const uint16_t* r_hi;
  const uint16_t* r_lo;
  const uint16_t* s_hi;
  const uint16_t* s_lo;
  int64_t n_new, pos, capacity;
  int n_seq;
  int rec_words;
  _Float16 m1;  // -1 (a run-time value: see split2m)
  CodebookDev cb;
};

constexpr int kRImg = kD * kLdsStride;  // halves per R image

template <int M>
constexpr size_t key_lds_bytes() {
  return (size_t)(2 * kRImg + 2 * M * kLdsStride) * 2;
}

// Copy n_halves fp16 values (a multiple of 8) from global memory into LDS,
// 8 independent 16-byte loads in flight per thread.
__device__ __forceinline__ void copy_u4(uint16_t* dst, const uint16_t* src, int n_halves) {
  const int n = n_halves / 8;
  for (int i0 = threadIdx.x; i0 < n; i0 += 8 * blockDim.x) {
    u4 v[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int i = i0 + j * blockDim.x;
      if (i < n) v[j] = ((const u4*)src)[i];
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int i = i0 + j * blockDim.x;
      if (i < n) ((u4*)dst)[i] = v[j];
    }
  }
}

// Load the 32 input coordinates a lane owns (8 per K block: 32 kb + 8 q ..)
// of one fp32 token and return the norm of the token shifted by 2^-ex, 2^ex
// the binary exponent of its largest magnitude (the four lanes q of the token
// reduce together): full precision for any finite row, ||x|| = ldexp(., ex).
// The caller needs the norm before it can split the row into fp16 hi/lo
// operands (split_row32), so the row comes back raw.
__device__ __forceinline__ float load_row32_norm(const void* x, int64_t row, int q, f4 (&v)[8], int& ex) {
  const float* src = (const float*)x + row * kD + 8 * q;
  float mx = 0.f;
#pragma unroll
  for (int kb = 0; kb < 4; ++kb) {
    v[2 * kb] = *(const f4*)(src + 32 * kb);
    v[2 * kb + 1] = *(const f4*)(src + 32 * kb + 4);
#pragma unroll
    for (int e = 0; e < 4; ++e) mx = fmaxf(mx, fmaxf(fabsf(v[2 * kb][e]), fabsf(v[2 * kb + 1][e])));
  }
  mx = fmaxf(mx, shfl_xor(mx, 16));
  mx = fmaxf(mx, shfl_xor(mx, 32));
  ex = pow2_exponent(mx);
  float ss[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int kb = 0; kb < 4; ++kb)
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float u0 = ldexpf(v[2 * kb][e], -ex), u1 = ldexpf(v[2 * kb + 1][e], -ex);
      ss[kb] = fmaf(u1, u1, fmaf(u0, u0, ss[kb]));
    }
  float t = (ss[0] + ss[1]) + (ss[2] + ss[3]);
  t += shfl_xor(t, 16);
  t += shfl_xor(t, 32);
  return sqrtf(t);
}

// The row shifted by 2^sh (input_shift of its norm) as fp16 hi/lo operands.
__device__ __forceinline__ void split_row32(const f4 (&v)[8], int sh, h8 (&xh)[4], h8 (&xl)[4]) {
#pragma unroll
  for (int kb = 0; kb < 4; ++kb) {
    u4 hi, lo;
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      const f4& src = v[2 * kb + p / 2];
      const HiLo t = split2(ldexpf(src[2 * (p % 2)], sh), ldexpf(src[2 * (p % 2) + 1], sh));
      hi[p] = t.hi;
      lo[p] = t.lo;
    }
    xh[kb] = as_h8(hi);
    xl[kb] = as_h8(lo);
  }
}

template <int B, int M, bool F32>
__global__ __launch_bounds__(512, 1) void compress_keys_kernel(const KeyArgs a) {
  // 8 waves (2 per SIMD) share the LDS images; 2 (fp32: 1) 16-token tiles per
  // wave iteration keep a wave within 256 registers
  constexpr int H = 1 << (B - 1);
  constexpr int NT = (F32 || M > 64) ? 1 : 2;  // 16-token N tiles per wave iteration
  constexpr int PT = M / 16;       // projection M tiles
  constexpr int NCH = M / 64;      // 16-bit sign chunks per lane
  extern __shared__ __align__(16) uint16_t lds[];
  __shared__ float ctab[16];       // 2^12 c_i
  uint16_t* Rh = lds;
  uint16_t* Rl = Rh + kRImg;
  uint16_t* Sh = Rl + kRImg;
  uint16_t* Sl = Sh + M * kLdsStride;
  copy_u4(Rh, a.r_hi, kRImg);
  copy_u4(Rl, a.r_lo, kRImg);
  copy_u4(Sh, a.s_hi, M * kLdsStride);
  copy_u4(Sl, a.s_lo, M * kLdsStride);
  if (threadIdx.x < 16) ctab[threadIdx.x] = a.cb.cent[threadIdx.x] * kResScale;
  __syncthreads();

  float bpos[8];
  load_pos_beta<B>(bpos, a.cb);
  // wave-uniform (a scalar register): tile, slot and offset arithmetic stays on the scalar unit
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int r16 = lane & 15, q = lane >> 4;
  const int64_t tps = (a.n_new + 16 * NT - 1) / (16 * NT);
  const int64_t ntiles = tps * a.n_seq;
  const int waves = blockDim.x >> 6;

  for (int64_t tile = (int64_t)blockIdx.x * waves + wave; tile < ntiles; tile += (int64_t)gridDim.x * waves) {
    const int slot = (int)(tile / tps);
    const int64_t t0 = (tile - (int64_t)slot * tps) * (16 * NT);

    // Inputs.  Rows past n_new are clamped to the last row: their results
    // are never stored, they only need to be finite.  Per token: the norm,
    // the boundaries scaled to the accumulator (sigma = 2^8 2^sh ||k||, 2^sh
    // the fp32 pre-shift, 1 for fp16) and s16 = 2^12 / sigma.
    h8 xh[NT][4];
    h8 xl[F32 ? NT : 1][4];
    float nrm[NT], s16[NT], bs[NT][8];
#pragma unroll
    for (int j = 0; j < NT; ++j) {
      const int64_t tok = t0 + 16 * j + r16;
      const int64_t row = (int64_t)slot * a.n_new + (tok < a.n_new ? tok : a.n_new - 1);
      float n, sigma;
      if constexpr (F32) {
        f4 v[8];
        int ex = 0;
        const float ns = load_row32_norm(a.x, row, q, v, ex);  // ||k 2^-ex||
        const int s0 = input_shift(ns);                        // |k 2^(s0 - ex)| < 2^13
        split_row32(v, s0 - ex, xh[j], xl[j]);
        sigma = kRotScale * ldexpf(ns, s0);
        n = ldexpf(ns, ex);
      } else {
        const _Float16* src = (const _Float16*)a.x + row * kD + 8 * q;
#pragma unroll
        for (int kb = 0; kb < 4; ++kb) xh[j][kb] = *(const h8*)(src + 32 * kb);
        float ss = sq_norm16(xh[j]);
        ss += shfl_xor(ss, 16);
        ss += shfl_xor(ss, 32);
        n = sqrtf(ss);
        sigma = kRotScale * n;
      }
      nrm[j] = n;
      s16[j] = n > 0.f ? kResScale / sigma : 0.f;
#pragma unroll
      for (int t = 0; t < 8; ++t) bs[j][t] = t < H - 1 ? bpos[t] * sigma : 0.f;
    }

    f4 zacc[NT][PT];
    uint32_t cw[NT][B];
    float g2[NT];
#pragma unroll
    for (int j = 0; j < NT; ++j) {
      g2[j] = 0.f;
#pragma unroll
      for (int w = 0; w < B; ++w) cw[j][w] = 0u;
#pragma unroll
      for (int p = 0; p < PT; ++p) zacc[j][p] = f4{0.f, 0.f, 0.f, 0.f};
    }

#pragma unroll
    for (int kb2 = 0; kb2 < 4; ++kb2) {  // output tiles 2 kb2, 2 kb2 + 1 = projection K block kb2
      // one pass per pair of output tiles; the barrier below keeps the
      // scheduler from hoisting later passes' LDS loads (register pressure)
      __builtin_amdgcn_sched_barrier(0);
      f4 yacc[NT][2];
#pragma unroll
      for (int j = 0; j < NT; ++j) yacc[j][0] = yacc[j][1] = f4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) {
        h8 ah[2], al[2];
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          const int off = (16 * (2 * kb2 + u) + r16) * kLdsStride + 32 * kb + 8 * q;
          ah[u] = *(const h8*)(Rh + off);
          al[u] = *(const h8*)(Rl + off);
        }
#pragma unroll
        for (int j = 0; j < NT; ++j)
#pragma unroll
          for (int u = 0; u < 2; ++u) {
            yacc[j][u] = mfma(ah[u], xh[j][kb], yacc[j][u]);
            yacc[j][u] = mfma(al[u], xh[j][kb], yacc[j][u]);
            if constexpr (F32) yacc[j][u] = mfma(ah[u], xl[j][kb], yacc[j][u]);
          }
      }
      h8 sh[PT], sl[PT];
#pragma unroll
      for (int p = 0; p < PT; ++p) {
        const int off = (16 * p + r16) * kLdsStride + 32 * kb2 + 8 * q;
        sh[p] = *(const h8*)(Sh + off);
        sl[p] = *(const h8*)(Sl + off);
      }
#pragma unroll
      for (int j = 0; j < NT; ++j) {
        // cells, scaled residual 2^12 (y - c[idx]), codes, residual operands
        u4 rhi, rlo;
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          float rs[4];
          const uint32_t x4 = quantize4<B>(yacc[j][u], bs[j], s16[j], ctab, rs, g2[j]);
          const HiLo t01 = split2m(rs[0], rs[1], a.m1), t23 = split2m(rs[2], rs[3], a.m1);
          rhi[2 * u] = t01.hi;
          rlo[2 * u] = t01.lo;
          rhi[2 * u + 1] = t23.hi;
          rlo[2 * u + 1] = t23.lo;
          put_sel4_rt<B>(cw[j], 2 * kb2 + u, x4);
        }
        const h8 rh = as_h8(rhi), rl = as_h8(rlo);
#pragma unroll
        for (int p = 0; p < PT; ++p) {
          zacc[j][p] = mfma(sh[p], rh, zacc[j][p]);
          zacc[j][p] = mfma(sl[p], rh, zacc[j][p]);
          zacc[j][p] = mfma(sh[p], rl, zacc[j][p]);
        }
      }
    }

#pragma unroll
    for (int j = 0; j < NT; ++j) {
      float g = g2[j];
      g += shfl_xor(g, 16);
      g += shfl_xor(g, 32);
      const float gamma = sqrtf(g) * (1.f / kResScale);
      uint32_t bits[NCH];
#pragma unroll
      for (int c = 0; c < NCH; ++c)
        bits[c] = sign_bits16(zacc[j][4 * c], zacc[j][4 * c + 1], zacc[j][4 * c + 2], zacc[j][4 * c + 3]);
      const int64_t tok = t0 + 16 * j + r16;
      if (tok < a.n_new) {
        uint32_t* rp = a.rec + ((int64_t)slot * a.capacity + a.pos + tok) * a.rec_words;
#pragma unroll
        for (int w = 0; w < B; ++w) rp[q * B + w] = cw[j][w];
#pragma unroll
        for (int c = 0; c < NCH; ++c) ((uint16_t*)(rp + 4 * B + 2 * c + (q >> 1)))[q & 1] = (uint16_t)bits[c];
        if (q == 0) rp[a.rec_words - 2] = __float_as_uint(nrm[j]);
        if (q == 1) rp[a.rec_words - 1] = __float_as_uint(gamma);
      }
    }
  }
}

// Keys on 32 x 32 x 16 matrix-core tiles (fp16 keys, m = 64).  A wave takes
// 32 tokens per iteration.  Lane l owns token l % 32 and, of every 32-
// coordinate output tile t, the 16 coordinates 32 t + 8 j + 4 g + i
// (g = l / 32, acc[4 j + i]); over the four tiles those are exactly the
// record's code groups g and g + 2, so the record is written lane-locally in
// the same layout as above.  The residual of tile t feeds projection K steps
// 2t and 2t + 1 straight from the accumulator (S's columns are permuted to
// match, bits 2 and 3 of the coordinate swapped).  Rotation t + 1 is issued
// before the bucketing of tile t so the two can overlap on a SIMD.  With
// B = 0 (one cell at 0: signs and norms only) the residual is the rotated
// coordinate itself and no code words are written.
template <int B>
__global__ __launch_bounds__(512, 1) void compress_keys32_kernel(const KeyArgs a) {
  constexpr int H = B > 0 ? 1 << (B - 1) : 1;
  constexpr int BW = B > 0 ? B : 1;  // code words per group (none at 0 bits)
  extern __shared__ __align__(16) uint16_t lds[];
  __shared__ float ctab[16];  // 2^12 c_i
  uint16_t* Rh = lds;
  uint16_t* Rl = Rh + kRImg;
  uint16_t* Sh = Rl + kRImg;
  uint16_t* Sl = Sh + 64 * kLdsStride;
  copy_u4(Rh, a.r_hi, kRImg);
  copy_u4(Rl, a.r_lo, kRImg);
  copy_u4(Sh, a.s_hi, 64 * kLdsStride);
  copy_u4(Sl, a.s_lo, 64 * kLdsStride);
  if (threadIdx.x < 16) ctab[threadIdx.x] = a.cb.cent[threadIdx.x] * kResScale;
  __syncthreads();

  float bpos[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  if constexpr (B > 0) load_pos_beta<B>(bpos, a.cb);
  // wave-uniform (a scalar register): tile, slot and offset arithmetic stays on the scalar unit
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int n32 = lane & 31, g = lane >> 5;
  const int64_t tps = (a.n_new + 31) / 32;
  const int64_t ntiles = tps * a.n_seq;
  const int waves = blockDim.x >> 6;
  const int arow = n32 * kLdsStride + 8 * g;  // this lane's A-operand offset in a 32-row band

  for (int64_t tile = (int64_t)blockIdx.x * waves + wave; tile < ntiles; tile += (int64_t)gridDim.x * waves) {
    const int slot = (int)(tile / tps);
    const int64_t t0 = (tile - (int64_t)slot * tps) * 32;
    const int64_t tok = t0 + n32;
    // rows past n_new are clamped to the last row (computed, never stored)
    const int64_t row = (int64_t)slot * a.n_new + (tok < a.n_new ? tok : a.n_new - 1);
    const _Float16* src = (const _Float16*)a.x + row * kD + 8 * g;
    h8 xk[8];  // B operands: coordinates 16 kk + 8 g .. + 7
#pragma unroll
    for (int kk = 0; kk < 8; ++kk) xk[kk] = *(const h8*)(src + 16 * kk);
    float ss[2] = {0.f, 0.f};
#pragma unroll
    for (int kk = 0; kk < 8; ++kk)
#pragma unroll
      for (int e = 0; e < 8; e += 2) {
        const h2 v = {xk[kk][e], xk[kk][e + 1]};
        ss[kk & 1] = __builtin_amdgcn_fdot2(v, v, ss[kk & 1], false);
      }
    float sq = ss[0] + ss[1];
    sq += shfl_xor(sq, 32);
    const float nrm = sqrtf(sq);
    const float sigma = kRotScale * nrm;
    const float s16 = nrm > 0.f ? kResScale / sigma : 0.f;
    float bs[8];
#pragma unroll
    for (int t = 0; t < 8; ++t) bs[t] = t < H - 1 ? bpos[t] * sigma : 0.f;

    auto rotate = [&](int t) {
      f16v y;
#pragma unroll
      for (int e = 0; e < 16; ++e) y[e] = 0.f;
      const int o = 32 * t * kLdsStride + arow;
#pragma unroll
      for (int kk = 0; kk < 8; ++kk) {
        const h8 ah = *(const h8*)(Rh + o + 16 * kk);
        const h8 al = *(const h8*)(Rl + o + 16 * kk);
        y = mfma32(ah, xk[kk], y);
        y = mfma32(al, xk[kk], y);
      }
      return y;
    };

    f16v zacc[2];
#pragma unroll
    for (int p = 0; p < 2; ++p)
#pragma unroll
      for (int e = 0; e < 16; ++e) zacc[p][e] = 0.f;
    uint32_t cw[2][BW];
#pragma unroll
    for (int w = 0; w < BW; ++w) cw[0][w] = cw[1][w] = 0u;
    float g2 = 0.f;

    f16v ycur = rotate(0);
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      __builtin_amdgcn_sched_barrier(0x0008);  // (matrix-core instructions may cross)
      f16v ynext;
      if (t < 3) ynext = rotate(t + 1);
      // Raised wave priority while this wave buckets and projects tile t:
      // the other wave of the SIMD then issues its rotation MFMAs in the
      // gaps rather than competing for VALU issue (measured ~2% faster).
      __builtin_amdgcn_s_setprio(1);
      // cells, scaled residual 2^12 (y - c[idx]) as the B operands of
      // projection K steps 2t (acc 0..7) and 2t + 1 (acc 8..15)
      u4 rhi[2], rlo[2];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        float rs[4];  // -residual
        uint32_t x4 = 0u;
        if constexpr (B > 0) {
          x4 = quantize4_signs<B>(quarter(ycur, j), bs, -s16, ctab, rs, g2);
        } else {
          const f4 y4 = quarter(ycur, j);
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            rs[i] = -s16 * y4[i];
            g2 = fmaf(rs[i], rs[i], g2);
          }
        }
        const HiLo t01 = split2m(rs[0], rs[1], a.m1), t23 = split2m(rs[2], rs[3], a.m1);
        rhi[j >> 1][2 * (j & 1)] = t01.hi;
        rlo[j >> 1][2 * (j & 1)] = t01.lo;
        rhi[j >> 1][2 * (j & 1) + 1] = t23.hi;
        rlo[j >> 1][2 * (j & 1) + 1] = t23.lo;
        if constexpr (B > 0) put_sel4_rt<B>(cw[j & 1], 2 * t + (j >> 1), x4);
      }
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const h8 rh = as_h8(rhi[h]), rl = as_h8(rlo[h]);
#pragma unroll
        for (int p = 0; p < 2; ++p) {
          const int o = 32 * p * kLdsStride + arow + 16 * (2 * t + h);
          const h8 sh = *(const h8*)(Sh + o);
          const h8 sl = *(const h8*)(Sl + o);
          zacc[p] = mfma32(sh, rh, zacc[p]);
          zacc[p] = mfma32(sl, rh, zacc[p]);
          zacc[p] = mfma32(sh, rl, zacc[p]);
        }
      }
      __builtin_amdgcn_s_setprio(0);
      if (t < 3) ycur = ynext;
    }

    g2 += shfl_xor(g2, 32);
    const float gamma = sqrtf(g2) * (1.f / kResScale);
    // projection 32 p + 8 j + 4 g + i = 16 (2 p + j/2) + 4 (2 (j%2) + g) + i:
    // sign group g (j even) and g + 2 (j odd), bit 4 (2 p + j/2) + i
    // (zacc holds S applied to the negated residual)
    uint32_t bits_a = sign_bits16_neg(quarter(zacc[0], 0), quarter(zacc[0], 2), quarter(zacc[1], 0),
                                      quarter(zacc[1], 2));
    uint32_t bits_b = sign_bits16_neg(quarter(zacc[0], 1), quarter(zacc[0], 3), quarter(zacc[1], 1),
                                      quarter(zacc[1], 3));
    if (nrm == 0.f) {
      if constexpr (B > 0) {
        // A zero key has every rotated coordinate +0, which quantize4_signs
        // puts in cell H with residual -c+_0.  Its cell is H - 1 (0 is the
        // middle boundary and ties go to the lower cell), whose residual is
        // +c+_0: the opposite residual, so every projection flips sign.
        fill_code_words<B>(cw[0], (uint32_t)H - 1u);
        fill_code_words<B>(cw[1], (uint32_t)H - 1u);
        bits_a = ~bits_a & 0xFFFFu;
        bits_b = ~bits_b & 0xFFFFu;
      } else {
        // residual 0: every projection is 0, whose bit is 1
        bits_a = bits_b = 0xFFFFu;
      }
    }
    if (tok < a.n_new) {
      uint32_t* rp = a.rec + ((int64_t)slot * a.capacity + a.pos + tok) * a.rec_words;
#pragma unroll
      for (int w = 0; w < B; ++w) {
        rp[g * B + w] = cw[0][w];
        rp[(g + 2) * B + w] = cw[1][w];
      }
      ((uint16_t*)(rp + 4 * B))[g] = (uint16_t)bits_a;
      ((uint16_t*)(rp + 4 * B + 1))[g] = (uint16_t)bits_b;
      rp[a.rec_words - 2 + g] = __float_as_uint(g == 0 ? nrm : gamma);
    }
  }
}

// ---------------------------------------------------------------------------
// values
// ---------------------------------------------------------------------------

struct ValArgs {
  const void* x;
  uint32_t* blocks;
  const uint16_t* r_hi;
  const uint16_t* r_lo;
  int64_t n_new, pos, capacity;
  int64_t blk0, nblk;  // first touched block of a slot, blocks touched per slot
  int n_seq;
  int block_words;
  CodebookDev cb;
};

constexpr size_t kValLds = (size_t)2 * kRImg * 2;

template <int B, bool F32>
__global__ __launch_bounds__(256, F32 ? 1 : 2) void compress_values_kernel(const ValArgs a) {
  extern __shared__ __align__(16) uint16_t lds[];
  uint16_t* Rh = lds;
  uint16_t* Rl = Rh + kRImg;
  copy_u4(Rh, a.r_hi, kRImg);
  copy_u4(Rl, a.r_lo, kRImg);
  __syncthreads();

  float bp[8];
  load_pos_beta<B>(bp, a.cb);
  // wave-uniform (a scalar register): tile, slot and offset arithmetic stays on the scalar unit
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int r16 = lane & 15, q = lane >> 4;
  const int waves = blockDim.x >> 6;
  const int64_t nitems = a.nblk * a.n_seq;
  const int64_t nblk_cap = a.capacity / kBlockTokens;

  for (int64_t item = (int64_t)blockIdx.x * waves + wave; item < nitems; item += (int64_t)gridDim.x * waves) {
    const int slot = (int)(item / a.nblk);
    const int64_t blk = a.blk0 + (item - (int64_t)slot * a.nblk);
    const int64_t tok0 = blk * kBlockTokens;
    uint32_t* vb = a.blocks + ((int64_t)slot * nblk_cap + blk) * a.block_words;
    float* vnorm = (float*)(vb + 4 * B * kD);

    uint32_t cw[8][B];
#pragma unroll
    for (int nt = 0; nt < 8; ++nt)
#pragma unroll
      for (int w = 0; w < B; ++w) cw[nt][w] = 0u;

    // One half block (64 tokens, slots 4 half .. 4 half + 3).  The half is a
    // compile-time constant so that the code slots are too: with a run-time
    // slot the packing goes through a branchy switch and register copies.
    auto run_half = [&](auto half_tag) {
      constexpr int half = decltype(half_tag)::value;
      // a half with no token of [pos, pos + n_new) keeps all its codes (a
      // short append, e.g. one decode token, touches one half)
      const int64_t h0 = tok0 + 64 * half;
      if (h0 + 64 <= a.pos || h0 >= a.pos + a.n_new) return;
      h8 xa[4][4];
      h8 xl[F32 ? 4 : 1][4];
      float tok_sc[4];  // per token: sigma = 2^8 2^sh ||v|| (4-bit codes: 1 / sigma)
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) {
        // block token tau -> input row; rows outside [pos, pos + n_new) are
        // clamped to a valid row (finite data whose codes are masked out)
        const int tau = 16 * (4 * half + mt) + r16;
        int64_t row = tok0 + tau - a.pos;
        const bool valid = row >= 0 && row < a.n_new;
        row = (int64_t)slot * a.n_new + (row < 0 ? 0 : (row >= a.n_new ? a.n_new - 1 : row));
        if constexpr (F32) {
          f4 v[8];
          int ex = 0;
          const float n0 = load_row32_norm(a.x, row, q, v, ex);  // ||v 2^-ex||
          const int s0 = input_shift(n0);
          split_row32(v, s0 - ex, xa[mt], xl[mt]);
          const float ns = ldexpf(n0, s0);  // the shifted row's norm, in [2^12, 2^13)
          const float n = ldexpf(n0, ex);
          tok_sc[mt] = B <= 3 ? kRotScale * ns : (n0 > 0.f ? 1.f / (kRotScale * ns) : 0.f);
          if (q == 0 && valid) vnorm[tau] = n;
        } else {
          const _Float16* src = (const _Float16*)a.x + row * kD + 8 * q;
#pragma unroll
          for (int kb = 0; kb < 4; ++kb) xa[mt][kb] = *(const h8*)(src + 32 * kb);
          float ss = sq_norm16(xa[mt]);
          ss += shfl_xor(ss, 16);
          ss += shfl_xor(ss, 32);
          const float n = sqrtf(ss);
          tok_sc[mt] = B <= 3 ? kRotScale * n : (n > 0.f ? 1.f / (kRotScale * n) : 0.f);
          if (q == 0 && valid) vnorm[tau] = n;
        }
      }
      // Per token in the output layout (lane (coordinate, q) holds tokens
      // 4q+i): the boundaries scaled to the accumulator, bs = beta sigma with
      // sigma = 2^8 2^sh ||v||; for 4-bit codes (7 boundaries a token) the
      // coordinates are normalised instead, y = a / sigma, against the
      // unscaled boundaries
      constexpr bool kScaled = B <= 3;
      float inv_d[4][4];
      float bsd[4][4][kScaled ? 8 : 1];
      uint32_t zmask[4];  // per row tile: bytes 0xFF for tokens of zero norm
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) {
        zmask[mt] = 0u;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float v = __shfl(tok_sc[mt], 4 * q + i, 64);
          zmask[mt] |= v == 0.f ? 0xFFu << (8 * i) : 0u;
          if constexpr (kScaled) {
#pragma unroll
            for (int t = 0; t < 8; ++t) bsd[mt][i][t] = t < (1 << (B - 1)) - 1 ? bp[t] * v : 0.f;
          } else {
            inv_d[mt][i] = v;
          }
        }
      }

#pragma unroll
      for (int ntp = 0; ntp < 4; ++ntp) {
        f4 acc[4][2];
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) acc[mt][0] = acc[mt][1] = f4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kb = 0; kb < 4; ++kb) {
          h8 bh[2], bl[2];
#pragma unroll
          for (int u = 0; u < 2; ++u) {
            const int off = (16 * (2 * ntp + u) + r16) * kLdsStride + 32 * kb + 8 * q;
            bh[u] = *(const h8*)(Rh + off);
            bl[u] = *(const h8*)(Rl + off);
          }
#pragma unroll
          for (int mt = 0; mt < 4; ++mt)
#pragma unroll
            for (int u = 0; u < 2; ++u) {
              acc[mt][u] = mfma(xa[mt][kb], bh[u], acc[mt][u]);
              acc[mt][u] = mfma(xa[mt][kb], bl[u], acc[mt][u]);
              if constexpr (F32) acc[mt][u] = mfma(xl[mt][kb], bh[u], acc[mt][u]);
            }
        }
        // raised wave priority while bucketing (the other wave's MFMAs fill
        // the gaps; measured ~2% faster)
        __builtin_amdgcn_s_setprio(1);
#pragma unroll
        for (int mt = 0; mt < 4; ++mt)
#pragma unroll
          for (int u = 0; u < 2; ++u) {
            f4 v = acc[mt][u];
            float bsx[4][8];
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
              for (int t = 0; t < 8; ++t) {
                if constexpr (kScaled) {
                  bsx[i][t] = bsd[mt][i][t];
                } else {
                  bsx[i][t] = bp[t];
                  if (t == 0) v[i] *= inv_d[mt][i];
                }
              }
            const uint32_t x4 = cells4_signs<B>(v, bsx, zmask[mt]);
            put_sel4_rt<B>(cw[2 * ntp + u], 4 * half + mt, x4);  // slot of these 16 tokens
          }
        __builtin_amdgcn_s_setprio(0);
        // keep the scheduler from hoisting the next coordinate tiles' R loads
        __builtin_amdgcn_sched_barrier(0);
      }
    };
    run_half(std::integral_constant<int, 0>{});
    run_half(std::integral_constant<int, 1>{});

    const bool full = tok0 >= a.pos && tok0 + kBlockTokens <= a.pos + a.n_new;
    if (full) {
#pragma unroll
      for (int nt = 0; nt < 8; ++nt)
#pragma unroll
        for (int w = 0; w < B; ++w) vb[(w * 4 + q) * kD + 16 * nt + r16] = cw[nt][w];
    } else {
      // keep the codes of tokens outside [pos, pos + n_new)
      uint32_t keep[B];
#pragma unroll
      for (int w = 0; w < B; ++w) keep[w] = 0u;
      for (int s = 0; s < 8; ++s)
        for (int i = 0; i < 4; ++i) {
          const int64_t p = tok0 + 16 * s + 4 * q + i;
          if (p < a.pos || p >= a.pos + a.n_new)
#pragma unroll
            for (int w = 0; w < B; ++w) keep[w] |= field_mask_rt(B, s, w, i);
        }
#pragma unroll
      for (int nt = 0; nt < 8; ++nt)
#pragma unroll
        for (int w = 0; w < B; ++w) {
          uint32_t* dst = vb + (w * 4 + q) * kD + 16 * nt + r16;
          *dst = (*dst & keep[w]) | (cw[nt][w] & ~keep[w]);
        }
    }
  }
}

// ---------------------------------------------------------------------------
// launchers
// ---------------------------------------------------------------------------

static int g_num_cus = 0;

template <int B, int M, bool F32>
static int set_key_attr() {
  return hipFuncSetAttribute((const void*)compress_keys_kernel<B, M, F32>,
                             hipFuncAttributeMaxDynamicSharedMemorySize, (int)key_lds_bytes<M>()) == hipSuccess
             ? 0 : -1;
}

template <int B>
static int set_key32_attr() {
  return hipFuncSetAttribute((const void*)compress_keys32_kernel<B>, hipFuncAttributeMaxDynamicSharedMemorySize,
                             (int)key_lds_bytes<64>()) == hipSuccess
             ? 0 : -1;
}

template <int B, bool F32>
static int set_val_attr() {
  return hipFuncSetAttribute((const void*)compress_values_kernel<B, F32>,
                             hipFuncAttributeMaxDynamicSharedMemorySize, (int)kValLds) == hipSuccess
             ? 0 : -1;
}

int compress_device_init() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return -1;
  if (hipDeviceGetAttribute(&g_num_cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return -1;
  int rc = 0;
#define TQ_KEY_ATTR(B)                                                                   \
  rc |= set_key_attr<B, 64, false>() | set_key_attr<B, 64, true>() |                     \
        set_key_attr<B, 128, false>() | set_key_attr<B, 128, true>();
  TQ_KEY_ATTR(1) TQ_KEY_ATTR(2) TQ_KEY_ATTR(3) TQ_KEY_ATTR(4)
#undef TQ_KEY_ATTR
  rc |= set_key32_attr<0>() | set_key32_attr<1>() | set_key32_attr<2>() | set_key32_attr<3>() |
        set_key32_attr<4>();
  rc |= set_val_attr<1, false>() | set_val_attr<1, true>() | set_val_attr<2, false>() | set_val_attr<2, true>();
  rc |= set_val_attr<3, false>() | set_val_attr<3, true>() | set_val_attr<4, false>() | set_val_attr<4, true>();
  return rc;
}

template <int B, int M, bool F32>
static void key_launch(const KeyArgs& a, int64_t ntiles, hipStream_t st) {
  const int waves = 8;
  int64_t grid = (ntiles + waves - 1) / waves;
  const int64_t cap = (int64_t)(g_num_cus > 0 ? g_num_cus : 256);
  if (grid > cap) grid = cap;
  hipLaunchKernelGGL((compress_keys_kernel<B, M, F32>), dim3((unsigned)grid), dim3(64 * waves),
                     key_lds_bytes<M>(), st, a);
}

template <int B>
static void key32_launch(const KeyArgs& a, int64_t ntiles, hipStream_t st) {
  const int waves = 8;
  int64_t grid = (ntiles + waves - 1) / waves;
  const int64_t cap = (int64_t)(g_num_cus > 0 ? g_num_cus : 256);
  if (grid > cap) grid = cap;
  hipLaunchKernelGGL((compress_keys32_kernel<B>), dim3((unsigned)grid), dim3(64 * waves), key_lds_bytes<64>(), st,
                     a);
}

int launch_compress_keys(const Matrices& mats, const CodebookDev& cb, int bits, int m, const AppendShape& s,
                         void* key_records, void* stream) {
  KeyArgs a;
  a.x = s.x;
  a.rec = (uint32_t*)key_records;
  a.r_hi = mats.r_hi;
  a.r_lo = mats.r_lo;
  a.s_hi = mats.s_hi;
  a.s_lo = mats.s_lo;
  a.n_new = s.n_new;
  a.pos = s.pos;
  a.capacity = s.capacity;
  a.n_seq = s.n_seq;
  a.rec_words = bits * kD / 32 + m / 32 + 2;
  a.m1 = (_Float16)-1.0f;
  a.cb = cb;
  const bool f32 = s.dtype == TQ_F32;
  const int64_t per = (f32 || m > 64) ? 16 : 32;
  const int64_t ntiles = ((s.n_new + per - 1) / per) * s.n_seq;
  hipStream_t st = (hipStream_t)stream;
  if (!f32 && m == 64 && bits >= 0 && bits <= 4) {  // fp16 keys, m = 64: the 32 x 32 tile kernel
    a.s_hi = mats.s_hi32;
    a.s_lo = mats.s_lo32;
    switch (bits) {
      case 0: key32_launch<0>(a, ntiles, st); break;
      case 1: key32_launch<1>(a, ntiles, st); break;
      case 2: key32_launch<2>(a, ntiles, st); break;
      case 3: key32_launch<3>(a, ntiles, st); break;
      default: key32_launch<4>(a, ntiles, st); break;
    }
    return hipGetLastError() == hipSuccess ? 0 : TQ_EDEVICE;
  }
#define TQ_KEY_CASE(B, M)                                  \
  if (bits == B && m == M) {                               \
    if (f32) key_launch<B, M, true>(a, ntiles, st);        \
    else key_launch<B, M, false>(a, ntiles, st);           \
    return hipGetLastError() == hipSuccess ? 0 : TQ_EDEVICE; \
  }
  TQ_KEY_CASE(1, 64) TQ_KEY_CASE(2, 64) TQ_KEY_CASE(3, 64) TQ_KEY_CASE(4, 64)
  TQ_KEY_CASE(1, 128) TQ_KEY_CASE(2, 128) TQ_KEY_CASE(3, 128) TQ_KEY_CASE(4, 128)
#undef TQ_KEY_CASE
  return TQ_EUNSUPPORTED;
}

template <int B, bool F32>
static void val_launch(const ValArgs& a, int64_t nitems, hipStream_t st) {
  const int waves = 4;
  int64_t grid = (nitems + waves - 1) / waves;
  const int64_t cap = (int64_t)(g_num_cus > 0 ? g_num_cus : 256) * (F32 ? 1 : 2);
  if (grid > cap) grid = cap;
  hipLaunchKernelGGL((compress_values_kernel<B, F32>), dim3((unsigned)grid), dim3(64 * waves), kValLds, st, a);
}

int launch_compress_values(const Matrices& mats, const CodebookDev& cb, int bits, const AppendShape& s,
                           void* value_blocks, void* stream) {
  ValArgs a;
  a.x = s.x;
  a.blocks = (uint32_t*)value_blocks;
  a.r_hi = mats.r_hi;
  a.r_lo = mats.r_lo;
  a.n_new = s.n_new;
  a.pos = s.pos;
  a.capacity = s.capacity;
  a.blk0 = s.pos / kBlockTokens;
  a.nblk = (s.pos + s.n_new - 1) / kBlockTokens - a.blk0 + 1;
  a.n_seq = s.n_seq;
  a.block_words = 4 * bits * kD + kBlockTokens;
  a.cb = cb;
  const bool f32 = s.dtype == TQ_F32;
  const int64_t nitems = a.nblk * s.n_seq;
  hipStream_t st = (hipStream_t)stream;
#define TQ_VAL_CASE(B)                                     \
  if (bits == B) {                                         \
    if (f32) val_launch<B, true>(a, nitems, st);           \
    else val_launch<B, false>(a, nitems, st);              \
    return hipGetLastError() == hipSuccess ? 0 : TQ_EDEVICE; \
  }
  TQ_VAL_CASE(1) TQ_VAL_CASE(2) TQ_VAL_CASE(3) TQ_VAL_CASE(4)
#undef TQ_VAL_CASE
  return TQ_EUNSUPPORTED;
}

}  // namespace tq
