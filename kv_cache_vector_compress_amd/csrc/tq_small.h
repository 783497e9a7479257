// Device code of the small appends (a few tokens per slot), shared by the
// append kernels of tq_small.hip and the fused decode step of
// tq_attention.hip.
// Appends of a few tokens per slot (a decode step appends one), for any
// shape of the layout.  The bulk kernels stage R (and S) images in LDS and
// fill whole 16- to 64-token matrix-core tiles; for a handful of tokens that
// set-up is most of their time.  Here the arithmetic runs in fp32 on the
// vector units with R and S read from L2 (they are shared by every
// workgroup): stage 1 (nav.superapi.store "turboquant-pytorch", 主要能力;
// atskills.one Stage 1): n = ||x||, y = R x / n, idx = #{i : beta_i < y};
// keys also take stage 2 (atskills.one Stage 2): r = y - c[idx],
// gamma = ||r||, s = [S r >= 0].  fp32 dot products of d terms are within
// about 1e-7 of the exact values, inside the tolerance of the codes.
//
//   small_keys_kernel:   one workgroup per (slot, new token); writes the
//                        token's record.
//   small_values_kernel: one workgroup per (slot, touched 128-token block);
//                        the block's new tokens are coded one after the
//                        other and each code word is read, merged and
//                        written by one thread (words are shared by tokens).
#pragma once

#include <algorithm>

#include "tq_device.h"
#include "tq_prep.h"

namespace tq {

constexpr int kSmallThreads = 256;

struct SmallArgs {
  const void* x;        // [n_seq][n_new][d]
  int dtype;
  uint32_t* out;        // key records or value blocks
  const float* r32;     // R [d][d]
  const float* s32;     // S [m][d]
  int64_t n_new, pos, capacity;
  int64_t bid0;         // first (slot, token) index of this launch
  int n_seq, d, m, bits, rec_words, block_words;
  float beta[16];       // boundaries (+inf past the last)
  float cent[16];
};

__device__ __forceinline__ float block_sum(float v, float* red) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += shfl_xor(v, o);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  __syncthreads();
  if (lane == 0) red[wave] = v;
  __syncthreads();
  float s = 0.f;
  for (int w = 0; w < (int)(blockDim.x >> 6); ++w) s += red[w];
  return s;
}

// out[j] = sum_k mat[j][k] x[k] for j < n_rows (mat row-major, n_cols
// columns, x in LDS): two threads per row, halves of the columns.
__device__ __forceinline__ void matvec(const float* mat, int n_rows, int n_cols, const float* x, float* out) {
  const int half = threadIdx.x & 1, h = n_cols / 2;
  for (int j0 = 0; j0 < n_rows; j0 += blockDim.x / 2) {
    const int j = j0 + (threadIdx.x >> 1);
    float t0 = 0.f, t1 = 0.f;
    if (j < n_rows) {
      const f4* row = (const f4*)(mat + (size_t)j * n_cols + half * h);
      const float* xx = x + half * h;
      for (int k4 = 0; k4 < h / 4; k4 += 2) {
        const f4 u = row[k4], v = row[k4 + 1];
        t0 = fmaf(u[0], xx[4 * k4], fmaf(u[1], xx[4 * k4 + 1], fmaf(u[2], xx[4 * k4 + 2], fmaf(u[3], xx[4 * k4 + 3], t0))));
        t1 = fmaf(v[0], xx[4 * k4 + 4], fmaf(v[1], xx[4 * k4 + 5], fmaf(v[2], xx[4 * k4 + 6], fmaf(v[3], xx[4 * k4 + 7], t1))));
      }
    }
    float t = t0 + t1;
    t += shfl_xor(t, 1);
    if (j < n_rows && half == 0) out[j] = t;
  }
}

// head_dim 128: a thread's half row (64 floats) of one matrix, loaded before
// the input arrives so that the matrix and the input travel together.
struct HalfRows {
  f4 v[16];
};
__device__ __forceinline__ void prefetch_rows(const float* mat, int n_rows, HalfRows& h) {
  const int j = threadIdx.x >> 1, half = threadIdx.x & 1;
  if (j < n_rows) {
    const f4* row = (const f4*)(mat + (size_t)j * 128 + 64 * half);
#pragma unroll
    for (int u = 0; u < 16; ++u) h.v[u] = row[u];
  }
}
__device__ __forceinline__ void matvec_pref(const HalfRows& h, int n_rows, const float* x, float* out) {
  const int j = threadIdx.x >> 1, half = threadIdx.x & 1;
  const float* xx = x + 64 * half;
  float t0 = 0.f, t1 = 0.f;
#pragma unroll
  for (int u = 0; u < 16; u += 2) {
    t0 = fmaf(h.v[u][0], xx[4 * u], fmaf(h.v[u][1], xx[4 * u + 1], fmaf(h.v[u][2], xx[4 * u + 2], fmaf(h.v[u][3], xx[4 * u + 3], t0))));
    t1 = fmaf(h.v[u + 1][0], xx[4 * u + 4], fmaf(h.v[u + 1][1], xx[4 * u + 5],
             fmaf(h.v[u + 1][2], xx[4 * u + 6], fmaf(h.v[u + 1][3], xx[4 * u + 7], t1))));
  }
  float t = t0 + t1;
  t += shfl_xor(t, 1);
  if (j < n_rows && half == 0) out[j] = t;
}

// Load row `row` of the input into LDS as fp32, shifted by 2^-e with 2^e the
// binary exponent of its largest magnitude (exact), so that sums of squares
// and products with R and S neither overflow nor underflow for any finite
// row.  Returns the norm of the stored (shifted) row; the row's own norm is
// ldexp of it by e (*ex).  One block reduction of (exponent, sum) partials.
// d <= 1024: a thread holds at most 4 coordinates.
__device__ __forceinline__ float load_input(const SmallArgs& a, int64_t row, float* xs, float* red, int* ex) {
  float v[4], mx = 0.f;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int k = threadIdx.x + i * (int)blockDim.x;
    v[i] = 0.f;
    if (k < a.d) {
      const int64_t o = row * a.d + k;
      v[i] = a.dtype == TQ_F32 ? ((const float*)a.x)[o] : (float)((const _Float16*)a.x)[o];
    }
    mx = fmaxf(mx, fabsf(v[i]));
  }
  int e;
  norm2_partial(mx, e);
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float u = ldexpf(v[i], -e);
    s = fmaf(u, u, s);
  }
  wave_norm2(e, s);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  __syncthreads();  // (red may still be read by an earlier reduction)
  if (lane == 0) {
    red[2 * wave] = s;
    red[2 * wave + 1] = __int_as_float(e);
  }
  __syncthreads();
  float S = red[0];
  int E = __float_as_int(red[1]);
  for (int w = 1; w < (int)(blockDim.x >> 6); ++w) merge_norm2(E, S, __float_as_int(red[2 * w + 1]), red[2 * w]);
  if (E == kNoExp) E = 0;  // a zero row
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int k = threadIdx.x + i * (int)blockDim.x;
    if (k < a.d) xs[k] = ldexpf(v[i], -E);
  }
  *ex = E;
  return sqrtf(S);
}

// #{i : beta_i < u}; beta holds +inf past the last boundary, so all 15
// compares run with constant indices (the boundaries stay in registers).
__device__ __forceinline__ int cell(float u, const float (&beta)[15]) {
  int idx = 0;
#pragma unroll
  for (int i = 0; i < 15; ++i) idx += beta[i] < u ? 1 : 0;
  return idx;
}

// The part of code `v` (slot s, byte lane i) that word w of a b-bit code
// group holds, in place (record layout v2).
__device__ __forceinline__ uint32_t code_bits(int b, int w, int s, int i, uint32_t v) {
  uint32_t f = 0;
  switch (b) {
    case 0: break;  // no code words
    case 1: f = w == 0 ? v << s : 0u; break;
    case 2: f = w == (s >> 2) ? v << (2 * (s & 3)) : 0u; break;
    case 4: f = w == (s >> 1) ? v << (4 * (s & 1)) : 0u; break;
    default:
      if (s < 6) {
        f = w == (s >> 1) ? v << (3 * (s & 1)) : 0u;
      } else {
        if (w == s - 6) f = (v & 3u) << 6;         // code bits 0-1 at bits 6-7 of word s - 6
        if (w == 2) f |= ((v >> 2) & 1u) << s;     // code bit 2 at bit s (6 or 7) of word 2
      }
  }
  return f << (8 * i);
}

__device__ __forceinline__ uint32_t code_mask(int b, int w, int s, int i) { return code_bits(b, w, s, i, 0xFu >> (4 - b)); }

// One workgroup's work of small_keys_kernel for block index bid.
__device__ __forceinline__ void small_keys_block(const SmallArgs& a, int64_t bid) {
  extern __shared__ float ssm[];
  float* xs = ssm;             // [d] input
  float* ys = xs + a.d;        // [d] R x
  float* rs = ys + a.d;        // [d] residual
  float* zs = rs + a.d;        // [m] S r
  int* is = (int*)(zs + a.m);  // [d] cells
  __shared__ float red[2 * (kSmallThreads / 64)];
  __shared__ float ctab[16];
  const int slot = (int)(bid / a.n_new);
  const int64_t t = bid - (int64_t)slot * a.n_new;
  float beta[15];
#pragma unroll
  for (int i = 0; i < 15; ++i) beta[i] = a.beta[i];
  if (threadIdx.x < 16) ctab[threadIdx.x] = a.cent[threadIdx.x];
  // (head_dim 128 with proj_dim 64 or 128 takes the matrix-core kernel, so
  // the matrices here are read row by row from L2)
  int ex = 0;
  const float ns = load_input(a, (int64_t)slot * a.n_new + t, xs, red, &ex);  // norm of the shifted row
  const float n = ldexpf(ns, ex);
  __syncthreads();
  matvec(a.r32, a.d, a.d, xs, ys);
  __syncthreads();
  const float inv = ns > 0.f ? 1.f / ns : 0.f;
  float g2 = 0.f;
  for (int j = threadIdx.x; j < a.d; j += blockDim.x) {
    const float u = ns > 0.f ? ys[j] * inv : 0.f;
    const int idx = cell(u, beta);
    const float r = u - ctab[idx];
    is[j] = idx;
    rs[j] = r;
    g2 = fmaf(r, r, g2);
  }
  const float gamma = sqrtf(block_sum(g2, red));  // (block_sum synchronises)
  matvec(a.s32, a.m, a.d, rs, zs);
  __syncthreads();
  uint32_t* rec = a.out + ((int64_t)slot * a.capacity + a.pos + t) * a.rec_words;
  const int n_full = a.d / 128, code_words = a.bits * a.d / 32, sign_words = a.m / 32;
  // code words: thread (word, slot s) places the 4 codes of slot s, the 8
  // slot threads of a word (consecutive lanes) are OR-ed by lane exchange;
  // full group (q, g) at words b (q n_full + g) ..; slot s, byte lane i is
  // coordinate 128 g + 16 s + 4 q + i.  A half chunk (d = 128 n + 64) has
  // groups p = 0, 1 at words b (4 n + p) ..; slot s, byte lane i is
  // coordinate 128 n + 16 (s % 4) + 4 (p + 2 (s / 4)) + i.
  for (int e0 = 0; e0 < code_words * 8; e0 += blockDim.x) {
    const int e = e0 + threadIdx.x, wi = e >> 3, sl = e & 7;
    uint32_t part = 0u;
    if (wi < code_words) {
      const int grp = wi / a.bits, w = wi % a.bits;
      const int base = grp < 4 * n_full ? 128 * (grp % n_full) + 16 * sl + 4 * (grp / n_full)
                                        : 128 * n_full + 16 * (sl % 4) + 4 * (grp - 4 * n_full + 2 * (sl / 4));
#pragma unroll
      for (int i = 0; i < 4; ++i) part |= code_bits(a.bits, w, sl, i, (uint32_t)is[base + i]);
    }
    part |= __shfl_xor(part, 1, 64);
    part |= __shfl_xor(part, 2, 64);
    part |= __shfl_xor(part, 4, 64);
    if (wi < code_words && sl == 0) rec[wi] = part;
  }
  // sign words: thread (word, bit) and a ballot per 32 bits.  Projection
  // 16 tt + 4 q + i is bit 16 (q%2) + 4 (tt%4) + i of word 2 (tt/4) + q/2;
  // a half block (m = 64 n' + 32) is word 2 n' with projection 64 n' + j at
  // bit j.
  for (int e0 = 0; e0 < sign_words * 32; e0 += blockDim.x) {
    const int e = e0 + threadIdx.x, sw = e >> 5, bit = e & 31;
    bool on = false;
    if (sw < sign_words) {
      const int h = bit >> 4, tt = 4 * (sw >> 1) + ((bit >> 2) & 3), q = 2 * (sw & 1) + h, i = bit & 3;
      on = zs[(sw & 1) == 0 && 32 * sw + 64 > a.m ? 32 * sw + bit : 16 * tt + 4 * q + i] >= 0.f;
    }
    const uint64_t mask = __ballot(on);
    if (sw < sign_words && bit == 0) rec[code_words + sw] = (uint32_t)(mask >> (threadIdx.x & 32));
  }
  if (threadIdx.x == 0) {
    rec[a.rec_words - 2] = __float_as_uint(n);
    rec[a.rec_words - 1] = __float_as_uint(gamma);
  }
}

// One workgroup's work of small_values_kernel for block index bid.
__device__ __forceinline__ void small_values_block(const SmallArgs& a, int64_t bid) {
  extern __shared__ float ssm[];
  float* xs = ssm;             // [d]
  float* ys = xs + a.d;        // [d]
  int* cs = (int*)(ys + a.d);  // [16][d] cells of the block's new tokens (at most 16)
  __shared__ float red[2 * (kSmallThreads / 64)];
  __shared__ float nrm[16];
  __shared__ int tau_of[16];
  const int64_t blk0 = a.pos / kBlockTokens;
  const int64_t nblk = (a.pos + a.n_new - 1) / kBlockTokens - blk0 + 1;
  const int slot = (int)(bid / nblk);
  const int64_t blk = blk0 + (bid - (int64_t)slot * nblk);
  const int64_t t_lo = max(a.pos, blk * kBlockTokens), t_hi = min(a.pos + a.n_new, (blk + 1) * kBlockTokens);
  const int nt = (int)(t_hi - t_lo);  // <= n_new <= 16
  float beta[15];
#pragma unroll
  for (int i = 0; i < 15; ++i) beta[i] = a.beta[i];
  const bool d128 = a.d == 128;
  HalfRows hr;
  if (d128) prefetch_rows(a.r32, 128, hr);
  for (int u = 0; u < nt; ++u) {
    const int64_t t = t_lo + u;
    int ex = 0;
    const float ns = load_input(a, (int64_t)slot * a.n_new + (t - a.pos), xs, red, &ex);  // shifted row's norm
    __syncthreads();
    if (d128) matvec_pref(hr, 128, xs, ys);
    else matvec(a.r32, a.d, a.d, xs, ys);
    __syncthreads();
    const float inv = ns > 0.f ? 1.f / ns : 0.f;
    for (int j = threadIdx.x; j < a.d; j += blockDim.x) cs[u * a.d + j] = cell(ns > 0.f ? ys[j] * inv : 0.f, beta);
    if (threadIdx.x == 0) {
      nrm[u] = ldexpf(ns, ex);
      tau_of[u] = (int)(t - blk * kBlockTokens);
    }
    __syncthreads();
  }
  uint32_t* vb = a.out + ((int64_t)slot * (a.capacity / kBlockTokens) + blk) * a.block_words;
  // word (w 4 + q) d + c holds, for coordinate c, the codes of block tokens
  // 16 s + 4 q + i (slot s, byte lane i)
  for (int e = threadIdx.x; e < 4 * a.bits * a.d; e += blockDim.x) {
    const int c = e % a.d, wq = e / a.d, q = wq % 4, w = wq / 4;
    uint32_t keep = 0xFFFFFFFFu, bits = 0u;
    for (int u = 0; u < nt; ++u) {
      const int tau = tau_of[u];
      if (((tau >> 2) & 3) != q) continue;
      const int s = tau >> 4, i = tau & 3;
      keep &= ~code_mask(a.bits, w, s, i);
      bits |= code_bits(a.bits, w, s, i, (uint32_t)cs[u * a.d + c]);
    }
    if (keep != 0xFFFFFFFFu) vb[e] = (vb[e] & keep) | bits;
  }
  float* vnorm = (float*)(vb + 4 * a.bits * a.d);
  if (threadIdx.x < nt) vnorm[tau_of[threadIdx.x]] = nrm[threadIdx.x];
}

// Host: the arguments of a small append.
inline SmallArgs small_args(const Matrices& mats, const CodebookDev& cb, int bits, int d, int m, const AppendShape& s,
                            void* out) {
  SmallArgs a;
  a.x = s.x;
  a.dtype = s.dtype;
  a.out = (uint32_t*)out;
  a.r32 = mats.r32;
  a.s32 = mats.s32;
  a.n_new = s.n_new;
  a.pos = s.pos;
  a.bid0 = 0;
  a.capacity = s.capacity;
  a.n_seq = s.n_seq;
  a.d = d;
  a.m = m;
  a.bits = bits;
  a.rec_words = bits * d / 32 + m / 32 + 2;
  a.block_words = 4 * bits * d + kBlockTokens;
  for (int i = 0; i < 16; ++i) {
    a.beta[i] = cb.beta[i];
    a.cent[i] = cb.cent[i];
  }
  return a;
}


}  // namespace tq
