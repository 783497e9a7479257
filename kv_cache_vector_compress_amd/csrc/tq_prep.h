// Query preparation shared by the attention paths and the fused decode step
// (device code, included by the .hip sources that launch it).
//
// q~ = R q and p = S q~ for one query head (the query side of the asymmetric
// estimate: nav.superapi.store "turboquant-pytorch", 常见使用模式), then the
// fp16 MFMA B operands divided by ||q||, in the lane layout the score and
// attend kernels read.
#pragma once

#include "tq_device.h"

namespace tq {

struct GenPrepArgs {
  const void* q;
  int dtype, G, HG, n_seq, d, m, n_oct;
  const float* r32;
  const float* s32;
  uint16_t* wq;   // [n_seq][HG][KBT][64][8] fp16, KBT = d/32 + m/32
  float* wqn;     // [n_seq][16 HG]
};

// The work of one workgroup (256 threads) for block index bid: slot
// bid / (16 HG), head lane bid % (16 HG).  Dynamic LDS: (2 d + m) floats.
__device__ __forceinline__ void gen_prep_block(const GenPrepArgs& a, int bid) {
  extern __shared__ float gsm[];
  float* qs = gsm;          // [d]
  float* qt = qs + a.d;     // [d]
  float* pp = qt + a.d;     // [m]
  __shared__ float red[8];
  const int H16 = 16 * a.HG;
  const int slot = bid / H16, h = bid % H16;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const bool live = h < a.G;
  // The query is kept in LDS shifted by 2^-e, 2^e the binary exponent of its
  // largest magnitude (exact), so that its norm and the products below
  // neither overflow nor underflow for any finite query; qn is the shifted
  // query's norm, the operands q~/||q|| are unchanged, and ||q|| = ldexp(qn, e).
  // (256 threads and d <= 1024: at most 4 coordinates a thread.)
  float v4[4], mx = 0.f;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int k = tid + i * (int)blockDim.x;
    v4[i] = 0.f;
    if (live && k < a.d) {
      const int64_t off = ((int64_t)slot * a.G + h) * a.d + k;
      v4[i] = a.dtype == TQ_F32 ? ((const float*)a.q)[off] : (float)((const _Float16*)a.q)[off];
    }
    mx = fmaxf(mx, fabsf(v4[i]));
  }
  // one block reduction of (exponent, sum of squares) partials
  int e;
  norm2_partial(mx, e);
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float u = ldexpf(v4[i], -e);
    s = fmaf(u, u, s);
  }
  wave_norm2(e, s);
  if (lane == 0) {
    red[2 * wave] = s;
    red[2 * wave + 1] = __int_as_float(e);
  }
  __syncthreads();
  float S = red[0];
  int ex = __float_as_int(red[1]);
#pragma unroll
  for (int w = 1; w < 4; ++w) merge_norm2(ex, S, __float_as_int(red[2 * w + 1]), red[2 * w]);
  if (ex == kNoExp) ex = 0;  // a zero query (or a head lane past G)
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int k = tid + i * (int)blockDim.x;
    if (k < a.d) qs[k] = ldexpf(v4[i], -ex);
  }
  const float qn = sqrtf(S);
  __syncthreads();  // qs complete
  // q~ = R q and p = S q~.  A head lane past G has q = 0 and takes no
  // products.  Each output row is split over 4 neighbouring threads (a
  // quarter of its columns each, all of their loads in flight at once), and
  // the quarters are summed with two lane exchanges.
  if (live) {
    auto rows = [&](const float* mat, int n_rows, const float* x, float* y) {
      const int c = tid & 3, d4 = a.d / 4;
      for (int j0 = 0; j0 < n_rows; j0 += blockDim.x / 4) {
        const int j = j0 + (tid >> 2);
        float t = 0.f;
        if (j < n_rows) {
          const f4* rr = (const f4*)(mat + (size_t)j * a.d + c * d4);
          const float* xx = x + c * d4;
          float t1 = 0.f;
#pragma unroll 8
          for (int k4 = 0; k4 < d4 / 4; k4 += 2) {
            const f4 u = rr[k4], v = rr[k4 + 1];
            t = fmaf(u[0], xx[4 * k4], fmaf(u[1], xx[4 * k4 + 1], fmaf(u[2], xx[4 * k4 + 2], fmaf(u[3], xx[4 * k4 + 3], t))));
            t1 = fmaf(v[0], xx[4 * k4 + 4], fmaf(v[1], xx[4 * k4 + 5], fmaf(v[2], xx[4 * k4 + 6], fmaf(v[3], xx[4 * k4 + 7], t1))));
          }
          t += t1;
        }
        t += shfl_xor(t, 1);
        t += shfl_xor(t, 2);
        if (j < n_rows && c == 0) y[j] = t;
      }
    };
    rows(a.r32, a.d, qs, qt);
    __syncthreads();
    rows(a.s32, a.m, qt, pp);
  } else {
    for (int k = tid; k < a.d; k += blockDim.x) qt[k] = 0.f;
    for (int i = tid; i < a.m; i += blockDim.x) pp[i] = 0.f;
  }
  __syncthreads();
  const float inv = live && qn > 0.f ? 1.f / qn : 0.f;
  const int KBT = a.d / 32 + a.m / 32;
  const int hg = h / 16, h16 = h % 16;
  for (int idx = tid; idx < KBT * 4; idx += blockDim.x) {
    const int kb = idx / 4, qq = idx % 4;
    h8 v;
    if (kb < a.d / 32) {
      // centroid part of chunk kb/4: k slot e <-> coordinate 128 (kb/4) + 16 (2 (kb%4) + e/4) + 4 qq + e%4
      const int base = 128 * (kb / 4) + 32 * (kb % 4);
      for (int e = 0; e < 8; ++e) v[e] = (_Float16)(qt[base + 16 * (e / 4) + 4 * qq + e % 4] * inv);
    } else {
      // sign part: k slot 2e+half <-> bit p + 16 half of sign word 2 (kbp/2) + qq/2,
      // p = 8 (qq%2) + 4 (kbp%2) + e, which holds projection coordinate 16 t + 4 qs + p%4
      // with qs = 2 (qq/2) + half, t = 4 (kbp/2) + p/4
      // (a half sign block, the last of m = 64 n' + 32, is one word in
      // projection order: k slot 2e+half <-> projection 64 n' + 16 half + 4 qq + e)
      const int kbp = kb - a.d / 32;
      const bool hb = 32 * kbp + 64 > a.m && (kbp % 2) == 0;
      for (int e = 0; e < 4; ++e)
        for (int half = 0; half < 2; ++half) {
          const int p = 8 * (qq % 2) + 4 * (kbp % 2) + e;
          const int qsg = 2 * (qq / 2) + half;
          const int t = 4 * (kbp / 2) + p / 4;
          const int j = hb ? 32 * kbp + 16 * half + 4 * qq + e : 16 * t + 4 * qsg + p % 4;
          v[2 * e + half] = (_Float16)(pp[j] * inv);
        }
    }
    const int l = 16 * qq + h16;
    *(h8*)(a.wq + ((((int64_t)slot * a.HG + hg) * KBT + kb) * 64 + l) * 8) = v;
  }
  if (tid == 0) a.wqn[(int64_t)slot * H16 + h] = live ? ldexpf(qn, ex) : 0.f;
}


}  // namespace tq
