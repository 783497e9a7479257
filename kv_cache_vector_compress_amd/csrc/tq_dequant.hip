// Stage-1 reconstruction of cached keys and values for gfx950:
//     x^ = ||x|| R^T c[idx]
// (nav.superapi.store "turboquant-pytorch", 核心 API: TurboQuantMSE.dequantize
// and TurboQuantKVCache.get_values; 生产级压缩器: the value compressor keeps
// only the MSE reconstruction).  For keys this is the MSE part: the QJL sign
// bits estimate inner products and do not reconstruct the residual.
//
// Not on the attention path (the attend kernel never materialises x^): this
// serves consumers that want the vectors back.  One workgroup takes 32
// tokens of one slot.  It decodes their codes into LDS in the rotated domain
// (c[idx], coordinate-major), then thread (coordinate c, token half) forms
// sum_j R[j][c] y[j][t] in fp32 with R's row j read across threads
// (coalesced) and y broadcast from LDS, and scales the sum by ||x|| last (no
// intermediate overflows or denormals at any norm).  Any head_dim of the
// layout.
#include "tq_device.h"
#include "tq_layout.h"

namespace tq {

constexpr int kDqTok = 32;  // tokens per workgroup

struct DequantArgs {
  const uint32_t* key_rec;
  const uint32_t* val_blocks;
  const float* r32;  // R, [d][d] row-major
  float* out;        // [n_seq][n_tokens][d]
  int64_t pos, n_tokens, capacity;
  int n_seq, d, bits, rec_words, block_words;
  int keys;          // 1: key records, 0: value blocks
  float cent[16];
};

// Code of slot s, byte lane i of a code group whose b words sit `stride`
// words apart (record layout v2).
__device__ __forceinline__ int group_code(const uint32_t* w, int stride, int b, int s, int i) {
  const int sh = 8 * i;
  auto byte = [&](int k) { return (w[k * stride] >> sh) & 0xFFu; };
  switch (b) {
    case 0: return 0;  // one cell
    case 1: return (byte(0) >> s) & 1;
    case 2: return (byte(s >> 2) >> (2 * (s & 3))) & 3;
    case 4: return (byte(s >> 1) >> (4 * (s & 1))) & 15;
    default:
      if (s < 6) return (byte(s >> 1) >> (3 * (s & 1))) & 7;
      return ((byte(s - 6) >> 6) & 3) | (((byte(2) >> s) & 1) << 2);  // s = 6: bit 6 of word 2; s = 7: bit 7
  }
}

__global__ __launch_bounds__(256) void dequant_kernel(const DequantArgs a) {
  extern __shared__ __align__(16) float ys[];  // [d][kDqTok] centroids of the codes
  __shared__ float nsh[kDqTok];                // the tokens' norms, applied last
  const int64_t tiles = (a.n_tokens + kDqTok - 1) / kDqTok;
  const int slot = (int)(blockIdx.x / tiles);
  const int64_t tl0 = (int64_t)(blockIdx.x - (int64_t)slot * tiles) * kDqTok;  // first token, relative to pos
  const int nt = (int)min((int64_t)kDqTok, a.n_tokens - tl0);
  const int nblk = (int)(a.capacity / kBlockTokens);
  auto key_rec = [&](int tl) { return a.key_rec + ((int64_t)slot * a.capacity + a.pos + tl0 + tl) * a.rec_words; };
  auto val_blk = [&](int tl) {
    return a.val_blocks + ((int64_t)slot * nblk + (a.pos + tl0 + tl) / kBlockTokens) * a.block_words;
  };
  if (threadIdx.x < kDqTok) {
    const int tl = threadIdx.x;
    float n = 0.f;
    if (tl < nt)
      n = __uint_as_float(a.keys ? key_rec(tl)[a.rec_words - 2]
                                 : val_blk(tl)[4 * a.bits * a.d + (int)((a.pos + tl0 + tl) % kBlockTokens)]);
    nsh[tl] = n;
  }
  for (int e = threadIdx.x; e < a.d * kDqTok; e += blockDim.x) {
    const int tl = e % kDqTok, j = e / kDqTok;
    float v = 0.f;
    if (tl < nt) {
      int code;
      if (a.keys) {
        int word, sl;
        key_code_place(j, a.d, a.bits, word, sl);
        code = group_code(key_rec(tl) + word, 1, a.bits, sl, j & 3);
      } else {
        const int tau = (int)((a.pos + tl0 + tl) % kBlockTokens);
        code = group_code(val_blk(tl) + ((tau >> 2) & 3) * a.d + j, 4 * a.d, a.bits, tau >> 4, tau & 3);
      }
      v = a.cent[code];
    }
    ys[j * kDqTok + tl] = v;
  }
  __syncthreads();
  const int half = threadIdx.x >> 7;  // tokens 16 half .. 16 half + 15
  for (int c = threadIdx.x & 127; c < a.d; c += 128) {
    float acc[16];
#pragma unroll
    for (int u = 0; u < 16; ++u) acc[u] = 0.f;
    for (int j = 0; j < a.d; ++j) {
      const float r = a.r32[(size_t)j * a.d + c];
      const f4* y = (const f4*)(ys + j * kDqTok + 16 * half);
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const f4 yy = y[u];
        acc[4 * u] = fmaf(r, yy[0], acc[4 * u]);
        acc[4 * u + 1] = fmaf(r, yy[1], acc[4 * u + 1]);
        acc[4 * u + 2] = fmaf(r, yy[2], acc[4 * u + 2]);
        acc[4 * u + 3] = fmaf(r, yy[3], acc[4 * u + 3]);
      }
    }
#pragma unroll
    for (int u = 0; u < 16; ++u) {
      const int tl = 16 * half + u;
      if (tl < nt) a.out[((int64_t)slot * a.n_tokens + tl0 + tl) * a.d + c] = acc[u] * nsh[tl];
    }
  }
}

int dequant_device_init() {
  // up to head_dim 1024: 1024 x 32 fp32 of decoded coordinates in LDS
  return hipFuncSetAttribute((const void*)dequant_kernel, hipFuncAttributeMaxDynamicSharedMemorySize,
                             (int)(sizeof(float) * 1024 * kDqTok)) == hipSuccess
             ? 0 : -1;
}

int launch_dequant(const Matrices& mats, const CodebookDev& cb, int bits, int d, int m, bool keys,
                   const void* key_records, const void* value_blocks, int64_t capacity, int n_seq, int64_t pos,
                   int64_t n_tokens, float* out, void* stream) {
  DequantArgs a;
  a.key_rec = (const uint32_t*)key_records;
  a.val_blocks = (const uint32_t*)value_blocks;
  a.r32 = mats.r32;
  a.out = out;
  a.pos = pos;
  a.n_tokens = n_tokens;
  a.capacity = capacity;
  a.n_seq = n_seq;
  a.d = d;
  a.bits = bits;
  a.rec_words = bits * d / 32 + m / 32 + 2;
  a.block_words = 4 * bits * d + kBlockTokens;
  a.keys = keys ? 1 : 0;
  for (int i = 0; i < 16; ++i) a.cent[i] = cb.cent[i];
  const int64_t tiles = (n_tokens + kDqTok - 1) / kDqTok;
  const size_t lds = sizeof(float) * (size_t)d * kDqTok;
  hipLaunchKernelGGL(dequant_kernel, dim3((unsigned)(tiles * n_seq)), dim3(256), lds, (hipStream_t)stream, a);
  return hipGetLastError() == hipSuccess ? 0 : TQ_EDEVICE;
}

}  // namespace tq
