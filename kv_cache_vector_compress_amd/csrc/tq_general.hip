// General-shape path on gfx950: head_dim d a multiple of 64 up to 1024,
// proj_dim m a multiple of 32 up to 512 (the d = 128, m in {64, 128} shapes
// have their own single-kernel path in tq_compress.hip / tq_attention.hip).
//
// The computation is the same as on the fast path (nav.superapi.store
// "turboquant-pytorch", 主要能力 / 算法细节; atskills.one Stage 1 / Stage 2):
//   keys:   y = R k / ||k||, idx = #{i : beta_i < y}, r = y - c[idx],
//           gamma = ||r||, s = [S r >= 0]
//   values: y = R v / ||v||, idx
//   scores: est = ||k|| (<R q, c[idx]> + gamma sqrt(pi/2)/m <S R q, 2s - 1>)
// with the same split-fp16 arithmetic (R, S scaled by 2^8 and split into fp16
// hi + lo; fp16 inputs exact, fp32 inputs split after a power-of-two scale)
// and the same record layout (a d of 128 n + 64 ends in a half chunk and an
// m of 64 n' + 32 in a half sign block, tq_layout.h).  The kernels work on
// whole 128-coordinate chunks and 64-projection tiles: the R and S images
// carry zero rows up to those sizes, and the coordinates and projections
// past d and m are computed as zeros and never stored or summed.  What
// changes is the blocking: R (up to 4 MB as hi/lo
// fp16) no longer fits in LDS, so the rotation and the projection are tiled
// GEMMs that stream 32-column slices of R and S through LDS, and the key
// residual goes through a scratch buffer between the two.
//
//   gen_row_norms     ||x|| of every row of the launch
//   gen_keys_rotate   y for a 128-token x 128-coordinate tile; cells, codes,
//                     residual (to scratch, fp16 hi/lo in slot order), and
//                     the tile's share of gamma^2
//   gen_keys_project  z = S r for a 64-token x 64-projection tile; sign bits,
//                     and gamma from the shares
//   gen_values        y for one 128-token block x 128 coordinates; codes
//   gen_prep_queries  q~ = R q and p = S q~ per query head, as MFMA operands
//   gen_scores        scores of 16 tokens for every query head
#include <algorithm>

#include "tq_device.h"
#include "tq_layout.h"
#include "tq_prep.h"

namespace tq {

constexpr int kSliceLS = 40;  // LDS row stride (halves) of a 32-column slice: conflict-free b128 reads

struct GenArgs {
  const void* x;
  int64_t n_new;      // tokens per slot in x (the call's n_new)
  int64_t pos;        // the call's first token position
  int64_t tok_off;    // first token of this launch, relative to x
  int64_t n_sub;      // tokens per slot in this launch
  int64_t capacity;
  int n_seq, d, m, n_oct, ld, rec_words, block_words;
  const uint16_t* r_hi;
  const uint16_t* r_lo;
  const uint16_t* s_hi;
  const uint16_t* s_lo;
  float* nrm;         // [n_seq * n_sub] rows' (||x 2^-e||, e): norm of the row shifted by its exponent
  uint16_t* res_hi;   // [n_seq * n_sub][d] residual 2^12 (y - c), slot order, fp16 high part
  uint16_t* res_lo;
  float* g2p;         // [n_seq * n_sub][n_oct] partial sums of the squared residual
  uint32_t* out;      // key records or value blocks
  _Float16 m1;        // -1 (a run-time value: see split2m)
  CodebookDev cb;
};

// Input row of launch row r (slot-major over the launch's tokens).
__device__ __forceinline__ int64_t gen_in_row(const GenArgs& a, int64_t r) {
  const int64_t slot = r / a.n_sub;
  return slot * a.n_new + a.tok_off + (r - slot * a.n_sub);
}

// A slice of an fp16 image pair (hi, lo; row stride ld halves): rows
// [row0, row0 + NR) x columns [k0, k0 + 32), 2 NR 16-byte pieces, fetched
// into registers by a 256-thread workgroup (NR / 32 pieces a thread) and then
// stored into LDS (row stride kSliceLS).  The fetch of the next slice is
// issued before the current one is multiplied, so its latency is hidden.
template <int NR>
struct Slice {
  static constexpr int kPer = 2 * NR * 4 / 256;
  u4 v[kPer];
  __device__ __forceinline__ void fetch(const uint16_t* hi, const uint16_t* lo, int ld, int row0, int k0) {
#pragma unroll
    for (int j = 0; j < kPer; ++j) {
      const int i = threadIdx.x + 256 * j;
      const int img = i / (NR * 4), rr = (i / 4) % NR, cc = (i % 4) * 8;
      v[j] = *(const u4*)((img ? lo : hi) + (size_t)(row0 + rr) * ld + k0 + cc);
    }
  }
  __device__ __forceinline__ void store(uint16_t* lds) const {  // lds: [2][NR * kSliceLS]
#pragma unroll
    for (int j = 0; j < kPer; ++j) {
      const int i = threadIdx.x + 256 * j;
      const int img = i / (NR * 4), rr = (i / 4) % NR, cc = (i % 4) * 8;
      *(u4*)(lds + img * NR * kSliceLS + rr * kSliceLS + cc) = v[j];
    }
  }
};

// 8 inputs of a row as an MFMA operand: fp16 rows as they are; fp32 rows
// scaled by sc (|x sc| < 2^13) and split into fp16 hi + lo.
template <bool F32>
__device__ __forceinline__ void load_x8(const void* x, int64_t row, int d, int k, int sh, h8& xh, h8& xl) {
  if constexpr (F32) {
    const float* p = (const float*)x + row * d + k;
    const f4 v0 = *(const f4*)p, v1 = *(const f4*)(p + 4);
    u4 hi, lo;
    HiLo t = split2(ldexpf(v0[0], sh), ldexpf(v0[1], sh));
    hi[0] = t.hi; lo[0] = t.lo;
    t = split2(ldexpf(v0[2], sh), ldexpf(v0[3], sh));
    hi[1] = t.hi; lo[1] = t.lo;
    t = split2(ldexpf(v1[0], sh), ldexpf(v1[1], sh));
    hi[2] = t.hi; lo[2] = t.lo;
    t = split2(ldexpf(v1[2], sh), ldexpf(v1[3], sh));
    hi[3] = t.hi; lo[3] = t.lo;
    xh = as_h8(hi);
    xl = as_h8(lo);
  } else {
    xh = *(const h8*)((const _Float16*)x + row * d + k);
  }
}

// Workgroup -> (row tile, chunk) for a 1-D grid of ntiles x nchunk
// workgroups.  Consecutive workgroups go to the 8 XCDs in turn, each with its
// own L2; this order sends all chunks of a row tile to the same XCD, close
// together in time, so the tile's rows come from HBM once and then from that
// L2.
__device__ __forceinline__ void xcd_tile_chunk(int64_t b, int64_t ntiles, int nchunk, int64_t& tile, int& chunk) {
  const int64_t full = ntiles / 8 * 8;      // row tiles in complete groups of 8
  if (b < full * nchunk) {
    const int64_t grp = b / (8 * nchunk), rem = b % (8 * nchunk);
    chunk = (int)(rem / 8);
    tile = grp * 8 + rem % 8;
  } else {
    const int64_t r = b - full * nchunk, tail = ntiles - full;
    chunk = (int)(r / tail);
    tile = full + r % tail;
  }
}


// ---------------------------------------------------------------------------

__global__ __launch_bounds__(256) void gen_row_norms(const GenArgs a, int dtype) {
  const int64_t r = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (r >= (int64_t)a.n_seq * a.n_sub) return;
  const int64_t row = gen_in_row(a, r);
  float s = 0.f;
  int ex = 0;
  if (dtype == TQ_F32) {
    // (pre-scaled by the largest magnitude: any finite row; d <= 1024, so a
    // lane holds at most 4 quads)
    const float* p = (const float*)a.x + row * a.d;
    f4 v[4];
    float mx = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int c = 4 * lane + 256 * i;
      v[i] = c < a.d ? *(const f4*)(p + c) : f4{0.f, 0.f, 0.f, 0.f};
      mx = fmaxf(mx, fmaxf(fmaxf(fabsf(v[i][0]), fabsf(v[i][1])), fmaxf(fabsf(v[i][2]), fabsf(v[i][3]))));
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) mx = fmaxf(mx, shfl_xor(mx, o));
    ex = pow2_exponent(mx);
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float u = ldexpf(v[i][e], -ex);
        s = fmaf(u, u, s);
      }
  } else {
    const _Float16* p = (const _Float16*)a.x + row * a.d;
    for (int c = 8 * lane; c < a.d; c += 512) {
      const h8 v = *(const h8*)(p + c);
#pragma unroll
      for (int e = 0; e < 8; e += 2) s = __builtin_amdgcn_fdot2(h2{v[e], v[e + 1]}, h2{v[e], v[e + 1]}, s, false);
    }
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) s += shfl_xor(s, o);
  if (lane == 0) ((float2*)a.nrm)[r] = make_float2(sqrtf(s), (float)ex);
}

// ---------------------------------------------------------------------------
// keys, part 1: rotation of a 128-row x 128-coordinate tile (4 waves x 2
// 16-row tiles; coordinates on the MFMA M axis, so a lane ends up with 32
// coordinates of one row: one code group), then cells, codes and residual.
// ---------------------------------------------------------------------------

template <int B, bool F32>
__global__ __launch_bounds__(256) void gen_keys_rotate(const GenArgs a) {
  constexpr int H = 1 << (B - 1);
  __shared__ __align__(16) uint16_t Rs[2][2 * 128 * kSliceLS];  // [buffer][hi, lo][128 rows]
  __shared__ float ctab[16];
  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int r16 = lane & 15, q = lane >> 4;
  const int64_t rows = (int64_t)a.n_seq * a.n_sub;
  int64_t rtile;
  int u;  // coordinate chunk
  xcd_tile_chunk(blockIdx.x, (rows + 127) / 128, a.n_oct, rtile, u);
  if (tid < 16) ctab[tid] = a.cb.cent[tid] * kResScale;

  int64_t row[2], in_row[2];
  float n[2], sigma[2];
  int sh[2];  // fp32 pre-shift: |x 2^sh| < 2^13; 0 for fp16
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    row[j] = rtile * 128 + wave * 32 + 16 * j + r16;
    const int64_t rr = row[j] < rows ? row[j] : rows - 1;  // rows past the end: any valid row, not stored
    in_row[j] = gen_in_row(a, rr);
    const float2 ne = ((const float2*)a.nrm)[rr];
    const int ex = (int)ne.y, s0 = input_shift(ne.x);
    n[j] = ldexpf(ne.x, ex);
    sh[j] = F32 ? s0 - ex : 0;
    sigma[j] = kRotScale * (F32 ? ldexpf(ne.x, s0) : n[j]);
  }
  f4 acc[2][8];
#pragma unroll
  for (int j = 0; j < 2; ++j)
#pragma unroll
    for (int s = 0; s < 8; ++s) acc[j][s] = f4{0.f, 0.f, 0.f, 0.f};

  Slice<128> sl;
  sl.fetch(a.r_hi, a.r_lo, a.ld, 128 * u, 0);
  h8 xh[2], xl[2];
#pragma unroll
  for (int j = 0; j < 2; ++j) load_x8<F32>(a.x, in_row[j], a.d, 8 * q, sh[j], xh[j], xl[j]);
  sl.store(Rs[0]);
  __syncthreads();
  for (int k0 = 0, buf = 0; k0 < a.d; k0 += 32, buf ^= 1) {
    const bool more = k0 + 32 < a.d;
    h8 nh[2], nl[2];
    if (more) {
      sl.fetch(a.r_hi, a.r_lo, a.ld, 128 * u, k0 + 32);
#pragma unroll
      for (int j = 0; j < 2; ++j) load_x8<F32>(a.x, in_row[j], a.d, k0 + 32 + 8 * q, sh[j], nh[j], nl[j]);
    }
    const uint16_t* Rh = Rs[buf];
    const uint16_t* Rl = Rs[buf] + 128 * kSliceLS;
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      const h8 ah = *(const h8*)(Rh + (16 * s + r16) * kSliceLS + 8 * q);
      const h8 al = *(const h8*)(Rl + (16 * s + r16) * kSliceLS + 8 * q);
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        acc[j][s] = mfma(ah, xh[j], acc[j][s]);
        acc[j][s] = mfma(al, xh[j], acc[j][s]);
        if constexpr (F32) acc[j][s] = mfma(ah, xl[j], acc[j][s]);
      }
    }
    if (more) {
      sl.store(Rs[buf ^ 1]);
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        xh[j] = nh[j];
        xl[j] = nl[j];
      }
    }
    __syncthreads();
  }

  float bpos[8];
  load_pos_beta<B>(bpos, a.cb);
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const bool valid = row[j] < rows;
    const float s16 = n[j] > 0.f ? kResScale / sigma[j] : 0.f;
    float bs[8];
#pragma unroll
    for (int t = 0; t < 8; ++t) bs[t] = t < H - 1 ? bpos[t] * sigma[j] : 0.f;
    uint32_t cw[B];
#pragma unroll
    for (int w = 0; w < B; ++w) cw[w] = 0u;
    float g2 = 0.f;
    // a half chunk (the last 64 coordinates of d = 128 n + 64) keeps slots
    // 0..3: its rotated coordinates 16 s + 4 q + i with s >= 4 lie past d
    const int n_kb2 = min(4, (a.d - 128 * u) / 32);
#pragma unroll
    for (int kb2 = 0; kb2 < 4; ++kb2) {
      if (kb2 >= n_kb2) break;
      u4 rhi, rlo;
#pragma unroll
      for (int uu = 0; uu < 2; ++uu) {
        float rs[4];
        const uint32_t x4 = quantize4<B>(acc[j][2 * kb2 + uu], bs, s16, ctab, rs, g2);
        const HiLo t01 = split2m(rs[0], rs[1], a.m1), t23 = split2m(rs[2], rs[3], a.m1);
        rhi[2 * uu] = t01.hi;
        rlo[2 * uu] = t01.lo;
        rhi[2 * uu + 1] = t23.hi;
        rlo[2 * uu + 1] = t23.lo;
        put_sel4_rt<B>(cw, 2 * kb2 + uu, x4);
      }
      if (valid) {
        const size_t o = (size_t)row[j] * a.d + 128 * u + 32 * kb2 + 8 * q;
        *(u4*)(a.res_hi + o) = rhi;
        *(u4*)(a.res_lo + o) = rlo;
      }
    }
    g2 += shfl_xor(g2, 16);
    g2 += shfl_xor(g2, 32);
    const int n_full = key_full_chunks(a.d);
    const bool half = u >= n_full;  // (uniform over the workgroup)
    if (half) {
      // lane groups q and q + 2 share code group q % 2: q + 2 takes slots
      // 4..7, and the two halves are merged across lanes l and l ^ 32
      if (q >= 2) lift_half<B>(cw);
#pragma unroll
      for (int w = 0; w < B; ++w) cw[w] |= (uint32_t)__shfl_xor((int)cw[w], 32, 64);
    }
    if (valid) {
      const int64_t slot = row[j] / a.n_sub, t = row[j] - slot * a.n_sub;
      uint32_t* rp = a.out + (slot * a.capacity + a.pos + a.tok_off + t) * a.rec_words;
      if (!half || q < 2) {
        const int w0 = key_group_word(q, u, n_full, B);
#pragma unroll
        for (int w = 0; w < B; ++w) rp[w0 + w] = cw[w];
      }
      if (q == 0) a.g2p[row[j] * a.n_oct + u] = g2;
      if (q == 0 && u == 0) rp[a.rec_words - 2] = __float_as_uint(n[j]);
    }
  }
}

// ---------------------------------------------------------------------------
// keys, part 2: z = S r for a 64-row x 64-projection tile (4 waves x 16
// rows; projection coordinates on M), sign bits, and gamma.
// ---------------------------------------------------------------------------

__global__ __launch_bounds__(256) void gen_keys_project(const GenArgs a, int bits) {
  __shared__ __align__(16) uint16_t Ss[2][2 * 64 * kSliceLS];  // [buffer][hi, lo][64 rows]
  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int r16 = lane & 15, q = lane >> 4;
  const int64_t rows = (int64_t)a.n_seq * a.n_sub;
  int64_t rtile;
  int u;  // 64-projection chunk
  xcd_tile_chunk(blockIdx.x, (rows + 63) / 64, sign_blocks(a.m), rtile, u);
  const int64_t row = rtile * 64 + wave * 16 + r16;
  const int64_t rr = row < rows ? row : rows - 1;
  f4 z[4];
#pragma unroll
  for (int p = 0; p < 4; ++p) z[p] = f4{0.f, 0.f, 0.f, 0.f};
  const uint16_t* rhp = a.res_hi + (size_t)rr * a.d + 8 * q;
  const uint16_t* rlp = a.res_lo + (size_t)rr * a.d + 8 * q;
  Slice<64> sv;
  sv.fetch(a.s_hi, a.s_lo, a.ld, 64 * u, 0);
  h8 rh = *(const h8*)rhp, rl = *(const h8*)rlp;
  sv.store(Ss[0]);
  __syncthreads();
  for (int k0 = 0, buf = 0; k0 < a.d; k0 += 32, buf ^= 1) {
    const bool more = k0 + 32 < a.d;
    h8 nh, nl;
    if (more) {
      sv.fetch(a.s_hi, a.s_lo, a.ld, 64 * u, k0 + 32);
      nh = *(const h8*)(rhp + k0 + 32);
      nl = *(const h8*)(rlp + k0 + 32);
    }
    const uint16_t* Sh = Ss[buf];
    const uint16_t* Sl = Ss[buf] + 64 * kSliceLS;
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      const h8 sh = *(const h8*)(Sh + (16 * p + r16) * kSliceLS + 8 * q);
      const h8 sl = *(const h8*)(Sl + (16 * p + r16) * kSliceLS + 8 * q);
      z[p] = mfma(sh, rh, z[p]);
      z[p] = mfma(sl, rh, z[p]);
      z[p] = mfma(sh, rl, z[p]);
    }
    if (more) {
      sv.store(Ss[buf ^ 1]);
      rh = nh;
      rl = nl;
    }
    __syncthreads();
  }
  const uint32_t bits16 = sign_bits16(z[0], z[1], z[2], z[3]);
  // A half block (the last 32 projections of m = 64 n' + 32) is one word
  // holding projection 64 u + j at bit j: lane group q holds j = 16 p + 4 q + i
  // at bit 4 p + i (p = 0, 1), and the four lane groups' parts are merged.
  const bool half_blk = 64 * u + 64 > a.m;  // (uniform over the workgroup)
  uint32_t hw = 0u;
  if (half_blk) {
    hw = ((bits16 & 0xFu) << (4 * q)) | (((bits16 >> 4) & 0xFu) << (16 + 4 * q));
    hw |= (uint32_t)__shfl_xor((int)hw, 16, 64);
    hw |= (uint32_t)__shfl_xor((int)hw, 32, 64);
  }
  if (row < rows) {
    const int64_t slot = row / a.n_sub, t = row - slot * a.n_sub;
    uint32_t* rp = a.out + (slot * a.capacity + a.pos + a.tok_off + t) * a.rec_words;
    const int sw0 = bits * a.d / 32;
    if (!half_blk) ((uint16_t*)(rp + sw0 + 2 * u + (q >> 1)))[q & 1] = (uint16_t)bits16;
    else if (q == 0) rp[sw0 + 2 * u] = hw;
    if (u == 0 && q == 1) {
      float g = 0.f;
      for (int c = 0; c < a.n_oct; ++c) g += a.g2p[row * a.n_oct + c];
      rp[a.rec_words - 1] = __float_as_uint(sqrtf(g) * (1.f / kResScale));
    }
  }
}

// ---------------------------------------------------------------------------
// values: one 128-token block of one slot x one 128-coordinate chunk.  Tokens
// on M (so a lane ends up with one coordinate of 4 tokens per tile, the
// order of the value block); wave w owns coordinate tiles 2w and 2w + 1 of
// the chunk for all 8 token tiles, i.e. whole code words.
// ---------------------------------------------------------------------------

template <int B, bool F32>
__global__ __launch_bounds__(256) void gen_values(const GenArgs a) {
  __shared__ __align__(16) uint16_t Rs[2][2 * 128 * kSliceLS];  // [buffer][hi, lo][128 rows]
  __shared__ float inv_sh[kBlockTokens];  // 1 / sigma per block token (0: not in this launch or zero row)
  __shared__ float nrm_sh[kBlockTokens];
  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int r16 = lane & 15, q = lane >> 4;
  const int64_t P0 = a.pos + a.tok_off, P1 = P0 + a.n_sub;  // token positions of this launch
  const int64_t blk0 = P0 / kBlockTokens, nblk = (P1 - 1) / kBlockTokens - blk0 + 1;
  int64_t item;
  int u;
  xcd_tile_chunk(blockIdx.x, nblk * a.n_seq, a.n_oct, item, u);
  const int64_t slot = item / nblk, blk = blk0 + (item - slot * nblk);
  const int64_t tok0 = blk * kBlockTokens;
  if (tid < kBlockTokens) {
    const int64_t p = tok0 + tid;
    const bool valid = p >= P0 && p < P1;
    const float2 ne = valid ? ((const float2*)a.nrm)[slot * a.n_sub + (p - P0)] : make_float2(0.f, 0.f);
    const float nn = ldexpf(ne.x, (int)ne.y);
    const float sigma = kRotScale * (F32 ? ldexpf(ne.x, input_shift(ne.x)) : nn);
    inv_sh[tid] = sigma > 0.f ? 1.f / sigma : 0.f;
    nrm_sh[tid] = nn;
  }
  // A operand rows: block token 16 mt + r16
  int64_t in_row[8];
  int sh[8];  // fp32 pre-shift (input_shift); 0 for fp16
#pragma unroll
  for (int mt = 0; mt < 8; ++mt) {
    int64_t p = tok0 + 16 * mt + r16;
    p = p < P0 ? P0 : (p >= P1 ? P1 - 1 : p);  // clamp to a row of this launch (codes masked later)
    const int64_t r = slot * a.n_sub + (p - P0);
    in_row[mt] = gen_in_row(a, r);
    const float2 ne = ((const float2*)a.nrm)[r];
    sh[mt] = F32 ? input_shift(ne.x) - (int)ne.y : 0;
  }
  f4 acc[8][2];
#pragma unroll
  for (int mt = 0; mt < 8; ++mt) acc[mt][0] = acc[mt][1] = f4{0.f, 0.f, 0.f, 0.f};
  Slice<128> sl;
  sl.fetch(a.r_hi, a.r_lo, a.ld, 128 * u, 0);
  sl.store(Rs[0]);
  __syncthreads();
  for (int k0 = 0, buf = 0; k0 < a.d; k0 += 32, buf ^= 1) {
    const bool more = k0 + 32 < a.d;
    if (more) sl.fetch(a.r_hi, a.r_lo, a.ld, 128 * u, k0 + 32);
    const uint16_t* Rh = Rs[buf];
    const uint16_t* Rl = Rs[buf] + 128 * kSliceLS;
    h8 bh[2], bl[2];
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      bh[t] = *(const h8*)(Rh + (16 * (2 * wave + t) + r16) * kSliceLS + 8 * q);
      bl[t] = *(const h8*)(Rl + (16 * (2 * wave + t) + r16) * kSliceLS + 8 * q);
    }
#pragma unroll
    for (int mt = 0; mt < 8; ++mt) {
      h8 xh, xl;
      load_x8<F32>(a.x, in_row[mt], a.d, k0 + 8 * q, sh[mt], xh, xl);
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        acc[mt][t] = mfma(xh, bh[t], acc[mt][t]);
        acc[mt][t] = mfma(xh, bl[t], acc[mt][t]);
        if constexpr (F32) acc[mt][t] = mfma(xl, bh[t], acc[mt][t]);
      }
    }
    if (more) sl.store(Rs[buf ^ 1]);
    __syncthreads();
  }

  float bpos[8];
  load_pos_beta<B>(bpos, a.cb);
  float bsx[4][8];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int t = 0; t < 8; ++t) bsx[i][t] = bpos[t];
  uint32_t cw[2][B];
#pragma unroll
  for (int t = 0; t < 2; ++t)
#pragma unroll
    for (int w = 0; w < B; ++w) cw[t][w] = 0u;
#pragma unroll
  for (int mt = 0; mt < 8; ++mt) {
    const f4 inv = *(const f4*)&inv_sh[16 * mt + 4 * q];
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      f4 y = acc[mt][t];
#pragma unroll
      for (int i = 0; i < 4; ++i) y[i] *= inv[i];
      put_sel4_rt<B>(cw[t], mt, cells4<B>(y, bsx));
    }
  }
  uint32_t* vb = a.out + (slot * (a.capacity / kBlockTokens) + blk) * a.block_words;
  const bool full = tok0 >= P0 && tok0 + kBlockTokens <= P1;
  uint32_t keep[B];  // bits of tokens outside this launch: left as they are
#pragma unroll
  for (int w = 0; w < B; ++w) keep[w] = 0u;
  if (!full)
    for (int s = 0; s < 8; ++s)
      for (int i = 0; i < 4; ++i) {
        const int64_t p = tok0 + 16 * s + 4 * q + i;
        if (p < P0 || p >= P1)
#pragma unroll
          for (int w = 0; w < B; ++w) keep[w] |= field_mask_rt(B, s, w, i);
      }
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    const int c = 128 * u + 16 * (2 * wave + t) + r16;
    if (128 * u + 16 * (2 * wave + t) >= a.d) break;  // past a half chunk (wave-uniform)
#pragma unroll
    for (int w = 0; w < B; ++w) {
      uint32_t* wp = vb + (size_t)(w * 4 + q) * a.d + c;
      *wp = full ? cw[t][w] : ((*wp & keep[w]) | (cw[t][w] & ~keep[w]));
    }
  }
  if (u == 0 && tid < kBlockTokens) {
    const int64_t p = tok0 + tid;
    if (p >= P0 && p < P1) ((float*)(vb + 4 * B * a.d))[tid] = nrm_sh[tid];
  }
}

// ---------------------------------------------------------------------------
// query preparation: one workgroup per (slot, query head) of the padded head
// range; q~ = R q and p = S q~ in fp32, then the fp16 MFMA B operands
// (divided by ||q||) in the lanes of this head.
// ---------------------------------------------------------------------------

// (GenPrepArgs and gen_prep_block: tq_prep.h)
__global__ __launch_bounds__(256) void gen_prep_queries(const GenPrepArgs a) { gen_prep_block(a, (int)blockIdx.x); }

// The same operands for d = 128 and m = 64, one workgroup of 512 threads
// per (slot, group of 16 head lanes): thread t holds a quarter of R's row
// t/4 and an eighth of S's row t/8 in registers, loaded before the queries
// arrive, and applies them to every live head of the group (R and S are read
// once per group rather than once per head).
__global__ __launch_bounds__(512) void prep_queries128(const GenPrepArgs a) {
  constexpr int D = 128, Mp = 64, KBT = D / 32 + Mp / 32;
  __shared__ __align__(16) float qs[16][D];
  __shared__ __align__(16) float qt[16][D];
  __shared__ float pp[16][Mp];
  __shared__ float qn[16];  // norms of the shifted queries
  __shared__ int qe[16];    // their shifts: ||q|| = ldexp(qn, qe)
  const int slot = blockIdx.x / a.HG, hg = blockIdx.x % a.HG;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int nl = max(0, min(16, a.G - 16 * hg));  // live head lanes of this group
  f4 rv[8], sv[4];
  {
    const f4* rr = (const f4*)(a.r32 + (size_t)(tid >> 2) * D + 32 * (tid & 3));
#pragma unroll
    for (int u = 0; u < 8; ++u) rv[u] = rr[u];
    const f4* sr = (const f4*)(a.s32 + (size_t)(tid >> 3) * D + 16 * (tid & 7));
#pragma unroll
    for (int u = 0; u < 4; ++u) sv[u] = sr[u];
  }
  for (int i = tid; i < 16 * D; i += blockDim.x) {
    const int hh = i / D, k = i % D;
    float v = 0.f;
    if (hh < nl) {
      const int64_t off = ((int64_t)slot * a.G + 16 * hg + hh) * D + k;
      v = a.dtype == TQ_F32 ? ((const float*)a.q)[off] : (float)((const _Float16*)a.q)[off];
    }
    qs[hh][k] = v;
  }
  __syncthreads();
  // each query shifted by 2^-e, 2^e the binary exponent of its largest
  // magnitude (exact): norms and products neither overflow nor underflow for
  // any finite query, and the operands q~/||q|| are unchanged
  for (int hh = wave; hh < 16; hh += 8) {
    const float x0 = qs[hh][lane], x1 = qs[hh][lane + 64];
    float mx = fmaxf(fabsf(x0), fabsf(x1));
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) mx = fmaxf(mx, shfl_xor(mx, o));
    const int ex = pow2_exponent(mx);
    const float u0 = ldexpf(x0, -ex), u1 = ldexpf(x1, -ex);
    qs[hh][lane] = u0;
    qs[hh][lane + 64] = u1;
    float s = u0 * u0 + u1 * u1;
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) s += shfl_xor(s, o);
    if (lane == 0) {
      qn[hh] = sqrtf(s);
      qe[hh] = ex;
    }
  }
  __syncthreads();
  // q~ = R q: row tid/4, columns 32 (tid%4) ..; the four parts summed by lane exchanges
  for (int hh = 0; hh < nl; ++hh) {
    const f4* x = (const f4*)(&qs[hh][32 * (tid & 3)]);
    float t0 = 0.f, t1 = 0.f;
#pragma unroll
    for (int u = 0; u < 8; u += 2) {
      const f4 x0 = x[u], x1 = x[u + 1];
      t0 = fmaf(rv[u][0], x0[0], fmaf(rv[u][1], x0[1], fmaf(rv[u][2], x0[2], fmaf(rv[u][3], x0[3], t0))));
      t1 = fmaf(rv[u + 1][0], x1[0], fmaf(rv[u + 1][1], x1[1], fmaf(rv[u + 1][2], x1[2], fmaf(rv[u + 1][3], x1[3], t1))));
    }
    float t = t0 + t1;
    t += shfl_xor(t, 1);
    t += shfl_xor(t, 2);
    if ((tid & 3) == 0) qt[hh][tid >> 2] = t;
  }
  __syncthreads();
  // p = S q~: row tid/8, columns 16 (tid%8) ..
  for (int hh = 0; hh < nl; ++hh) {
    const f4* x = (const f4*)(&qt[hh][16 * (tid & 7)]);
    float z0 = 0.f, z1 = 0.f;
#pragma unroll
    for (int u = 0; u < 4; u += 2) {
      const f4 x0 = x[u], x1 = x[u + 1];
      z0 = fmaf(sv[u][0], x0[0], fmaf(sv[u][1], x0[1], fmaf(sv[u][2], x0[2], fmaf(sv[u][3], x0[3], z0))));
      z1 = fmaf(sv[u + 1][0], x1[0], fmaf(sv[u + 1][1], x1[1], fmaf(sv[u + 1][2], x1[2], fmaf(sv[u + 1][3], x1[3], z1))));
    }
    float z = z0 + z1;
    z += shfl_xor(z, 1);
    z += shfl_xor(z, 2);
    z += shfl_xor(z, 4);
    if ((tid & 7) == 0) pp[hh][tid >> 3] = z;
  }
  __syncthreads();
  // operands, as gen_prep_queries lays them out (zeros for head lanes past G)
  for (int idx = tid; idx < 16 * KBT * 4; idx += blockDim.x) {
    const int h16 = idx / (KBT * 4), kb = (idx / 4) % KBT, qq = idx % 4;
    const bool live = h16 < nl;
    const float inv = live && qn[h16] > 0.f ? 1.f / qn[h16] : 0.f;
    h8 v;
    if (kb < D / 32) {
      const int base = 32 * kb;
#pragma unroll
      for (int e = 0; e < 8; ++e) v[e] = (_Float16)(live ? qt[h16][base + 16 * (e / 4) + 4 * qq + e % 4] * inv : 0.f);
    } else {
      const int kbp = kb - D / 32;
#pragma unroll
      for (int e = 0; e < 4; ++e)
#pragma unroll
        for (int half = 0; half < 2; ++half) {
          const int p = 8 * (qq % 2) + 4 * (kbp % 2) + e;
          const int qsg = 2 * (qq / 2) + half;
          const int t = 4 * (kbp / 2) + p / 4;
          v[2 * e + half] = (_Float16)(live ? pp[h16][16 * t + 4 * qsg + p % 4] * inv : 0.f);
        }
    }
    const int l = 16 * qq + h16;
    *(h8*)(a.wq + ((((int64_t)slot * a.HG + hg) * KBT + kb) * 64 + l) * 8) = v;
  }
  if (tid < 16) a.wqn[((int64_t)slot * a.HG + hg) * 16 + tid] = tid < nl ? ldexpf(qn[tid], qe[tid]) : 0.f;
}

// ---------------------------------------------------------------------------
// scores: one wave per 16-token tile; every chunk of a key record is decoded
// once and multiplied by the query operands of all HG head groups.
// ---------------------------------------------------------------------------

struct GenScoreArgs {
  const uint32_t* rec;
  float* scores;
  const uint16_t* wq;
  const float* wqn;
  int64_t n_tokens, capacity;
  int n_seq, G, HG, d, m, n_oct, rec_words;
  int64_t tiles_per_slot;
  int64_t gw0;  // first (slot, tile) wave of this launch
  float kappa;
  uint32_t tlo[4], thi[4];
};

template <int B, int HG>
__global__ __launch_bounds__(256) void gen_scores(const GenScoreArgs a) {
  const int lane = threadIdx.x & 63;
  const int r16 = lane & 15, q = lane >> 4;
  const int64_t gw = a.gw0 + (int64_t)blockIdx.x * 4 + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  if (gw >= a.tiles_per_slot * a.n_seq) return;
  const int slot = (int)(gw / a.tiles_per_slot);
  const int64_t tile = gw - (int64_t)slot * a.tiles_per_slot;
  const int n_tok = (int)a.n_tokens;
  const int t = min((int)(tile * 16) + r16, n_tok - 1);
  const uint32_t* rp = a.rec + ((int64_t)slot * a.capacity + t) * a.rec_words;
  const int KBT = a.d / 32 + a.m / 32;
  const uint16_t* wq = a.wq + (int64_t)slot * HG * KBT * 64 * 8 + lane * 8;
  uint32_t tlo[4], thi[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) { tlo[i] = a.tlo[i]; thi[i] = a.thi[i]; }
  f4 acc[HG];
#pragma unroll
  for (int g = 0; g < HG; ++g) acc[g] = f4{0.f, 0.f, 0.f, 0.f};
  // 0-bit keys have the single centroid 0: no MSE term
  if constexpr (B > 0) {
    const int n_full = key_full_chunks(a.d);
    for (int c = 0; c < n_full; ++c) {
      uint32_t cw[B];
#pragma unroll
      for (int w = 0; w < B; ++w) cw[w] = rp[(q * n_full + c) * B + w];
      const h8 A0 = decode_pair<B, 0>(cw, tlo, thi), A1 = decode_pair<B, 2>(cw, tlo, thi);
      const h8 A2 = decode_pair<B, 4>(cw, tlo, thi), A3 = decode_pair<B, 6>(cw, tlo, thi);
#pragma unroll
      for (int g = 0; g < HG; ++g) {
        const uint16_t* wg = wq + ((int64_t)g * KBT + 4 * c) * 64 * 8;
        acc[g] = mfma(A0, *(const h8*)(wg), acc[g]);
        acc[g] = mfma(A1, *(const h8*)(wg + 64 * 8), acc[g]);
        acc[g] = mfma(A2, *(const h8*)(wg + 2 * 64 * 8), acc[g]);
        acc[g] = mfma(A3, *(const h8*)(wg + 3 * 64 * 8), acc[g]);
      }
    }
    if (a.d % 128) {  // the half chunk: this lane group's slots 0..3 (two K blocks)
      uint32_t cw[B];
      const int w0 = key_group_word(q, n_full, n_full, B);
#pragma unroll
      for (int w = 0; w < B; ++w) cw[w] = rp[w0 + w];
      uint32_t cl[B];
#pragma unroll
      for (int w = 0; w < B; ++w) cl[w] = cw[w];
      lower_half<B>(cl);
#pragma unroll
      for (int w = 0; w < B; ++w) cw[w] = q >= 2 ? cl[w] : cw[w];
      const h8 A0 = decode_pair<B, 0>(cw, tlo, thi), A1 = decode_pair<B, 2>(cw, tlo, thi);
#pragma unroll
      for (int g = 0; g < HG; ++g) {
        const uint16_t* wg = wq + ((int64_t)g * KBT + 4 * n_full) * 64 * 8;
        acc[g] = mfma(A0, *(const h8*)(wg), acc[g]);
        acc[g] = mfma(A1, *(const h8*)(wg + 64 * 8), acc[g]);
      }
    }
  }
  const float gamma = __uint_as_float(rp[a.rec_words - 1]);
  const _Float16 gk = (_Float16)(gamma * a.kappa);
  const uint32_t gk2 = (uint32_t)__builtin_bit_cast(uint16_t, gk) * 0x00010001u;
  const int sh0 = 15 - 8 * (q & 1);
  const int sw0 = B * a.d / 32;
  for (int kbp = 0; kbp < a.m / 32; ++kbp) {
    // a half sign block (the last one of m = 64 n' + 32) is one word in
    // projection order: lane group q takes bits 4 q + e and 16 + 4 q + e
    const bool hb = 32 * kbp + 64 > a.m && (kbp % 2) == 0;
    const uint32_t w = ~rp[sw0 + 2 * (kbp / 2) + (hb ? 0 : (q >> 1))];
    const int sh1 = hb ? 15 - 4 * q : sh0 - 4 * (kbp % 2);
    u4 v;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const uint32_t sh = w << (sh1 - e);  // bits p, p+16 -> 15, 31
      v[e] = (sh & 0x80008000u) | (gk2 & 0x7FFF7FFFu);
    }
    const h8 A = as_h8(v);
#pragma unroll
    for (int g = 0; g < HG; ++g)
      acc[g] = mfma(A, *(const h8*)(wq + ((int64_t)g * KBT + a.d / 32 + kbp) * 64 * 8), acc[g]);
  }
  // acc[g][i]: token row 4q+i of the tile, query head 16 g + r16; ||k|| of
  // token row 4q+i comes from the lanes that loaded that record
  const float kn = __uint_as_float(rp[a.rec_words - 2]);
  f4 nk;
#pragma unroll
  for (int i = 0; i < 4; ++i) nk[i] = __shfl(kn, 4 * q + i, 64);
  const int t0 = (int)(tile * 16) + 4 * q;
  // a lane's 4 tokens of a head row are one 16-byte store when rows start
  // 16-byte aligned (the score buffer aligned and n_tokens a multiple of 4)
  const bool vec = (n_tok & 3) == 0 && ((uintptr_t)a.scores & 15) == 0 && t0 + 4 <= n_tok;
#pragma unroll
  for (int g = 0; g < HG; ++g) {
    const int h = 16 * g + r16;
    if (h >= a.G) continue;
    const float qn = a.wqn[(int64_t)slot * 16 * HG + h];
    float* out = a.scores + ((int64_t)slot * a.G + h) * (int64_t)n_tok;
    if (vec) {
      *(f4*)(out + t0) = acc[g] * nk * qn;
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i)
        if (t0 + i < n_tok) out[t0 + i] = acc[g][i] * nk[i] * qn;
    }
  }
}

// Scores for many head groups (HG >= 4, e.g. 512 queries against one slot):
// a wave takes NT consecutive tiles and the head groups CG at a time.  Only
// CG groups' accumulators are live, so the kernel holds ~100 registers a
// lane (gen_scores<4, 32> holds ~330, one wave per SIMD) and runs several
// waves per SIMD; the key words are decoded again for every group chunk.
// With NT > 1 each query operand read from L2 would feed NT tiles' products,
// but the registers that costs measured slower than the waves it loses.
// Each accumulator (tile, head group) takes its products in gen_scores'
// order (chunks, half chunk, sign blocks; K blocks in order), so the
// estimates are the same bits.
template <int B, int NT, int CG>
__global__ __launch_bounds__(256) void gen_scores_blk(const GenScoreArgs a) {
  const int lane = threadIdx.x & 63;
  const int r16 = lane & 15, q = lane >> 4;
  const int64_t wps = (a.tiles_per_slot + NT - 1) / NT;  // waves per slot
  const int64_t gw = a.gw0 + (int64_t)blockIdx.x * 4 + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  if (gw >= wps * a.n_seq) return;
  const int slot = (int)(gw / wps);
  const int64_t tile0 = (gw - (int64_t)slot * wps) * NT;
  const int n_tok = (int)a.n_tokens;
  const uint32_t* rp[NT];
  float gkf[NT];
  f4 nk[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    const int tok = min((int)((tile0 + t) * 16) + r16, n_tok - 1);
    rp[t] = a.rec + ((int64_t)slot * a.capacity + tok) * a.rec_words;
    gkf[t] = __uint_as_float(rp[t][a.rec_words - 1]) * a.kappa;
    const float kn = __uint_as_float(rp[t][a.rec_words - 2]);
#pragma unroll
    for (int i = 0; i < 4; ++i) nk[t][i] = __shfl(kn, 4 * q + i, 64);
  }
  const int KBT = a.d / 32 + a.m / 32;
  const uint16_t* wq = a.wq + (int64_t)slot * a.HG * KBT * 64 * 8 + lane * 8;
  uint32_t tlo[4], thi[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) { tlo[i] = a.tlo[i]; thi[i] = a.thi[i]; }
  const int sh0 = 15 - 8 * (q & 1);
  const int sw0 = B * a.d / 32;
  const bool vec = (n_tok & 3) == 0 && ((uintptr_t)a.scores & 15) == 0;
  for (int g0 = 0; g0 < a.HG; g0 += CG) {
    f4 acc[NT][CG];
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
      for (int g = 0; g < CG; ++g) acc[t][g] = f4{0.f, 0.f, 0.f, 0.f};
    const uint16_t* wg0 = wq + (int64_t)g0 * KBT * 64 * 8;
    if constexpr (B > 0) {
      const int n_full = key_full_chunks(a.d);
      auto kblock = [&](const uint32_t (&cw)[NT][B], int kb, auto kk_tag) {
        constexpr int KK = decltype(kk_tag)::value;
        h8 A[NT];
#pragma unroll
        for (int t = 0; t < NT; ++t) A[t] = decode_pair<B, 2 * KK>(cw[t], tlo, thi);
#pragma unroll
        for (int g = 0; g < CG; ++g) {
          const h8 b = *(const h8*)(wg0 + ((int64_t)g * KBT + kb) * 64 * 8);
#pragma unroll
          for (int t = 0; t < NT; ++t) acc[t][g] = mfma(A[t], b, acc[t][g]);
        }
      };
      for (int c = 0; c < n_full; ++c) {
        uint32_t cw[NT][B];
#pragma unroll
        for (int t = 0; t < NT; ++t)
#pragma unroll
          for (int w = 0; w < B; ++w) cw[t][w] = rp[t][(q * n_full + c) * B + w];
        kblock(cw, 4 * c, std::integral_constant<int, 0>{});
        kblock(cw, 4 * c + 1, std::integral_constant<int, 1>{});
        kblock(cw, 4 * c + 2, std::integral_constant<int, 2>{});
        kblock(cw, 4 * c + 3, std::integral_constant<int, 3>{});
      }
      if (a.d % 128) {  // the half chunk: this lane group's slots 0..3 (two K blocks)
        uint32_t cw[NT][B];
        const int w0 = key_group_word(q, n_full, n_full, B);
#pragma unroll
        for (int t = 0; t < NT; ++t) {
          uint32_t cl[B];
#pragma unroll
          for (int w = 0; w < B; ++w) cw[t][w] = cl[w] = rp[t][w0 + w];
          lower_half<B>(cl);
#pragma unroll
          for (int w = 0; w < B; ++w) cw[t][w] = q >= 2 ? cl[w] : cw[t][w];
        }
        kblock(cw, 4 * n_full, std::integral_constant<int, 0>{});
        kblock(cw, 4 * n_full + 1, std::integral_constant<int, 1>{});
      }
    }
    for (int kbp = 0; kbp < a.m / 32; ++kbp) {
      const bool hb = 32 * kbp + 64 > a.m && (kbp % 2) == 0;
      const int sh1 = hb ? 15 - 4 * q : sh0 - 4 * (kbp % 2);
      h8 A[NT];
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        const uint32_t w = ~rp[t][sw0 + 2 * (kbp / 2) + (hb ? 0 : (q >> 1))];
        const _Float16 gk = (_Float16)gkf[t];
        const uint32_t gk2 = (uint32_t)__builtin_bit_cast(uint16_t, gk) * 0x00010001u;
        u4 v;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const uint32_t sh = w << (sh1 - e);  // bits p, p+16 -> 15, 31
          v[e] = (sh & 0x80008000u) | (gk2 & 0x7FFF7FFFu);
        }
        A[t] = as_h8(v);
      }
#pragma unroll
      for (int g = 0; g < CG; ++g) {
        const h8 b = *(const h8*)(wg0 + ((int64_t)g * KBT + a.d / 32 + kbp) * 64 * 8);
#pragma unroll
        for (int t = 0; t < NT; ++t) acc[t][g] = mfma(A[t], b, acc[t][g]);
      }
    }
#pragma unroll
    for (int g = 0; g < CG; ++g) {
      const int h = 16 * (g0 + g) + r16;
      if (h >= a.G) continue;
      const float qn = a.wqn[(int64_t)slot * 16 * a.HG + h];
      float* out = a.scores + ((int64_t)slot * a.G + h) * (int64_t)n_tok;
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        const int t0 = (int)((tile0 + t) * 16) + 4 * q;
        if (vec && t0 + 4 <= n_tok) {
          *(f4*)(out + t0) = acc[t][g] * nk[t] * qn;
        } else {
#pragma unroll
          for (int i = 0; i < 4; ++i)
            if (t0 + i < n_tok) out[t0 + i] = acc[t][g][i] * nk[t][i] * qn;
        }
      }
    }
  }
}

// ---------------------------------------------------------------------------
// attend (general shapes): the scores come from gen_scores (materialised in
// the workspace); each wave runs the online softmax over a range of 128-token
// blocks of one slot and accumulates sum_t p_t ||v_t|| c[idx_t] for one
// 128-coordinate chunk of the output (the P V product of the single-kernel
// path, with the value words of that chunk), and gen_combine merges the
// ranges (log-sum-exp) and applies R^T.
// ---------------------------------------------------------------------------

constexpr int kGenPart = 4 + 128;  // m, l, pad, pad, acc[128] per (slot, range, chunk, head)

struct GenAttendArgs {
  const float* scores;   // [n_seq][G][n_tokens] unscaled estimates
  const uint32_t* vblocks;
  float* part;           // [n_seq][ranges][n_oct][G][kGenPart]
  int64_t n_tokens, capacity;
  int n_seq, G, d, n_oct, block_words;
  int blocks_per_wave, ranges;
  float scale2;          // scale * log2(e)
  uint32_t vtlo[4], vthi[4];
};

__device__ __forceinline__ uint32_t pack_h2f(float x0, float x1) {
  const h2 v = {(_Float16)x0, (_Float16)x1};
  return __builtin_bit_cast(uint32_t, v);
}

template <int BV>
__global__ __launch_bounds__(256) void gen_attend_kernel(const GenAttendArgs a) {
  __shared__ __align__(16) float vsh[4][kBlockTokens];  // per wave: ||v|| 2^-ve of the block's tokens
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int r16 = lane & 15, q = lane >> 4;
  const int64_t gw = (int64_t)blockIdx.x * 4 + wave;
  if (gw >= (int64_t)a.n_seq * a.ranges * a.n_oct) return;
  const int u = (int)(gw % a.n_oct);  // chunk fastest: the chunk waves of a range read the same scores
  const int64_t sr = gw / a.n_oct;
  const int slot = (int)(sr / a.ranges), rg = (int)(sr % a.ranges);
  const int n_tok = (int)a.n_tokens;
  const int nblk = (n_tok + kBlockTokens - 1) / kBlockTokens;
  const int b_begin = rg * a.blocks_per_wave, b_end = min(nblk, b_begin + a.blocks_per_wave);
  const int h = r16;
  const bool head_ok = h < a.G;
  const float* srow = a.scores + ((int64_t)slot * a.G + (head_ok ? h : 0)) * (int64_t)n_tok;
  const uint32_t* vbase = a.vblocks + (int64_t)slot * (a.capacity / kBlockTokens) * a.block_words;
  uint32_t vtlo[4], vthi[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) { vtlo[i] = a.vtlo[i]; vthi[i] = a.vthi[i]; }

  float m_run = -INFINITY, l_run = 0.f;
  int ve = -1000;  // running exponent of the value norms (wave-uniform)
  f4 acc[8];
#pragma unroll
  for (int nt = 0; nt < 8; ++nt) acc[nt] = f4{0.f, 0.f, 0.f, 0.f};
  for (int blk = b_begin; blk < b_end; ++blk) {
    const int tok0 = blk * kBlockTokens;
    const uint32_t* vb = vbase + (int64_t)blk * a.block_words;
    uint32_t vw[8][BV];
    // (a half chunk has coordinate tiles 0..3 only; the others decode zero
    // words into products that are never read)
#pragma unroll
    for (int nt = 0; nt < 8; ++nt)
#pragma unroll
      for (int w = 0; w < BV; ++w)
        vw[nt][w] = 128 * u + 16 * nt < a.d ? vb[(w * 4 + q) * a.d + 128 * u + 16 * nt + r16] : 0u;
    const float2 vn2 = *(const float2*)(vb + 4 * BV * a.d + 2 * lane);
    const float x0 = tok0 + 2 * lane < n_tok ? vn2.x : 0.f, x1 = tok0 + 2 * lane + 1 < n_tok ? vn2.y : 0.f;
    float bmax = fmaxf(x0, x1);
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) bmax = fmaxf(bmax, shfl_xor(bmax, o));
    int e_blk = 0;
    frexpf(bmax, &e_blk);
    if (e_blk > ve) {
      const float f = ldexpf(1.f, ve - e_blk);
#pragma unroll
      for (int nt = 0; nt < 8; ++nt) acc[nt] *= f;
      ve = e_blk;
    }
    const float vs = ldexpf(1.f, -ve);
    *(float2*)&vsh[wave][2 * lane] = make_float2(x0 * vs, x1 * vs);
#pragma unroll
    for (int step = 0; step < 4; ++step) {
      float lg[2][4];
      float cmax = -INFINITY;
#pragma unroll
      for (int uu = 0; uu < 2; ++uu) {
        const int t0 = tok0 + 16 * (2 * step + uu) + 4 * q;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float l = (head_ok && t0 + i < n_tok) ? srow[t0 + i] * a.scale2 : -INFINITY;
          lg[uu][i] = l;
          cmax = fmaxf(cmax, l);
        }
      }
      cmax = fmaxf(cmax, shfl_xor(cmax, 16));
      cmax = fmaxf(cmax, shfl_xor(cmax, 32));
      if (__any(cmax > m_run)) {
        const float m_new = fmaxf(m_run, cmax);
        const float alpha = m_new == -INFINITY ? 1.f : exp2_hw(m_run - m_new);
#pragma unroll
        for (int nt = 0; nt < 8; ++nt) acc[nt] *= alpha;
        l_run *= alpha;
        m_run = m_new;
      }
      u4 pw;
      float psum = 0.f;
#pragma unroll
      for (int uu = 0; uu < 2; ++uu) {
        const f4 vn = *(const f4*)&vsh[wave][16 * (2 * step + uu) + 4 * q];
#pragma unroll
        for (int i2 = 0; i2 < 2; ++i2) {
          const float p0 = m_run == -INFINITY ? 0.f : exp2_hw(lg[uu][2 * i2] - m_run);
          const float p1 = m_run == -INFINITY ? 0.f : exp2_hw(lg[uu][2 * i2 + 1] - m_run);
          psum += p0 + p1;
          pw[2 * uu + i2] = pack_h2f(p0 * vn[2 * i2], p1 * vn[2 * i2 + 1]);
        }
      }
      l_run += psum;
      const h8 P = as_h8(pw);
#pragma unroll
      for (int nt = 0; nt < 8; ++nt) {
        h8 A;
        if (step == 0) A = decode_pair<BV, 0>(vw[nt], vtlo, vthi);
        if (step == 1) A = decode_pair<BV, 2>(vw[nt], vtlo, vthi);
        if (step == 2) A = decode_pair<BV, 4>(vw[nt], vtlo, vthi);
        if (step == 3) A = decode_pair<BV, 6>(vw[nt], vtlo, vthi);
        acc[nt] = mfma(A, P, acc[nt]);
      }
    }
  }
  l_run += shfl_xor(l_run, 16);
  l_run += shfl_xor(l_run, 32);
  // (the accumulator stays in the scale of P, 2^-ve, with ve stored beside
  // it; gen_combine merges the ranges at their largest exponent)
  if (head_ok) {
    float* pr = a.part + ((((int64_t)slot * a.ranges + rg) * a.n_oct + u) * a.G + h) * kGenPart;
    if (q == 0) {
      pr[0] = m_run;
      pr[1] = l_run;
      pr[2] = (float)ve;
    }
#pragma unroll
    for (int nt = 0; nt < 8; ++nt) *(f4*)(pr + 4 + 16 * nt + 4 * q) = acc[nt];
  }
}

struct GenCombineArgs {
  const float* part;
  float* out;   // [n_seq][G][d]
  const float* r32;
  int n_seq, G, d, n_oct, ranges;
};

// One workgroup per (slot, query head): out = 2^VE R^T (sum_r w_r 2^(ve_r - VE)
// acc_r) / sum_r w_r l_r, w_r = exp2(m_r - max_r m_r), VE the largest ve_r of
// the ranges that carry weight (the accumulators are stored at scale 2^-ve_r).
__global__ __launch_bounds__(256) void gen_combine(const GenCombineArgs a) {
  extern __shared__ float ysh[];  // [d] combined rotated-domain accumulator, then [ranges] weights
  float* wsh = ysh + a.d;
  __shared__ float red[4], rede[4];
  __shared__ float Msh, Lsh, Esh;
  const int sh = blockIdx.x, slot = sh / a.G, h = sh % a.G, tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  auto P = [&](int r, int u) { return a.part + ((((int64_t)slot * a.ranges + r) * a.n_oct + u) * a.G + h) * kGenPart; };
  float mx = -INFINITY, ex = -INFINITY;
  for (int r = tid; r < a.ranges; r += blockDim.x) {
    const float mr = P(r, 0)[0];
    mx = fmaxf(mx, mr);
    if (mr != -INFINITY) ex = fmaxf(ex, P(r, 0)[2]);
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    mx = fmaxf(mx, shfl_xor(mx, o));
    ex = fmaxf(ex, shfl_xor(ex, o));
  }
  if (lane == 0) {
    red[wave] = mx;
    rede[wave] = ex;
  }
  __syncthreads();
  if (tid == 0) {
    Msh = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
    Esh = fmaxf(fmaxf(rede[0], rede[1]), fmaxf(rede[2], rede[3]));
  }
  __syncthreads();
  const float M = Msh;
  const int VE = Esh == -INFINITY ? 0 : (int)Esh;
  float L = 0.f;
  for (int r = tid; r < a.ranges; r += blockDim.x) {
    const float mr = P(r, 0)[0];
    const float w = (mr == -INFINITY || M == -INFINITY) ? 0.f : exp2f(mr - M);
    wsh[r] = ldexpf(w, (int)P(r, 0)[2] - VE);
    L += w * P(r, 0)[1];
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) L += shfl_xor(L, o);
  __syncthreads();
  if (lane == 0) red[wave] = L;
  __syncthreads();
  if (tid == 0) Lsh = (red[0] + red[1]) + (red[2] + red[3]);
  for (int c = tid; c < a.d; c += blockDim.x) {
    const int u = c / 128, cc = c % 128;
    float y = 0.f;
    for (int r = 0; r < a.ranges; ++r) y = fmaf(wsh[r], P(r, u)[4 + cc], y);
    ysh[c] = y;
  }
  __syncthreads();
  const float inv = Lsh > 0.f ? 1.f / Lsh : 0.f;
  float* out = a.out + ((int64_t)slot * a.G + h) * a.d;
  for (int j = tid; j < a.d; j += blockDim.x) {
    float t = 0.f;
    for (int i = 0; i < a.d; ++i) t = fmaf(a.r32[(size_t)i * a.d + j], ysh[i], t);
    out[j] = ldexpf(t * inv, VE);
  }
}

// ---------------------------------------------------------------------------
// launchers
// ---------------------------------------------------------------------------

static GenArgs gen_args(const GenMats& g, const CodebookDev& cb, int bits, const AppendShape& s, int d, int m,
                        int64_t tok_off, int64_t n_sub, void* out) {
  GenArgs a;
  a.x = s.x;
  a.n_new = s.n_new;
  a.pos = s.pos;
  a.tok_off = tok_off;
  a.n_sub = n_sub;
  a.capacity = s.capacity;
  a.n_seq = s.n_seq;
  a.d = d;
  a.m = m;
  a.n_oct = key_chunks(d);
  a.ld = g.ld;
  a.rec_words = bits * d / 32 + m / 32 + 2;
  a.block_words = 4 * bits * d + kBlockTokens;
  a.r_hi = g.mats.r_hi;
  a.r_lo = g.mats.r_lo;
  a.s_hi = g.mats.s_hi;
  a.s_lo = g.mats.s_lo;
  a.nrm = g.nrm;
  a.res_hi = g.res_hi;
  a.res_lo = g.res_lo;
  a.g2p = g.g2p;
  a.out = (uint32_t*)out;
  a.m1 = (_Float16)-1.0f;
  a.cb = cb;
  return a;
}

// Tokens per slot of one launch: the scratch holds scratch_rows rows, and for
// values the split points must fall on block boundaries.
static int64_t gen_sub_tokens(const GenMats& g, int n_seq) {
  int64_t t = g.scratch_rows / n_seq;
  t -= t % kBlockTokens;
  return t < kBlockTokens ? kBlockTokens : t;
}

int launch_general_keys(const GenMats& g, const CodebookDev& cb, int bits, int d, int m, const AppendShape& s,
                        void* key_records, void* stream) {
  hipStream_t st = (hipStream_t)stream;
  const int64_t sub = gen_sub_tokens(g, s.n_seq);
  if (sub * s.n_seq > g.scratch_rows) return TQ_EUNSUPPORTED;
  for (int64_t off = 0; off < s.n_new; off += sub) {
    const int64_t n_sub = s.n_new - off < sub ? s.n_new - off : sub;
    const GenArgs a = gen_args(g, cb, bits, s, d, m, off, n_sub, key_records);
    const int64_t rows = n_sub * s.n_seq;
    hipLaunchKernelGGL(gen_row_norms, dim3((unsigned)((rows + 3) / 4)), dim3(256), 0, st, a, s.dtype);
    const dim3 g1((unsigned)((rows + 127) / 128 * key_chunks(d))), g2((unsigned)((rows + 63) / 64 * sign_blocks(m)));
    const bool f32 = s.dtype == TQ_F32;
#define TQ_GK(B)                                                                              \
  if (bits == B) {                                                                            \
    if (f32) hipLaunchKernelGGL((gen_keys_rotate<B, true>), g1, dim3(256), 0, st, a);        \
    else hipLaunchKernelGGL((gen_keys_rotate<B, false>), g1, dim3(256), 0, st, a);           \
  }
    TQ_GK(1) TQ_GK(2) TQ_GK(3) TQ_GK(4)
#undef TQ_GK
    hipLaunchKernelGGL(gen_keys_project, g2, dim3(256), 0, st, a, bits);
    if (hipGetLastError() != hipSuccess) return TQ_EDEVICE;
  }
  return 0;
}

int launch_general_values(const GenMats& g, const CodebookDev& cb, int bits, int d, const AppendShape& s,
                          void* value_blocks, void* stream) {
  hipStream_t st = (hipStream_t)stream;
  const int64_t sub = gen_sub_tokens(g, s.n_seq);
  if (sub * s.n_seq > g.scratch_rows) return TQ_EUNSUPPORTED;  // (the row norms live in the scratch)
  // launch boundaries at absolute multiples of sub (a multiple of 128): no
  // value block is touched by two launches
  int64_t off = 0;
  while (off < s.n_new) {
    const int64_t p = s.pos + off;
    const int64_t end_abs = (p / sub + 1) * sub;
    int64_t n_sub = end_abs - p;
    if (n_sub > s.n_new - off) n_sub = s.n_new - off;
    const GenArgs a = gen_args(g, cb, bits, s, d, 64, off, n_sub, value_blocks);
    const int64_t rows = n_sub * s.n_seq;
    hipLaunchKernelGGL(gen_row_norms, dim3((unsigned)((rows + 3) / 4)), dim3(256), 0, st, a, s.dtype);
    const int64_t nblk = (p + n_sub - 1) / kBlockTokens - p / kBlockTokens + 1;
    const dim3 g1((unsigned)(nblk * s.n_seq * key_chunks(d)));
    const bool f32 = s.dtype == TQ_F32;
#define TQ_GV(B)                                                                   \
  if (bits == B) {                                                                 \
    if (f32) hipLaunchKernelGGL((gen_values<B, true>), g1, dim3(256), 0, st, a);  \
    else hipLaunchKernelGGL((gen_values<B, false>), g1, dim3(256), 0, st, a);     \
  }
    TQ_GV(1) TQ_GV(2) TQ_GV(3) TQ_GV(4)
#undef TQ_GV
    if (hipGetLastError() != hipSuccess) return TQ_EDEVICE;
    off += n_sub;
  }
  return 0;
}

static int head_groups_bucket(int G) {
  const int HG = (G + 15) / 16;
  int b = 1;
  while (b < HG) b *= 2;
  return b;
}

size_t general_scores_workspace(int d, int m, int n_seq, int G) {
  const int HG = head_groups_bucket(G);
  const size_t q_bytes = (size_t)n_seq * HG * (d / 32 + m / 32) * 64 * 8 * 2;
  const size_t qn_bytes = (size_t)n_seq * HG * 16 * 4;
  return ((q_bytes + 255) / 256 + (qn_bytes + 255) / 256) * 256;
}

int launch_gen_prep(const Matrices& mats, int d, int m, const AttnShape& s, int HG, uint16_t* wq, float* wqn,
                    void* stream) {
  // one head group at head_dim 128: the decode step's preparation on the
  // matrix cores, one workgroup per slot (tq_step.hip); the score kernels,
  // attend and top-k of these shapes all read its operands
  if (d == 128 && HG == 1 && (m == 64 || m == 128) && mats.r_hi && mats.p_hi)
    return launch_prep_step(mats, m, s, wq, wqn, stream);
  GenPrepArgs p;
  p.q = s.q;
  p.dtype = s.dtype;
  p.G = s.G;
  p.HG = HG;
  p.n_seq = s.n_seq;
  p.d = d;
  p.m = m;
  p.n_oct = key_chunks(d);
  p.r32 = mats.r32;
  p.s32 = mats.s32;
  p.wq = wq;
  p.wqn = wqn;
  // grouped form when there are enough groups to fill the chip; with a few
  // slots (a decode step) one workgroup per head lane has the shorter path
  if (d == 128 && m == 64 && (int64_t)s.n_seq * HG >= 32) {
    hipLaunchKernelGGL(prep_queries128, dim3((unsigned)(s.n_seq * HG)), dim3(512), 0, (hipStream_t)stream, p);
    return hipGetLastError() == hipSuccess ? 0 : TQ_EDEVICE;
  }
  const size_t lds = sizeof(float) * (2 * d + m);
  hipLaunchKernelGGL(gen_prep_queries, dim3((unsigned)(s.n_seq * 16 * HG)), dim3(256), lds, (hipStream_t)stream, p);
  return hipGetLastError() == hipSuccess ? 0 : TQ_EDEVICE;
}

int launch_general_scores(const Matrices& mats, const CodebookDev& cbk, int kbits, int d, int m,
                          const AttnShape& s, const void* key_records, float* scores, void* ws, void* stream) {
  hipStream_t st = (hipStream_t)stream;
  const int HG = head_groups_bucket(s.G);
  if (HG > 32) return TQ_EUNSUPPORTED;
  const size_t q_bytes = (size_t)s.n_seq * HG * (d / 32 + m / 32) * 64 * 8 * 2;
  uint16_t* wq = (uint16_t*)ws;
  float* wqn = (float*)((char*)ws + (q_bytes + 255) / 256 * 256);
  int rc = launch_gen_prep(mats, d, m, s, HG, wq, wqn, stream);
  if (rc) return rc;
  GenScoreArgs a;
  a.rec = (const uint32_t*)key_records;
  a.scores = scores;
  a.wq = wq;
  a.wqn = wqn;
  a.n_tokens = s.n_tokens;
  a.capacity = s.capacity;
  a.n_seq = s.n_seq;
  a.G = s.G;
  a.HG = HG;
  a.d = d;
  a.m = m;
  a.n_oct = key_chunks(d);
  a.rec_words = kbits * d / 32 + m / 32 + 2;
  a.tiles_per_slot = (s.n_tokens + 15) / 16;
  a.kappa = (float)(1.2533141373155002512 / m);  // sqrt(pi/2) / m
  for (int i = 0; i < 4; ++i) { a.tlo[i] = cbk.tlo[i]; a.thi[i] = cbk.thi[i]; }
  // many head groups: the blocked kernel (one tile a wave, 4 groups at a time;
  // of 1-8 tiles and 1-16 groups, measured best on 512 queries x 2M keys)
  constexpr int kBlkTiles = 1, kBlkGroups = 4;
  if (HG >= kBlkGroups) {
    const int64_t waves = (a.tiles_per_slot + kBlkTiles - 1) / kBlkTiles * s.n_seq, chunk = (int64_t)4 << 22;
    for (a.gw0 = 0; a.gw0 < waves; a.gw0 += chunk) {
      const int64_t nw = std::min(chunk, waves - a.gw0);
      const dim3 grid((unsigned)((nw + 3) / 4)), block(256);
#define TQ_GSK(B) \
  if (kbits == B) hipLaunchKernelGGL((gen_scores_blk<B, kBlkTiles, kBlkGroups>), grid, block, 0, st, a);
      TQ_GSK(0) TQ_GSK(1) TQ_GSK(2) TQ_GSK(3) TQ_GSK(4)
#undef TQ_GSK
      if (hipGetLastError() != hipSuccess) return TQ_EDEVICE;
    }
    return 0;
  }
  // one wave per (slot, 16-token tile), in launches of at most 2^22
  // workgroups so that a grid's thread count stays within 32 bits
  const int64_t waves = a.tiles_per_slot * s.n_seq, chunk = (int64_t)4 << 22;
  for (a.gw0 = 0; a.gw0 < waves; a.gw0 += chunk) {
    const int64_t nw = std::min(chunk, waves - a.gw0);
    const dim3 grid((unsigned)((nw + 3) / 4)), block(256);
#define TQ_GS(B, H) \
  if (kbits == B && HG == H) hipLaunchKernelGGL((gen_scores<B, H>), grid, block, 0, st, a);
#define TQ_GSB(B) TQ_GS(B, 1) TQ_GS(B, 2) TQ_GS(B, 4) TQ_GS(B, 8) TQ_GS(B, 16) TQ_GS(B, 32)
    TQ_GSB(0) TQ_GSB(1) TQ_GSB(2) TQ_GSB(3) TQ_GSB(4)
#undef TQ_GSB
#undef TQ_GS
    if (hipGetLastError() != hipSuccess) return TQ_EDEVICE;
  }
  return 0;
}


GenAttnPlan general_attend_plan(int d, int m, int n_seq, int G, int64_t n_tokens) {
  GenAttnPlan p;
  auto up = [](size_t x) { return (x + 255) / 256 * 256; };
  const int HG = head_groups_bucket(G);
  const size_t q_bytes = (size_t)n_seq * HG * (d / 32 + m / 32) * 64 * 8 * 2;
  const size_t qn_bytes = (size_t)n_seq * HG * 16 * 4;
  const int n_oct = key_chunks(d);
  const int64_t nblk = (n_tokens + kBlockTokens - 1) / kBlockTokens;
  int64_t R = (4096 + (int64_t)n_seq * n_oct - 1) / ((int64_t)n_seq * n_oct);  // ~16 waves per CU in all
  if (R > nblk) R = nblk;
  if (R > 1024) R = 1024;
  if (R < 1) R = 1;
  const int64_t bpw = (nblk + R - 1) / R;
  p.blocks_per_wave = (int)bpw;
  p.ranges = (int)((nblk + bpw - 1) / bpw);
  p.off_scores = up(q_bytes) + up(qn_bytes);
  p.off_part = p.off_scores + up((size_t)n_seq * G * n_tokens * 4);
  p.total = p.off_part + up((size_t)n_seq * p.ranges * n_oct * G * kGenPart * 4);
  return p;
}

int launch_general_attend(const Matrices& mats, const CodebookDev& cbk, int kbits, const CodebookDev& cbv, int vbits,
                          int d, int m, const AttnShape& s, const void* key_records, const void* value_blocks,
                          float scale, float* out, void* ws, void* stream) {
  hipStream_t st = (hipStream_t)stream;
  const GenAttnPlan p = general_attend_plan(d, m, s.n_seq, s.G, s.n_tokens);
  float* scores = (float*)((char*)ws + p.off_scores);
  int rc = launch_general_scores(mats, cbk, kbits, d, m, s, key_records, scores, ws, stream);
  if (rc) return rc;
  GenAttendArgs a;
  a.scores = scores;
  a.vblocks = (const uint32_t*)value_blocks;
  a.part = (float*)((char*)ws + p.off_part);
  a.n_tokens = s.n_tokens;
  a.capacity = s.capacity;
  a.n_seq = s.n_seq;
  a.G = s.G;
  a.d = d;
  a.n_oct = key_chunks(d);
  a.block_words = 4 * vbits * d + kBlockTokens;
  a.blocks_per_wave = p.blocks_per_wave;
  a.ranges = p.ranges;
  a.scale2 = scale * 1.4426950408889634f;
  for (int i = 0; i < 4; ++i) { a.vtlo[i] = cbv.tlo[i]; a.vthi[i] = cbv.thi[i]; }
  const int64_t waves = (int64_t)s.n_seq * p.ranges * key_chunks(d);
  const dim3 grid((unsigned)((waves + 3) / 4)), block(256);
  if (vbits == 1) hipLaunchKernelGGL(gen_attend_kernel<1>, grid, block, 0, st, a);
  if (vbits == 2) hipLaunchKernelGGL(gen_attend_kernel<2>, grid, block, 0, st, a);
  if (vbits == 3) hipLaunchKernelGGL(gen_attend_kernel<3>, grid, block, 0, st, a);
  if (vbits == 4) hipLaunchKernelGGL(gen_attend_kernel<4>, grid, block, 0, st, a);
  GenCombineArgs c;
  c.part = a.part;
  c.out = out;
  c.r32 = mats.r32;
  c.n_seq = s.n_seq;
  c.G = s.G;
  c.d = d;
  c.n_oct = key_chunks(d);
  c.ranges = p.ranges;
  hipLaunchKernelGGL(gen_combine, dim3((unsigned)(s.n_seq * s.G)), dim3(256), sizeof(float) * (d + p.ranges), st, c);
  return hipGetLastError() == hipSuccess ? 0 : TQ_EDEVICE;
}

}  // namespace tq
