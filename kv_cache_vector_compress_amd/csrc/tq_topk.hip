// Inner-product top-k over the packed keys, without materialising the scores
// (the vector-search use of the estimator: ai-manual.ru article, where
// TurboQuant pays off / Где TurboQuant выстреливает; jansverre.net post,
// Hvem er dette nyttig for?; the estimate itself as in the score kernels,
// nav.superapi.store "turboquant-pytorch" 常见使用模式).
//
// Pass 1 (topk_scores_kernel): one workgroup of 8 waves per (slot, range of
// 16-token tiles, block of 32 query lanes).  The block's query operands (two
// groups of 16 lanes, laid out by the query prep kernel) sit in LDS; each
// wave decodes a 16-token tile once and multiplies it by both groups, in the
// order of the chunked score kernel, so est = acc ||k|| ||q|| is the value
// tq_attention_scores would write.  Each wave keeps, per query, its best k
// candidates by (score descending, token index ascending) in LDS: a lane
// compares its candidates with the list's k-th entry (one register per
// query), and the rare candidate that beats it is inserted.  Tiles are
// visited in index order and the rows of a tile in (lane group, element)
// order, so a tie with an entry already listed keeps the earlier token.
// Pass 2 (topk_merge_kernel): per query, the k best of all the waves' lists
// in the same order.
#include <algorithm>

#include "tq_device.h"
#include "tq_layout.h"

namespace tq {

constexpr int kTkWaves = 8;

struct TopkArgs {
  const uint32_t* rec;
  const uint16_t* wq;  // [n_seq][HG][KBT][64][8] query operands
  const float* wqn;    // [n_seq][16 HG] query norms
  float* cs;           // candidates [n_seq][G][n_lists][k]
  int32_t* ci;
  int64_t n_tokens, capacity;
  int n_seq, G, HG, d, m, n_oct, rec_words, k, n_qblk, n_ranges;
  int64_t tiles_per_range, range_stride;  // range r: tiles [r range_stride, + tiles_per_range)
  const float* tau;  // nullable: [n_seq][G][k] a sample's top-k scores; its k-th entry starts the threshold
  float kappa;
  uint32_t tlo[4], thi[4];
};

// (s, i) ranks before (s2, i2): higher score, then lower index.
__device__ __forceinline__ bool tk_before(float s, int i, float s2, int i2) {
  return s > s2 || (s == s2 && i < i2);
}

// Insert (s, i) into a list of k entries sorted by tk_before (k-th = worst).
__device__ __forceinline__ void tk_insert(float* ls, int32_t* li, int k, float s, int i) {
  if (!tk_before(s, i, ls[k - 1], li[k - 1])) return;
  int p = k - 1;
  while (p > 0 && tk_before(s, i, ls[p - 1], li[p - 1])) {
    ls[p] = ls[p - 1];
    li[p] = li[p - 1];
    --p;
  }
  ls[p] = s;
  li[p] = i;
}

// A lane's words of one 16-token tile: code group (B words) of each of the
// NOCT full coordinate chunks and, with HALF, of the half chunk (already
// moved to slots 0..3), 8 sign words (one per 64 projections, a half block
// counting as one), ||k|| and gamma.
// Every word is loaded unconditionally (unused sign words read neighbouring
// record bytes, or zeros past the range's records), so the loads of the next
// tile can be counted exactly and stay in flight while the current tile is
// processed.
template <int B, int NOCT, bool HALF>
struct TkRec {
  static constexpr int NC = NOCT + (HALF ? 1 : 0);
  uint32_t cw[NC > 0 ? NC : 1][B > 0 ? B : 1];  // (0-bit keys: no code words, unused)
  uint32_t sw[8];
  float n, g;
};

template <int B, int NOCT, bool HALF>
__global__ __launch_bounds__(512) void topk_scores_kernel(const TopkArgs a) {
  extern __shared__ __align__(16) uint16_t tsm[];
  const int KBT = a.d / 32 + a.m / 32;
  uint16_t* qop = tsm;                                      // [2][KBT][64][8]
  float* ls = (float*)(tsm + 2 * KBT * 512);                // [waves][32][k]
  int32_t* li = (int32_t*)(ls + kTkWaves * 32 * a.k);
  float* thr_wg = (float*)(li + kTkWaves * 32 * a.k);  // [32]: the best k-th score of any wave's list
  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int r16 = lane & 15, q = lane >> 4;
  const int qblk = blockIdx.x % a.n_qblk;
  const int sr = blockIdx.x / a.n_qblk;
  const int range = sr % a.n_ranges, slot = sr / a.n_ranges;
  const int ng = min(2, a.HG - 2 * qblk);  // query groups of this block
  {
    const u4* src = (const u4*)(a.wq + ((int64_t)slot * a.HG + 2 * qblk) * KBT * 512);
    for (int i = tid; i < ng * KBT * 64; i += blockDim.x) ((u4*)qop)[i] = src[i];
    for (int i = tid; i < kTkWaves * 32 * a.k; i += blockDim.x) {
      ls[i] = -INFINITY;
      li[i] = -1;
    }
    if (tid < 32) {
      // a sample's k-th best score: k tokens reach it, so no token below it
      // is in the top k
      const int h = 32 * qblk + tid;
      thr_wg[tid] = a.tau && h < a.G ? a.tau[((int64_t)slot * a.G + h) * a.k + a.k - 1] : -INFINITY;
    }
  }
  __syncthreads();

  float qn[2], thr[2];
  bool live[2];
#pragma unroll
  for (int g = 0; g < 2; ++g) {
    const int h = 32 * qblk + 16 * g + r16;
    live[g] = g < ng && h < a.G;
    qn[g] = g < ng ? a.wqn[((int64_t)slot * a.HG + 2 * qblk + g) * 16 + r16] : 0.f;
    thr[g] = -INFINITY;
  }
  uint32_t tlo[4], thi[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) { tlo[i] = a.tlo[i]; thi[i] = a.thi[i]; }
  const int n_tok = (int)a.n_tokens;
  const int64_t ntile = (a.n_tokens + 15) / 16;
  const int64_t t_lo = (int64_t)range * a.range_stride;
  const int64_t t_hi = min(ntile, t_lo + a.tiles_per_range);
  const int sh0 = 15 - 8 * (q & 1);
  const int sw0 = B * a.d / 32;
  float* wls = ls + wave * 32 * a.k;
  int32_t* wli = li + wave * 32 * a.k;

  // this range's records as a buffer (the plan keeps a range's records
  // under 2^31 bytes, so 32-bit offsets reach them at any capacity); a
  // lane's words of one tile (its code group of every chunk, its sign words,
  // the two norms) are loaded one tile ahead of their use
  const int64_t r0 = t_lo * 16, r1 = min(a.capacity, t_hi * 16);
  const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint32_t*>(a.rec + ((int64_t)slot * a.capacity + r0) * a.rec_words), (short)0,
      (int)((uint32_t)(r1 - r0) * (uint32_t)a.rec_words * 4u), 0x00020000);
  auto load_tile = [&](TkRec<B, NOCT, HALF>& r, int64_t tile) {
    const int row = min((int)(tile * 16) + r16, n_tok - 1);
    const uint32_t ro = (uint32_t)(row - (int)r0) * (uint32_t)a.rec_words * 4u;
#pragma unroll
    for (int c = 0; c < (B > 0 ? TkRec<B, NOCT, HALF>::NC : 0); ++c) {
      const uint32_t oc = ro + 4u * (uint32_t)(B > 0 ? key_group_word(q, c, NOCT, B) : 0);
      if constexpr (B == 0) {
        (void)oc;
      } else if constexpr (B == 1) {
        r.cw[c][0] = __builtin_amdgcn_raw_buffer_load_b32(rs, oc, 0, 0);
      } else if constexpr (B == 2) {
        const auto v = __builtin_amdgcn_raw_buffer_load_b64(rs, oc, 0, 0);
        r.cw[c][0] = v[0]; r.cw[c][1] = v[1];
      } else if constexpr (B == 3) {
        const auto v = __builtin_amdgcn_raw_buffer_load_b96(rs, oc, 0, 0);
        r.cw[c][0] = v[0]; r.cw[c][1] = v[1]; r.cw[c][2] = v[2];
      } else {
        const auto v = __builtin_amdgcn_raw_buffer_load_b128(rs, oc, 0, 0);
        r.cw[c][0] = v[0]; r.cw[c][1] = v[1]; r.cw[c][2] = v[2]; r.cw[c][3] = v[3];
      }
    }
    if constexpr (HALF && B > 0) {  // the half chunk's group, at slots 0..3 for every lane group
      uint32_t cl[B];
#pragma unroll
      for (int w = 0; w < B; ++w) cl[w] = r.cw[NOCT][w];
      lower_half<B>(cl);
#pragma unroll
      for (int w = 0; w < B; ++w) r.cw[NOCT][w] = q >= 2 ? cl[w] : r.cw[NOCT][w];
    }
    // (a half sign block is a single word shared by the four lane groups)
#pragma unroll
    for (int j = 0; j < 8; ++j)
      r.sw[j] = __builtin_amdgcn_raw_buffer_load_b32(
          rs, ro + 4u * (uint32_t)(sw0 + 2 * j + (2 * j + 2 <= a.m / 32 ? (q >> 1) : 0)), 0, 0);
    const auto ng2 = __builtin_amdgcn_raw_buffer_load_b64(rs, ro + 4u * (uint32_t)(a.rec_words - 2), 0, 0);
    r.n = __uint_as_float(ng2[0]);
    r.g = __uint_as_float(ng2[1]);
  };

  auto step = [&](const TkRec<B, NOCT, HALF>& r, int64_t tile) {
    f4 acc[2];
    acc[0] = acc[1] = f4{0.f, 0.f, 0.f, 0.f};
    // per chunk: the 4 query operands of each group are read from LDS first,
    // so their latency overlaps the decode, then the 4 (8) products
    const uint16_t* ql = qop + lane * 8;
    // (with a single group the second products use LDS never written and
    // are not read)
    if constexpr (B > 0) {  // (0-bit keys: the centroid 0 adds nothing)
#pragma unroll
      for (int c = 0; c < NOCT; ++c) {
        h8 qa[2][4];
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
          qa[0][kk] = *(const h8*)(ql + (4 * c + kk) * 512);
          qa[1][kk] = *(const h8*)(ql + (KBT + 4 * c + kk) * 512);
        }
        const h8 A0 = decode_pair<B, 0>(r.cw[c], tlo, thi), A1 = decode_pair<B, 2>(r.cw[c], tlo, thi);
        const h8 A2 = decode_pair<B, 4>(r.cw[c], tlo, thi), A3 = decode_pair<B, 6>(r.cw[c], tlo, thi);
        acc[0] = mfma(A0, qa[0][0], acc[0]);
        acc[1] = mfma(A0, qa[1][0], acc[1]);
        acc[0] = mfma(A1, qa[0][1], acc[0]);
        acc[1] = mfma(A1, qa[1][1], acc[1]);
        acc[0] = mfma(A2, qa[0][2], acc[0]);
        acc[1] = mfma(A2, qa[1][2], acc[1]);
        acc[0] = mfma(A3, qa[0][3], acc[0]);
        acc[1] = mfma(A3, qa[1][3], acc[1]);
      }
      if constexpr (HALF) {  // the half chunk: K blocks 4 NOCT and 4 NOCT + 1
        h8 qa[2][2];
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
          qa[0][kk] = *(const h8*)(ql + (4 * NOCT + kk) * 512);
          qa[1][kk] = *(const h8*)(ql + (KBT + 4 * NOCT + kk) * 512);
        }
        const h8 A0 = decode_pair<B, 0>(r.cw[NOCT], tlo, thi), A1 = decode_pair<B, 2>(r.cw[NOCT], tlo, thi);
        acc[0] = mfma(A0, qa[0][0], acc[0]);
        acc[1] = mfma(A0, qa[1][0], acc[1]);
        acc[0] = mfma(A1, qa[0][1], acc[0]);
        acc[1] = mfma(A1, qa[1][1], acc[1]);
      }
    }
    const _Float16 gk = (_Float16)(r.g * a.kappa);
    const uint32_t gk2 = (uint32_t)__builtin_bit_cast(uint16_t, gk) * 0x00010001u;
    const int n_kbp = a.m / 32;
    const uint16_t* qs = ql + (a.d / 32) * 512;
#pragma unroll
    for (int k2 = 0; k2 < 16; k2 += 2) {  // the 2 sign steps of one sign word pair at a time
      if (k2 >= n_kbp) break;
      // a half block (the last of m = 64 n' + 32) has one step, its word in
      // projection order: lane group q takes bits 4 q + e and 16 + 4 q + e
      const bool hb = k2 + 1 >= n_kbp;
      h8 qa[2][2];
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
        const int kq = hb ? k2 : k2 + kk;
        qa[0][kk] = *(const h8*)(qs + kq * 512);
        qa[1][kk] = *(const h8*)(qs + (KBT + kq) * 512);
      }
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
        if (kk == 1 && hb) break;
        const int kbp = k2 + kk;
        const uint32_t w = ~r.sw[kbp / 2];
        const int sh1 = hb ? 15 - 4 * q : sh0 - 4 * (kbp % 2);
        u4 v;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const uint32_t sh = w << (sh1 - e);  // bits p, p+16 -> 15, 31
          v[e] = (sh & 0x80008000u) | (gk2 & 0x7FFF7FFFu);
        }
        const h8 A = as_h8(v);
        acc[0] = mfma(A, qa[0][kk], acc[0]);
        acc[1] = mfma(A, qa[1][kk], acc[1]);
      }
    }
    // acc[g][i]: token row 4q+i of the tile, query lane 16 g + r16
    const float kn = r.n;
    f4 nk;
#pragma unroll
    for (int i = 0; i < 4; ++i) nk[i] = __shfl(kn, 4 * q + i, 64);
    const int t0 = (int)(tile * 16) + 4 * q;
#pragma unroll
    for (int g = 0; g < 2; ++g) {
      if (g >= ng) break;
      // A candidate must beat this wave's own k-th entry and reach the best
      // k-th entry of any wave of the workgroup (or the sample's k-th best
      // score it started from): k tokens rank at least as high as that one,
      // so a token below it is in no top k (one equal to it may still rank
      // before by its index, so it goes on to the list).
      const float thw = thr_wg[16 * g + r16];
      float est[4];
      bool pass[4], any = false;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        est[i] = acc[g][i] * nk[i] * qn[g];
        pass[i] = live[g] && t0 + i < n_tok && est[i] > thr[g] && est[i] >= thw;
        any |= pass[i];
      }
      if (__any(any)) {  // rare once the lists are full
        float* cls = wls + (16 * g + r16) * a.k;
        int32_t* cli = wli + (16 * g + r16) * a.k;
        // one (lane group, row) at a time: at most one insertion per list per step
        for (int qq = 0; qq < 4; ++qq)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const bool me = q == qq && pass[i];
            if (__any(me)) {
              if (me) tk_insert(cls, cli, a.k, est[i], t0 + i);
              __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
            }
          }
        thr[g] = cls[a.k - 1];
        if (q == 0 && thr[g] != -INFINITY)
          (void)__hip_atomic_fetch_max(thr_wg + 16 * g + r16, thr[g], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
      }
    }
  };

  TkRec<B, NOCT, HALF> ra, rb;
  int64_t tile = t_lo + wave;
  if (tile < t_hi) load_tile(ra, tile);
  for (; tile < t_hi; tile += 2 * kTkWaves) {
    if (tile + kTkWaves < t_hi) load_tile(rb, tile + kTkWaves);
    step(ra, tile);
    if (tile + kTkWaves >= t_hi) break;
    if (tile + 2 * kTkWaves < t_hi) load_tile(ra, tile + 2 * kTkWaves);
    step(rb, tile + kTkWaves);
  }

  // this wave's lists -> candidates [slot][h][list][k]
  const int n_lists = a.n_ranges * kTkWaves, list = range * kTkWaves + wave;
#pragma unroll
  for (int g = 0; g < 2; ++g) {
    if (g >= ng) break;
    const int h = 32 * qblk + 16 * g + r16;
    if (!live[g]) continue;
    const int64_t o = (((int64_t)slot * a.G + h) * n_lists + list) * a.k;
    for (int j = q; j < a.k; j += 4) {
      a.cs[o + j] = wls[(16 * g + r16) * a.k + j];
      a.ci[o + j] = wli[(16 * g + r16) * a.k + j];
    }
  }
}

// Pass 2: one workgroup per (slot, query): the k best of its n_lists x k
// candidates, k rounds of a block-wide arg-best.
struct TopkMergeArgs {
  const float* cs;
  const int32_t* ci;
  float* out_s;    // [n_seq][G][k]
  int32_t* out_i;
  int n_cand, k;
};

__global__ __launch_bounds__(256) void topk_merge_kernel(const TopkMergeArgs a) {
  __shared__ float bs[8];    // [0]: the last winner; [4 + w]: wave w's pick
  __shared__ int32_t bi[8];
  __shared__ int32_t bw[8];  // position in the candidate array (-1: none)
  const int64_t sq = blockIdx.x;
  const float* cs = a.cs + sq * a.n_cand;
  const int32_t* ci = a.ci + sq * a.n_cand;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  for (int r = 0; r < a.k; ++r) {
    // this thread's best remaining candidate (candidates already output are
    // those ranking before the previous winner, or equal to it)
    float s = -INFINITY;
    int i = 0x7FFFFFFF, p = -1;
    for (int c = tid; c < a.n_cand; c += blockDim.x) {
      const float cs_ = cs[c];
      const int ci_ = ci[c];
      if (ci_ < 0) continue;
      if (r > 0 && !tk_before(bs[0], bi[0], cs_, ci_)) continue;  // not after the previous winner
      if (p < 0 || tk_before(cs_, ci_, s, i)) { s = cs_; i = ci_; p = c; }
    }
    // wave then block arg-best
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
      const float s2 = __shfl_xor(s, o, 64);
      const int i2 = __shfl_xor(i, o, 64), p2 = __shfl_xor(p, o, 64);
      if (p2 >= 0 && (p < 0 || tk_before(s2, i2, s, i))) { s = s2; i = i2; p = p2; }
    }
    __syncthreads();  // everyone is done reading the previous winner
    if (lane == 0) { bs[4 + wave] = s; bi[4 + wave] = i; bw[4 + wave] = p; }
    __syncthreads();
    if (tid == 0) {
      float S = -INFINITY;
      int I = 0x7FFFFFFF, P = -1;
      for (int w = 0; w < 4; ++w)
        if (bw[4 + w] >= 0 && (P < 0 || tk_before(bs[4 + w], bi[4 + w], S, I))) { S = bs[4 + w]; I = bi[4 + w]; P = bw[4 + w]; }
      bs[0] = S;
      bi[0] = I;
      bw[0] = P;
      a.out_s[sq * a.k + r] = P >= 0 ? S : -INFINITY;
      a.out_i[sq * a.k + r] = P >= 0 ? I : -1;
    }
    __syncthreads();
    if (bw[0] < 0) {  // fewer than k candidates: the rest stay empty
      for (int j = r + 1 + tid; j < a.k; j += blockDim.x) {
        a.out_s[sq * a.k + j] = -INFINITY;
        a.out_i[sq * a.k + j] = -1;
      }
      break;
    }
  }
}

// ---- plan and launch ----------------------------------------------------------

TopkPlan topk_plan(int d, int m, int n_seq, int G, int64_t n_tokens, int k) {
  TopkPlan p;
  auto up = [](size_t x) { return (x + 255) / 256 * 256; };
  p.HG = (G + 15) / 16;
  p.n_qblk = (p.HG + 1) / 2;
  const int64_t ntile = (n_tokens + 15) / 16;
  // about 1024 workgroups over the grid (a fixed count, so that the
  // workspace size does not depend on the device), each wave >= 1 tile
  int64_t R = (1024 + (int64_t)n_seq * p.n_qblk - 1) / ((int64_t)n_seq * p.n_qblk);
  R = std::min<int64_t>(R, (ntile + kTkWaves - 1) / kTkWaves);
  R = std::max<int64_t>(1, std::min<int64_t>(R, 256));
  // a range's records (4-bit codes at most) stay under 2^31 bytes: the
  // kernel addresses them with 32-bit offsets
  const int64_t rec_max = 4 * (4 * (int64_t)d / 32 + m / 32 + 2);
  const int64_t max_tiles = ((int64_t)1 << 31) / (16 * rec_max) - 1;
  R = std::max<int64_t>(R, (ntile + max_tiles - 1) / max_tiles);
  p.tiles_per_range = (ntile + R - 1) / R;
  p.n_ranges = (int)((ntile + p.tiles_per_range - 1) / p.tiles_per_range);
  p.n_lists = p.n_ranges * kTkWaves;
  const size_t KBT = (size_t)(d / 32 + m / 32);
  p.q_bytes = up((size_t)n_seq * p.HG * KBT * 64 * 8 * 2);
  p.qn_bytes = up((size_t)n_seq * p.HG * 16 * 4);
  p.cand_bytes = up((size_t)n_seq * G * p.n_lists * k * 4);
  p.total = p.q_bytes + p.qn_bytes + 2 * p.cand_bytes;
  return p;
}

static size_t topk_lds(int d, int m, int k) {
  return (size_t)2 * (d / 32 + m / 32) * 512 * 2 + (size_t)kTkWaves * 32 * k * 8 + 32 * 4;
}

int topk_device_init() {
  int rc = 0;
  const int lds = (int)topk_lds(1024, 512, kTopkMax);
#define TQ_TK_ATTR(B, N, H) \
  rc |= hipFuncSetAttribute((const void*)topk_scores_kernel<B, N, H>, hipFuncAttributeMaxDynamicSharedMemorySize, lds);
#define TQ_TK_ATTR_B(B) \
  TQ_TK_ATTR(B, 1, false) TQ_TK_ATTR(B, 2, false) TQ_TK_ATTR(B, 3, false) TQ_TK_ATTR(B, 4, false)            \
  TQ_TK_ATTR(B, 5, false) TQ_TK_ATTR(B, 6, false) TQ_TK_ATTR(B, 7, false) TQ_TK_ATTR(B, 8, false)            \
  TQ_TK_ATTR(B, 0, true) TQ_TK_ATTR(B, 1, true) TQ_TK_ATTR(B, 2, true) TQ_TK_ATTR(B, 3, true)                \
  TQ_TK_ATTR(B, 4, true) TQ_TK_ATTR(B, 5, true) TQ_TK_ATTR(B, 6, true) TQ_TK_ATTR(B, 7, true)
  TQ_TK_ATTR_B(1) TQ_TK_ATTR_B(2) TQ_TK_ATTR_B(3) TQ_TK_ATTR_B(4)
  TQ_TK_ATTR(0, 1, false)
#undef TQ_TK_ATTR_B
#undef TQ_TK_ATTR
  return rc == hipSuccess ? 0 : -1;
}

int launch_topk(const Matrices& mats, const CodebookDev& cbk, int kbits, int d, int m, const AttnShape& s, int k,
                const void* key_records, float* top_s, int32_t* top_i, void* ws, void* stream) {
  hipStream_t st = (hipStream_t)stream;
  const TopkPlan p = topk_plan(d, m, s.n_seq, s.G, s.n_tokens, k);
  char* w = (char*)ws;
  uint16_t* wq = (uint16_t*)w;
  float* wqn = (float*)(w + p.q_bytes);
  float* cs = (float*)(w + p.q_bytes + p.qn_bytes);
  int32_t* ci = (int32_t*)(w + p.q_bytes + p.qn_bytes + p.cand_bytes);
  int rc = launch_gen_prep(mats, d, m, s, p.HG, wq, wqn, stream);
  if (rc) return rc;
  TopkArgs a;
  a.rec = (const uint32_t*)key_records;
  a.wq = wq;
  a.wqn = wqn;
  a.cs = cs;
  a.ci = ci;
  a.n_tokens = s.n_tokens;
  a.capacity = s.capacity;
  a.n_seq = s.n_seq;
  a.G = s.G;
  a.HG = p.HG;
  a.d = d;
  a.m = m;
  a.n_oct = key_chunks(d);
  a.rec_words = kbits * d / 32 + m / 32 + 2;
  a.k = k;
  a.n_qblk = p.n_qblk;
  a.n_ranges = p.n_ranges;
  a.tiles_per_range = p.tiles_per_range;
  a.range_stride = p.tiles_per_range;
  a.tau = nullptr;
  a.kappa = (float)(1.2533141373155002512 / m);  // sqrt(pi/2) / m
  for (int i = 0; i < 4; ++i) { a.tlo[i] = cbk.tlo[i]; a.thi[i] = cbk.thi[i]; }
  const dim3 grid((unsigned)((int64_t)s.n_seq * p.n_ranges * p.n_qblk)), block(64 * kTkWaves);
  const size_t lds = topk_lds(d, m, k);
  const int n_full = d / 128;
  const bool half = d % 128 != 0;
  auto search = [&](const TopkArgs& x) -> int {
    bool launched = false;
#define TQ_TK(B, N, H) \
  if (!launched && kbits == B && n_full == N && half == H) { \
    hipLaunchKernelGGL((topk_scores_kernel<B, N, H>), grid, block, lds, st, x); \
    launched = true; \
  }
#define TQ_TK_B(B)                                                                                   \
  TQ_TK(B, 1, false) TQ_TK(B, 2, false) TQ_TK(B, 3, false) TQ_TK(B, 4, false) TQ_TK(B, 5, false)     \
  TQ_TK(B, 6, false) TQ_TK(B, 7, false) TQ_TK(B, 8, false) TQ_TK(B, 0, true) TQ_TK(B, 1, true)       \
  TQ_TK(B, 2, true) TQ_TK(B, 3, true) TQ_TK(B, 4, true) TQ_TK(B, 5, true) TQ_TK(B, 6, true)          \
  TQ_TK(B, 7, true)
    if (kbits == 0) {  // 0-bit keys: no code chunks, one instance for every head_dim
      hipLaunchKernelGGL((topk_scores_kernel<0, 1, false>), grid, block, lds, st, x);
      launched = true;
    }
    TQ_TK_B(1) TQ_TK_B(2) TQ_TK_B(3) TQ_TK_B(4)
#undef TQ_TK_B
#undef TQ_TK
    if (!launched) return TQ_EUNSUPPORTED;
    if (hipGetLastError() != hipSuccess) return TQ_EDEVICE;
    TopkMergeArgs b;
    b.cs = cs;
    b.ci = ci;
    b.out_s = top_s;
    b.out_i = top_i;
    b.n_cand = p.n_lists * k;
    b.k = k;
    hipLaunchKernelGGL(topk_merge_kernel, dim3((unsigned)(s.n_seq * s.G)), dim3(256), 0, st, b);
    return hipGetLastError() == hipSuccess ? 0 : TQ_EDEVICE;
  };
  // A sample first, when the ranges are long: the first 32 tiles of every
  // range's stretch of the token axis (4 tiles per wave), spread over the
  // whole axis, searched the same way into the outputs.  Its k-th best score
  // per query is reached by k tokens, so the full search starts every
  // workgroup's threshold there: only tokens at or above it become
  // candidates, and the lists are not filled from -inf.
  if (p.tiles_per_range >= 8 * 4 * kTkWaves) {  // (the sample is at most 1/8 of the work)
    TopkArgs smp = a;
    smp.tiles_per_range = 4 * kTkWaves;  // range r: tiles [r range_stride, + 32), clipped to the axis
    const int rc = search(smp);
    if (rc) return rc;
    a.tau = top_s;
  }
  return search(a);
}

}  // namespace tq
