// Attention over the packed cache on gfx950, head_dim 128.
//
// Scores (asymmetric_attention_scores, nav.superapi.store "turboquant-pytorch"
// 常见使用模式; the QJL stage makes the inner-product estimate unbiased,
// atskills.one Stage 2):
//     est = ||k|| ( <q~, c[idx]> + gamma sqrt(pi/2)/m <p, 2s-1> ),
//     q~ = R q, p = S q~.
// Both inner products run on the matrix cores in one accumulator: the packed
// key is decoded into an fp16 operand (centroids c[idx] for the first part,
// +-gamma sqrt(pi/2)/m for the second) and multiplied by the prepared query
// operand (q~ and p in fp16, scaled to unit query norm).  Decoding is byte
// permutes from an 8/16-entry fp16 table held in registers.
//
// Attend (常见使用模式: softmax of the scores, then the weighted sum of the
// decompressed values; values are stage-1 only, 算法细节): each wave streams a
// range of 128-token blocks, keeps a running max / sum / accumulator per
// query head (online softmax), and accumulates sum_t p_t ||v_t|| c[idx_t] in
// the rotated domain with the matrix cores.  A second kernel merges the
// per-wave partials (log-sum-exp) and applies R^T once per query head.
#include <algorithm>
#include <atomic>
#include <chrono>
#include <mutex>
#include <random>
#include <type_traits>

#include "tq_device.h"
#include "tq_small.h"

namespace tq {

constexpr int kPartFloats = 4 + kD;  // m, l, ve, pad, acc[d]
constexpr int kSyncWords = 40;       // fused decode step, per slot: producer flags (<= 16 + 2 + 16 = 34), done count
constexpr float kLog2e = 1.4426950408889634f;
// Waves over the whole grid, fixed so that the workspace size does not
// depend on the device.  The attend kernel holds ~230 VGPRs, so a SIMD runs
// two of its waves: 2048 waves are one resident round of a 256-CU MI355X,
// and each wave's fixed costs (tables, query operands, partials) are paid
// once.  The score kernel runs short waves of 8 tiles (16 tokens each)
// while there are at least 4096 of them, up to 65536 waves: on the
// long-context cache (524288 tiles) 4096 waves took 0.159 ms, 16384 0.141,
// 65536 0.132 and 131072 0.139; with fewer tiles, one-tile waves pay their
// fixed costs for too little work (the 36 layers of a decode step, 36864
// tiles: 0.029 ms at 9 tiles a wave, 0.047 ms at 1).
constexpr int64_t kAttendWaves = 256 * 8;
constexpr int64_t kScoreWavesMin = 256 * 16, kScoreWavesMax = 256 * 256, kScoreTilesPerWave = 8;
constexpr int kMaxPartials = 1024;

// ---------------------------------------------------------------------------
// shared pieces of the score computation
// ---------------------------------------------------------------------------

template <int B, int M>
struct KeyTile {
  uint32_t cw[B > 0 ? B : 1];  // (0-bit keys: no code words, unused)
  uint32_t sw[M / 64];
  float n, g;
};

// Raw buffer resource over one slot's region of the cache: dword loads with
// 32-bit byte offsets (no 64-bit address arithmetic per lane), reads past
// `bytes` return 0.  Word 3 selects the 32-bit data format.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t slot_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}

__device__ __forceinline__ uint32_t bld(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0);
}

// The words of one key record this lane needs (record at byte offset `ro`).
template <int B, int M>
__device__ __forceinline__ void load_key(KeyTile<B, M>& k, __amdgpu_buffer_rsrc_t r, uint32_t ro, int q) {
  constexpr int RW = B * kD / 32 + M / 32 + 2;
  const uint32_t oc = ro + 4u * (uint32_t)(q * B), os = ro + 4u * (uint32_t)(4 * B + (q >> 1));
#pragma unroll
  for (int w = 0; w < B; ++w) k.cw[w] = bld(r, oc + 4u * w);
#pragma unroll
  for (int c = 0; c < M / 64; ++c) k.sw[c] = bld(r, os + 8u * c);
  k.n = __uint_as_float(bld(r, ro + 4u * (RW - 2)));
  k.g = __uint_as_float(bld(r, ro + 4u * (RW - 1)));
}

// acc[i] = (unscaled, unnormalised) score of token row 4q+i of the tile for
// query head (lane % 16).  est = acc * ||k|| * ||q||.  With PT (3-bit keys)
// the centroids come from the LDS pair tables and qb[0..3] must be in pair
// order (to_pair_order).
template <int B, int M, bool PT = false>
__device__ __forceinline__ f4 key_tile_scores(const KeyTile<B, M>& k, const h8 (&qb)[4 + M / 32],
                                              const uint32_t (&tlo)[4], const uint32_t (&thi)[4], float kappa,
                                              int sh0, const PairTables* pt = nullptr) {
  f4 acc = {0.f, 0.f, 0.f, 0.f};
  if constexpr (B == 0) {
    // 0-bit keys: the single centroid 0 adds nothing
  } else if constexpr (PT) {
    static_assert(B == 3, "pair tables hold 3-bit codes");
    acc = mfma(decode_pair_lds<0>(k.cw, *pt), qb[0], acc);
    acc = mfma(decode_pair_lds<1>(k.cw, *pt), qb[1], acc);
    acc = mfma(decode_pair_lds<2>(k.cw, *pt), qb[2], acc);
    acc = mfma(decode_pair_lds<3>(k.cw, *pt), qb[3], acc);
  } else {
    acc = mfma(decode_pair<B, 0>(k.cw, tlo, thi), qb[0], acc);
    acc = mfma(decode_pair<B, 2>(k.cw, tlo, thi), qb[1], acc);
    acc = mfma(decode_pair<B, 4>(k.cw, tlo, thi), qb[2], acc);
    acc = mfma(decode_pair<B, 6>(k.cw, tlo, thi), qb[3], acc);
  }
  const _Float16 gk = (_Float16)(k.g * kappa);
  const uint32_t gk2 = (uint32_t)__builtin_bit_cast(uint16_t, gk) * 0x00010001u;
#pragma unroll
  for (int kbp = 0; kbp < M / 32; ++kbp) {
    const uint32_t w = ~k.sw[kbp / 2];
    u4 v;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const uint32_t sh = w << (sh0 - 4 * (kbp % 2) - e);  // bits p, p+16 -> 15, 31
      v[e] = (sh & 0x80008000u) | (gk2 & 0x7FFF7FFFu);
    }
    acc = mfma(as_h8(v), qb[4 + kbp], acc);
  }
  return acc;
}

// ---------------------------------------------------------------------------
// scores
// ---------------------------------------------------------------------------

struct ScoreArgs {
  const uint32_t* rec;
  float* scores;
  const uint16_t* wq;
  const float* wqn;
  int64_t n_tokens, capacity;
  int n_seq, G, rec_words;
  int tiles_per_wave, waves_per_slot;
  float kappa;
  uint32_t tlo[4], thi[4];
};

template <int B, int M>
constexpr int rec_words() { return B * kD / 32 + M / 32 + 2; }

__device__ __forceinline__ uint32_t pack_h2(float a, float b) {
  typedef _Float16 h2 __attribute__((ext_vector_type(2)));
  const h2 v = {(_Float16)a, (_Float16)b};  // v_cvt_pk_f16_f32 (round to nearest)
  return __builtin_bit_cast(uint32_t, v);
}

// Stage 16 U tokens of key records (one contiguous run of the cache) in this
// wave's LDS slice: the wave loads them with 16-byte loads, lane l taking
// bytes 16 l + 1024 j, so every load is fully coalesced; lanes then pick
// their words from LDS.  (A lane needs three or four scattered words of one
// record; loading those straight from memory reaches only about 60% of the
// read bandwidth a coalesced stream gets.)  In LDS a record takes STR >= RW
// words with STR/2 odd: the 16 records a read instruction touches then sit
// in distinct banks (word offsets 2 (STR/2) r mod 32 are distinct even
// numbers for r < 16).
template <int RW, int U>
struct KeyStage {
  static constexpr int TW = 16 * RW;                      // words per 16-token tile
  static constexpr int NL = (U * TW + 255) / 256;         // 16-byte loads per lane
  static constexpr int STR = ((RW + 2) / 2) % 2 ? RW + 2 : RW + 4;
  static constexpr int ROWS = (NL * 256 + RW - 1) / RW;   // records a stage covers
  static constexpr int SLICE = ROWS * STR;                // LDS words per wave
  u4 v[NL];
};

// Cache policy of the score kernel's record loads and score stores: each
// byte is touched once, and nontemporal accesses measured a few percent
// faster on this stream (the attend kernel, whose lanes read scattered words
// of lines other lanes also read, keeps the default policy).
constexpr int kNonTemporal = 2;

template <int RW, int U>
__device__ __forceinline__ void stage_load(KeyStage<RW, U>& s, __amdgpu_buffer_rsrc_t r, int tile, int lane) {
  const uint32_t o = (uint32_t)tile * (uint32_t)(KeyStage<RW, U>::TW * 4) + 16u * (uint32_t)lane;
#pragma unroll
  for (int j = 0; j < KeyStage<RW, U>::NL; ++j)
    s.v[j] = __builtin_amdgcn_raw_buffer_load_b128(r, o + 1024u * j, 0, kNonTemporal);
}

// Write the staged registers to the wave's LDS slice, one 8-byte store per
// word pair (RW is even, so a pair never straddles two records).  The fences
// keep the compiler from moving this wave's LDS reads of the previous
// contents past the writes, or its reads of the new contents before them (a
// wave's LDS operations complete in order, so lanes need no wait).
template <int RW, int U>
__device__ __forceinline__ void stage_store(uint32_t* slice, const KeyStage<RW, U>& s, int lane) {
  using S = KeyStage<RW, U>;
  static_assert(RW % 2 == 0, "records are whole word pairs");
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
#pragma unroll
  for (int j = 0; j < S::NL; ++j)
#pragma unroll
    for (int p = 0; p < 2; ++p) {
      const int g = 256 * j + 4 * lane + 2 * p;  // word index within the stage
      const int row = g / RW;
      *(uint2*)(slice + row * S::STR + (g - row * RW)) = make_uint2(s.v[j][2 * p], s.v[j][2 * p + 1]);
    }
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// The words of the staged record of token row t this lane needs.
template <int B, int M, int STR>
__device__ __forceinline__ void stage_key(KeyTile<B, M>& k, const uint32_t* slice, int t, int q) {
  constexpr int RW = B * kD / 32 + M / 32 + 2;
  const uint32_t* rp = slice + t * STR;
#pragma unroll
  for (int w = 0; w < B; ++w) k.cw[w] = rp[q * B + w];
#pragma unroll
  for (int c = 0; c < M / 64; ++c) k.sw[c] = rp[4 * B + 2 * c + (q >> 1)];
  const uint2 ng = *(const uint2*)(rp + RW - 2);
  k.n = __uint_as_float(ng.x);
  k.g = __uint_as_float(ng.y);
}

template <int B, int M>
__global__ __launch_bounds__(256) void scores_kernel(const ScoreArgs a) {
  constexpr int KBT = 4 + M / 32;
  constexpr int RW = rec_words<B, M>();
  constexpr int U = 4;          // 16-token tiles per iteration (the next U tiles in flight)
  using Stage = KeyStage<RW, U>;
  __shared__ __align__(16) uint32_t kst[4][Stage::SLICE];  // per wave: the iteration's records
  __shared__ float nsh[4][16 * U];  // per wave: ||k|| of the iteration's tokens
  // (byte-permute decoding: the LDS pair tables of the attend kernel add a
  // second dependent LDS round trip after the staged record here and
  // measured slower)
  uint32_t tlo[4], thi[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) { tlo[i] = a.tlo[i]; thi[i] = a.thi[i]; }
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int r16 = lane & 15, q = lane >> 4;
  const int64_t gw = (int64_t)blockIdx.x * (blockDim.x >> 6) + wave;
  const int slot = (int)(gw / a.waves_per_slot);
  if (slot >= a.n_seq) return;
  const int wc = (int)(gw - (int64_t)slot * a.waves_per_slot);
  h8 qb[KBT];
#pragma unroll
  for (int kb = 0; kb < KBT; ++kb) qb[kb] = *(const h8*)(a.wq + (((int64_t)slot * KBT + kb) * 64 + lane) * 8);
  const float qn = a.wqn[slot * 16 + r16];
  const int sh0 = 15 - 8 * (q & 1);
  const int n_tok = (int)a.n_tokens;
  const int ntile = (n_tok + 15) >> 4;
  const int t_begin = wc * a.tiles_per_wave;
  const int t_end = min(ntile, t_begin + a.tiles_per_wave);
  const uint32_t* base = a.rec + (size_t)slot * (size_t)a.capacity * RW;
  // scores of this slot: row h (query head) at byte offset 4 h n_tok; lanes
  // of heads >= G store past the end of the resource and are dropped
  const __amdgpu_buffer_rsrc_t ors =
      slot_rsrc(a.scores + (size_t)slot * a.G * (size_t)n_tok, (uint32_t)a.G * (uint32_t)n_tok * 4u);
  const uint32_t orow = (uint32_t)r16 * (uint32_t)n_tok;
  // records of tokens past n_tokens (up to the slot's capacity, zeros past
  // it) are staged too; their rows are never stored
  const __amdgpu_buffer_rsrc_t krs = slot_rsrc(base, (uint32_t)a.capacity * (uint32_t)(RW * 4));
  uint32_t* slice = kst[wave];

  // One iteration: scores of U tiles staged from `cur` while the next U
  // tiles load into `nxt`.  Iterations alternate the two buffers.
  auto iteration = [&](Stage& cur, Stage& nxt, int tile) {
    if (tile + U < t_end) stage_load<RW, U>(nxt, krs, tile + U, lane);
    stage_store<RW, U>(slice, cur, lane);
    f4 acc[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      KeyTile<B, M> k;
      stage_key<B, M, Stage::STR>(k, slice, 16 * u + r16, q);
      acc[u] = key_tile_scores<B, M>(k, qb, tlo, thi, a.kappa, sh0);
      if (q == 0) nsh[wave][16 * u + r16] = k.n;
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const f4 nk = *(const f4*)&nsh[wave][16 * u + 4 * q];  // ||k|| of token rows 4q..4q+3
      const int t0 = (tile + u) * 16 + 4 * q;
      if (tile + u < t_end) {
        const f4 v = acc[u] * nk * qn;
        const uint32_t ob = (orow + (uint32_t)t0) * 4u;
        if (t0 + 4 <= n_tok) {
          __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u4, v), ors, ob, 0, kNonTemporal);
        } else {
#pragma unroll
          for (int i = 0; i < 4; ++i)
            if (t0 + i < n_tok) __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(v[i]), ors, ob + 4u * i, 0, 0);
        }
      }
    }
  };

  Stage sa, sb;
  if (t_begin < t_end) stage_load<RW, U>(sa, krs, t_begin, lane);
  for (int tile = t_begin; tile < t_end; tile += 2 * U) {
    iteration(sa, sb, tile);
    if (tile + U < t_end) iteration(sb, sa, tile + U);
  }
}

// ---------------------------------------------------------------------------
// attend: per-wave partials
// ---------------------------------------------------------------------------

struct AttendArgs {
  const uint32_t* rec;
  const uint32_t* vblocks;
  float* part;        // [n_seq][waves_per_slot][G][kPartFloats]
  const uint16_t* wq;
  const float* wqn;
  int64_t n_tokens, capacity;
  int n_seq, G, rec_words, block_words;
  int blocks_per_wave, waves_per_slot;
  float kappa, scale2;  // scale * log2(e)
  uint32_t tlo[4], thi[4];    // key centroid tables
  uint32_t vtlo[4], vthi[4];  // value centroid tables
};

template <int BK, int BV, int M>
struct StepKeys {  // the two 16-token key tiles of a 32-token step
  KeyTile<BK, M> t[2];
};

template <int BV>
struct BlockValues {  // one 128-token value block as this lane needs it
  uint32_t vw[8][BV];
  float2 vn;          // norms of block tokens 2 lane, 2 lane + 1
};

// Scores of a 16-token tile come out as lane (q, r16) = column (query head)
// r16, token rows 4q + i.  With G <= 4 (GC = 4) only columns 0..3 are real,
// so before the softmax each lane (q, 4a + h) takes row 4q + a of column h
// (three DPP row shifts): every lane then carries one real score per tile
// and the softmax runs on a quarter of the values.  Three more row shifts
// bring the weights back to the column lanes for the P operand.
__device__ __forceinline__ float compact4(const f4& v) {
  float x = v[0];
  x = dpp_into<0x114, 0x2>(x, v[1]);
  x = dpp_into<0x118, 0x4>(x, v[2]);
  x = dpp_into<0x11C, 0x8>(x, v[3]);
  return x;
}

// With 5 <= G <= 8 (GC = 2) lane (q, 8c + h) takes rows 4q + 2c + i (i = 0,
// 1) of column h: lanes 8..15 fetch rows 2 and 3 from lane h by a row shift.
__device__ __forceinline__ float compact2(const f4& v, int i) {
  return dpp_into<0x118, 0xC>(i == 0 ? v[0] : v[1], i == 0 ? v[2] : v[3]);
}

// The attend work of wave gw of the grid (waves_per_slot waves per slot).
// Every wave of the workgroup must call it (the pair tables are filled
// under a workgroup barrier).  sync() is called once by every wave (it may
// hold a workgroup barrier) after the wave has issued the loads of its
// first key and value block, if that block lies wholly before token
// `fresh_from`, and before anything else the wave reads: the fused decode
// step waits there for the step's new records and prepared queries, while
// the loads of older blocks are already in flight.  sync() returns true if
// the inputs never became ready; the wave then writes NaN partials.
struct NoSync {
  __device__ bool operator()() const { return false; }
};

template <int BK, int BV, int M, int GC, typename Sync>
__device__ __forceinline__ void attend_body(const AttendArgs& a, int64_t gw, const Sync& sync, int64_t fresh_from) {
  static_assert(GC == 1 || GC == 2 || GC == 4, "head compaction by 1, 2 or 4");
  constexpr int KBT = 4 + M / 32;
  constexpr int RW = rec_words<BK, M>();
  constexpr int BW = 4 * BV * kD + kBlockTokens;
  __shared__ float nsh[4][32];               // per wave: ||k|| of the step's 32 tokens
  __shared__ __align__(16) float vsh[4][kBlockTokens];  // per wave: the block's ||v||
  // 3-bit keys / values decode through LDS pair tables
  constexpr bool KPT = BK == 3, VPT = BV == 3;
  __shared__ PairTables ktab, vtab;
  uint32_t tlo[4], thi[4], vtlo[4], vthi[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    tlo[i] = a.tlo[i]; thi[i] = a.thi[i]; vtlo[i] = a.vtlo[i]; vthi[i] = a.vthi[i];
  }
  if constexpr (KPT || VPT) {
    if constexpr (KPT) fill_pair_tables(ktab, tlo, thi, threadIdx.x);
    if constexpr (VPT) fill_pair_tables(vtab, vtlo, vthi, (int)threadIdx.x - 128);
    __syncthreads();
  }
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int r16 = lane & 15, q = lane >> 4;
  // gw is wave-uniform (a scalar register): the slot's buffer descriptors
  // then stay scalar too
  const int gwu = __builtin_amdgcn_readfirstlane((int)gw);
  const int slot = gwu / a.waves_per_slot;
  if (slot >= a.n_seq) {
    (void)sync();
    return;
  }
  const int wc = gwu - slot * a.waves_per_slot;
  const int a4 = r16 >> 2;  // with GC = 4: this lane's row within a token quad
  const int c2 = r16 >> 3;  // with GC = 2: this lane's row pair within a token quad
  const int sh0 = 15 - 8 * (q & 1);
  const int n_tok = (int)a.n_tokens;
  const int nblk = (n_tok + kBlockTokens - 1) / kBlockTokens;
  const int b_begin = wc * a.blocks_per_wave;
  const int b_end = min(nblk, b_begin + a.blocks_per_wave);
  const uint32_t* kbase = a.rec + (size_t)slot * (size_t)a.capacity * RW;
  const uint32_t* vbase = a.vblocks + (size_t)slot * (size_t)(a.capacity / kBlockTokens) * BW;

  const __amdgpu_buffer_rsrc_t krs = slot_rsrc(kbase, (uint32_t)a.capacity * (uint32_t)(RW * 4));
  const __amdgpu_buffer_rsrc_t vrs = slot_rsrc(vbase, (uint32_t)(a.capacity / kBlockTokens) * (uint32_t)(BW * 4));
  const uint32_t vlane = 4u * (uint32_t)(q * kD + r16);
  auto load_keys = [&](StepKeys<BK, BV, M>& k, int tt) {  // tt: first token of the step
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int t = min(tt + 16 * u + r16, n_tok - 1);  // rows past the end: any valid row
      load_key<BK, M>(k.t[u], krs, (uint32_t)t * (uint32_t)(RW * 4), q);
    }
  };
  auto load_values = [&](BlockValues<BV>& v, int blk) {
    const uint32_t ob = (uint32_t)blk * (uint32_t)(BW * 4);
#pragma unroll
    for (int nt = 0; nt < 8; ++nt)
#pragma unroll
      for (int w = 0; w < BV; ++w) v.vw[nt][w] = bld(vrs, ob + vlane + 4u * (uint32_t)(w * 4 * kD + 16 * nt));
    const uint32_t on = ob + 4u * (uint32_t)(4 * BV * kD + 2 * lane);
    v.vn = make_float2(__uint_as_float(bld(vrs, on)), __uint_as_float(bld(vrs, on + 4u)));
  };

  float m_run = -INFINITY, l_run = 0.f;
  int ve = -1000;  // running exponent of the value norms (wave-uniform)
  f4 acc[8];
#pragma unroll
  for (int nt = 0; nt < 8; ++nt) acc[nt] = f4{0.f, 0.f, 0.f, 0.f};

  BlockValues<BV> vcur;
  StepKeys<BK, BV, M> kcur;
  const bool early = (int64_t)(b_begin + 1) * kBlockTokens <= fresh_from;  // first block holds no new token
  if (early && b_begin < b_end) {
    load_values(vcur, b_begin);
    load_keys(kcur, b_begin * kBlockTokens);
  }
  const bool poison = sync();
  if (!early && b_begin < b_end) {
    load_values(vcur, b_begin);
    load_keys(kcur, b_begin * kBlockTokens);
  }
  h8 qb[KBT];
#pragma unroll
  for (int kb = 0; kb < KBT; ++kb) qb[kb] = *(const h8*)(a.wq + (((int64_t)slot * KBT + kb) * 64 + lane) * 8);
  if constexpr (KPT) {
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) qb[kb] = to_pair_order(qb[kb]);
  }
  const float qsc = a.wqn[slot * 16 + (r16 & (16 / GC - 1))] * a.scale2;
  // One 128-token block.  MASK (the block holds the end of the cache) is a
  // compile-time flag so that full blocks carry no per-token masking code.
  auto run_block = [&](int blk, auto mask_tag) {
    constexpr bool MASK = decltype(mask_tag)::value;
    const int tok0 = blk * kBlockTokens;
    const bool more = blk + 1 < b_end;
    BlockValues<BV> vnext;
    if (more) load_values(vnext, blk + 1);  // in flight during this block
    // Value norms enter P as ||v|| 2^-ve with ve the running maximum
    // exponent of the norms seen so far, so P stays in fp16 range whatever
    // the norms' scale; the accumulator is rescaled when ve grows.
    float x0 = vcur.vn.x, x1 = vcur.vn.y;
    if constexpr (MASK) {
      x0 = tok0 + 2 * lane < n_tok ? x0 : 0.f;
      x1 = tok0 + 2 * lane + 1 < n_tok ? x1 : 0.f;
    }
    const float bmax = wave_max(fmaxf(x0, x1));
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
      StepKeys<BK, BV, M> knext;
      if (step < 3) load_keys(knext, tok0 + 32 * (step + 1));
      else if (more) load_keys(knext, tok0 + kBlockTokens);
      f4 sc[2];
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        sc[u] = key_tile_scores<BK, M, KPT>(kcur.t[u], qb, tlo, thi, a.kappa, sh0, &ktab);
        if (q == 0) nsh[wave][16 * u + r16] = kcur.t[u].n;
      }
      // NV score values per tile in this lane: rows 4q + i (GC = 1) or row
      // 4q + a4 (GC = 4)
      constexpr int NV = 4 / GC;
      float nk[2][NV], vn[2][NV], lg[2][NV];
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        if constexpr (GC == 1) {
          const f4 n4 = *(const f4*)&nsh[wave][16 * u + 4 * q];
          const f4 v4 = *(const f4*)&vsh[wave][16 * (2 * step + u) + 4 * q];
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            nk[u][i] = n4[i];
            vn[u][i] = v4[i];
            lg[u][i] = sc[u][i];
          }
        } else if constexpr (GC == 2) {
#pragma unroll
          for (int i = 0; i < 2; ++i) {
            nk[u][i] = nsh[wave][16 * u + 4 * q + 2 * c2 + i];
            vn[u][i] = vsh[wave][16 * (2 * step + u) + 4 * q + 2 * c2 + i];
            lg[u][i] = compact2(sc[u], i);
          }
        } else {
          nk[u][0] = nsh[wave][16 * u + 4 * q + a4];
          vn[u][0] = vsh[wave][16 * (2 * step + u) + 4 * q + a4];
          lg[u][0] = compact4(sc[u]);
        }
      }
      float cmax = -INFINITY;
#pragma unroll
      for (int u = 0; u < 2; ++u)
#pragma unroll
        for (int i = 0; i < NV; ++i) {
          float l = lg[u][i] * nk[u][i] * qsc;
          if constexpr (MASK)
            l = tok0 + 16 * (2 * step + u) + 4 * q + (GC == 4 ? a4 : GC == 2 ? 2 * c2 + i : i) < n_tok ? l : -INFINITY;
          lg[u][i] = l;
          cmax = fmaxf(cmax, l);
        }
      if constexpr (GC == 4) {  // the four row lanes 4a + h of a head
        cmax = fmaxf(cmax, dpp_f<0x124>(cmax));
        cmax = fmaxf(cmax, dpp_f<0x128>(cmax));
      } else if constexpr (GC == 2) {  // the two row lanes h, h + 8 of a head
        cmax = fmaxf(cmax, dpp_f<0x128>(cmax));
      }
      cmax = max_xor16_32(cmax);
      // Online softmax with lazy rescaling: the accumulator is rescaled only
      // when some head's running maximum grows (rare after the first blocks).
      if (__any(cmax > m_run)) {
        const float m_new = fmaxf(m_run, cmax);
        const float alpha = exp2_hw(m_run - m_new);  // 0 on the first step
#pragma unroll
        for (int nt = 0; nt < 8; ++nt) acc[nt] *= alpha;
        l_run *= alpha;
        m_run = m_new;
      }
      float psum = 0.f;
      float pv[2][NV];
#pragma unroll
      for (int u = 0; u < 2; ++u)
#pragma unroll
        for (int i = 0; i < NV; ++i) {
          const float p = exp2_hw(lg[u][i] - m_run);
          psum += p;
          pv[u][i] = p * vn[u][i];
        }
      l_run += psum;
      // P operand: slot order (tokens of tile 0, then tile 1) for byte-permute
      // decoding, pair order (tile 0 / tile 1 of each row i) for the pair
      // tables.  With GC = 4 row i of head h sits in lane 4i + h (read back by
      // row shifts; lanes of columns >= 4 take values of no head, and their
      // accumulator columns are never stored).
      u4 pw;
      if constexpr (GC == 1) {
#pragma unroll
        for (int j = 0; j < 4; ++j)
          pw[j] = VPT ? pack_h2(pv[0][j], pv[1][j]) : pack_h2(pv[j >> 1][2 * (j & 1)], pv[j >> 1][2 * (j & 1) + 1]);
      } else if constexpr (GC == 2 && VPT) {  // rows 2, 3 of head h sit in lane h + 8
        const uint32_t x0 = pack_h2(pv[0][0], pv[1][0]), x1 = pack_h2(pv[0][1], pv[1][1]);
        pw[0] = x0;
        pw[1] = x1;
        pw[2] = dpp_into<0x108, 0xF>(0u, x0);
        pw[3] = dpp_into<0x108, 0xF>(0u, x1);
      } else if constexpr (GC == 2) {
        float pr[2][4];
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          pr[u][0] = pv[u][0];
          pr[u][1] = pv[u][1];
          pr[u][2] = dpp_into<0x108, 0xF>(0.f, pv[u][0]);
          pr[u][3] = dpp_into<0x108, 0xF>(0.f, pv[u][1]);
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) pw[j] = pack_h2(pr[j >> 1][2 * (j & 1)], pr[j >> 1][2 * (j & 1) + 1]);
      } else if constexpr (VPT) {
        const uint32_t x = pack_h2(pv[0][0], pv[1][0]);
        pw[0] = x;
        pw[1] = dpp_into<0x104, 0xF>(0u, x);
        pw[2] = dpp_into<0x108, 0xF>(0u, x);
        pw[3] = dpp_into<0x10C, 0xF>(0u, x);
      } else {
        float pr[2][4];
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          pr[u][0] = pv[u][0];
          pr[u][1] = dpp_into<0x104, 0xF>(0.f, pv[u][0]);
          pr[u][2] = dpp_into<0x108, 0xF>(0.f, pv[u][0]);
          pr[u][3] = dpp_into<0x10C, 0xF>(0.f, pv[u][0]);
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) pw[j] = pack_h2(pr[j >> 1][2 * (j & 1)], pr[j >> 1][2 * (j & 1) + 1]);
      }
      const h8 P = as_h8(pw);
#pragma unroll
      for (int nt = 0; nt < 8; ++nt) {
        h8 A;
        if constexpr (VPT) {
          if (step == 0) A = decode_pair_lds<0>(vcur.vw[nt], vtab);
          if (step == 1) A = decode_pair_lds<1>(vcur.vw[nt], vtab);
          if (step == 2) A = decode_pair_lds<2>(vcur.vw[nt], vtab);
          if (step == 3) A = decode_pair_lds<3>(vcur.vw[nt], vtab);
        } else {
          if (step == 0) A = decode_pair<BV, 0>(vcur.vw[nt], vtlo, vthi);
          if (step == 1) A = decode_pair<BV, 2>(vcur.vw[nt], vtlo, vthi);
          if (step == 2) A = decode_pair<BV, 4>(vcur.vw[nt], vtlo, vthi);
          if (step == 3) A = decode_pair<BV, 6>(vcur.vw[nt], vtlo, vthi);
        }
        acc[nt] = mfma(A, P, acc[nt]);
      }
      kcur = knext;
    }
    vcur = vnext;
  };
  for (int blk = b_begin; blk < b_end; ++blk) {
    if ((blk + 1) * kBlockTokens <= n_tok)  // wave-uniform
      run_block(blk, std::false_type{});
    else
      run_block(blk, std::true_type{});
  }
  if constexpr (GC == 4) {  // the four row lanes of a head
    l_run += dpp_f<0x124>(l_run);
    l_run += dpp_f<0x128>(l_run);
  } else if constexpr (GC == 2) {  // the two row lanes of a head
    l_run += dpp_f<0x128>(l_run);
  }
  l_run += shfl_xor(l_run, 16);
  l_run += shfl_xor(l_run, 32);
  // The partial keeps the accumulator in the scale of P (value norms times
  // 2^-ve) and stores ve beside it: the combine merges partials at their
  // largest exponent, so no intermediate leaves the fp32 range when the true
  // output is inside it (value norms up to the fp32 maximum).
  if (r16 < a.G) {
    float* pr = a.part + (((int64_t)slot * a.waves_per_slot + wc) * a.G + r16) * kPartFloats;
    if (poison) {
      m_run = l_run = __builtin_nanf("");
#pragma unroll
      for (int nt = 0; nt < 8; ++nt) acc[nt] = f4{m_run, m_run, m_run, m_run};
    }
    if (q == 0) {
      pr[0] = m_run;
      pr[1] = l_run;
      pr[2] = (float)ve;
    }
#pragma unroll
    for (int nt = 0; nt < 8; ++nt) *(f4*)(pr + 4 + 16 * nt + 4 * q) = acc[nt];
  }
}

template <int BK, int BV, int M, int GC>
__global__ __launch_bounds__(256) void attend_kernel(const AttendArgs a) {
  attend_body<BK, BV, M, GC>(a, (int64_t)blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6), NoSync{},
                             INT64_MAX);
}

// ---------------------------------------------------------------------------
// combine partials, rotate back: out = R^T (sum_c w_c acc_c / sum_c w_c l_c)
// ---------------------------------------------------------------------------

struct CombineArgs {
  const float* part;
  float* out;
  const float* r32;
  int n_seq, G, waves_per_slot;
};

// The combine of one (slot, query head) by a workgroup of NG x 128 threads
// (NG = 2 or 4): thread (g, j) takes coordinate j of every NG-th partial,
// then 128 / NG of R's rows.  A partial c holds (m_c, l_c, ve_c, acc_c) with
// the head's output share acc_c 2^ve_c; the merge scales each by
// exp2(m_c - M) 2^(ve_c - VE) with M and VE the largest m_c and ve_c of the
// partials that carry weight, divides by L before the final 2^VE, and rotates
// back last.  The workgroup's shared arrays are reused by the next call, so
// calls are separated by the barriers inside.
template <int NG>
__device__ __forceinline__ void combine_body(const CombineArgs& a, int slot, int h) {
  __shared__ float w[kMaxPartials];  // per-partial weights exp2(m_c - M) 2^(ve_c - VE)
  __shared__ float red[3][8];
  __shared__ float part[NG][kD];
  __shared__ __align__(16) float y[kD];
  constexpr int nw = 2 * NG;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int j = tid & (kD - 1), g = tid >> 7;
  const int W = a.waves_per_slot;
  const float* pr = a.part + ((int64_t)slot * W * a.G + h) * kPartFloats;
  const int64_t stride = (int64_t)a.G * kPartFloats;
  __syncthreads();  // (the previous call's reads of the shared arrays are done)
  // M = max of the partial maxima; VE = max exponent among partials with weight
  float M = -INFINITY, VE = -INFINITY;
  for (int c = tid; c < W; c += blockDim.x) {
    const float mc = pr[c * stride];
    M = fmaxf(M, mc);
    if (mc != -INFINITY) VE = fmaxf(VE, pr[c * stride + 2]);
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    M = fmaxf(M, shfl_xor(M, o));
    VE = fmaxf(VE, shfl_xor(VE, o));
  }
  if (lane == 0) {
    red[0][wave] = M;
    red[2][wave] = VE;
  }
  __syncthreads();
  M = red[0][0];
  VE = red[2][0];
#pragma unroll
  for (int i = 1; i < nw; ++i) {
    M = fmaxf(M, red[0][i]);
    VE = fmaxf(VE, red[2][i]);
  }
  const int ve_max = VE == -INFINITY ? 0 : (int)VE;
  // weights and the weighted sum of the partial sums (l_c is in softmax
  // units, so it takes exp2(m_c - M) only)
  float L = 0.f;
  for (int c = tid; c < W; c += blockDim.x) {
    const float mc = pr[c * stride];
    const float e = mc == -INFINITY ? 0.f : exp2f(mc - M);
    w[c] = ldexpf(e, (int)pr[c * stride + 2] - ve_max);
    L = fmaf(e, pr[c * stride + 1], L);
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) L += shfl_xor(L, o);
  if (lane == 0) red[1][wave] = L;
  __syncthreads();
  L = 0.f;
#pragma unroll
  for (int i = 0; i < nw; ++i) L += red[1][i];
  // thread (g, j): partials c = g, g + NG, ..., 8 loads in flight
  float acc[8];
#pragma unroll
  for (int u = 0; u < 8; ++u) acc[u] = 0.f;
  int c = g;
  for (; c + 7 * NG < W; c += 8 * NG) {
#pragma unroll
    for (int u = 0; u < 8; ++u) acc[u] = fmaf(w[c + NG * u], pr[(c + NG * u) * stride + 4 + j], acc[u]);
  }
  for (; c < W; c += NG) acc[0] = fmaf(w[c], pr[c * stride + 4 + j], acc[0]);
#pragma unroll
  for (int u = 1; u < 8; ++u) acc[0] += acc[u];
  part[g][j] = acc[0];
  __syncthreads();
  if (g == 0) {
    float t = part[0][j];
#pragma unroll
    for (int i = 1; i < NG; ++i) t += part[i][j];
    y[j] = t / L;
  }
  __syncthreads();
  // out = 2^VE R^T y: thread (g, j) sums rows g (128/NG) .. of column j
  constexpr int nr = kD / NG;
  float o[8];
#pragma unroll
  for (int u = 0; u < 8; ++u) o[u] = 0.f;
  const float* rc = a.r32 + (size_t)(nr * g) * kD + j;
#pragma unroll
  for (int i = 0; i < nr; i += 8) {
#pragma unroll
    for (int u = 0; u < 8; ++u) o[u] = fmaf(rc[(i + u) * kD], y[nr * g + i + u], o[u]);
  }
#pragma unroll
  for (int u = 1; u < 8; ++u) o[0] += o[u];
  __syncthreads();
  part[g][j] = o[0];
  __syncthreads();
  if (g == 0) {
    float t = part[0][j];
#pragma unroll
    for (int i = 1; i < NG; ++i) t += part[i][j];
    a.out[((int64_t)slot * a.G + h) * kD + j] = ldexpf(t, ve_max);
  }
}

// One workgroup of 4 x 128 threads per (slot, query head).
__global__ __launch_bounds__(512) void combine_kernel(const CombineArgs a) {
  combine_body<4>(a, (int)(blockIdx.x / a.G), (int)(blockIdx.x % a.G));
}

// The combine of all G query heads of one slot by a workgroup of 256
// threads (the fused decode step's last workgroup of the slot), over W
// partials [c][h][kPartFloats] at pr, with the arithmetic of combine_body.
// Written for latency (the partials come from other compute units, past
// this unit's caches), in three rounds of loads issued together:
//  1. thread t loads its 64 entries of R (rows 16 (t / 32) .. + 15,
//     columns 4 (t % 32) .. + 3) and the (m, l, ve) of the partials of its
//     heads;
//  2. thread (h, j4) loads coordinates 4 j4 .. 4 j4 + 3 of head h of every
//     partial and forms the merged rotated-domain output y[h] in LDS;
//  3. R^T y: each thread multiplies its R entries with y of every head, and
//     the 8 row blocks are summed through LDS (two of them per wave by a
//     lane exchange first).
__device__ __forceinline__ void combine_slot(const CombineArgs& a, int slot, const float* pr, int W) {
  __shared__ float wsh[kStepMaxPartials];  // weights of (c, h); W G <= kStepMaxPartials (checked by the launcher)
  __shared__ float hL[16];
  __shared__ int hE[16];
  __shared__ __align__(16) float y[16][kD];
  __shared__ __align__(16) float ob[4][16][kD];  // R^T y partial sums of the 4 waves
  const int G = a.G, tid = threadIdx.x;
  const int j4 = tid & 31, rb = tid >> 5;  // R: columns 4 j4 .. +3, rows 16 rb .. +15
  f4 rr[16];
#pragma unroll
  for (int u = 0; u < 16; ++u) rr[u] = *(const f4*)(a.r32 + (size_t)(16 * rb + u) * kD + 4 * j4);
  __syncthreads();  // (the shared arrays are free)
  {
    const int h = tid >> 4, sub = tid & 15;
    float M = -INFINITY, VE = -INFINITY;
    if (h < G)
      for (int c = sub; c < W; c += 16) {
        const float* p = pr + ((int64_t)c * G + h) * kPartFloats;
        const float mc = p[0];
        M = fmaxf(M, mc);
        if (mc != -INFINITY) VE = fmaxf(VE, p[2]);
      }
#pragma unroll
    for (int o = 8; o > 0; o >>= 1) {
      M = fmaxf(M, shfl_xor(M, o));
      VE = fmaxf(VE, shfl_xor(VE, o));
    }
    const int ve_max = VE == -INFINITY ? 0 : (int)VE;
    float L = 0.f;
    if (h < G)
      for (int c = sub; c < W; c += 16) {  // (the same lines again: now cached here)
        const float* p = pr + ((int64_t)c * G + h) * kPartFloats;
        const float mc = p[0];
        const float e = mc == -INFINITY ? 0.f : exp2f(mc - M);
        wsh[c * G + h] = ldexpf(e, (int)p[2] - ve_max);
        L = fmaf(e, p[1], L);
      }
#pragma unroll
    for (int o = 8; o > 0; o >>= 1) L += shfl_xor(L, o);
    if (sub == 0 && h < G) {
      hL[h] = L;
      hE[h] = ve_max;
    }
  }
  __syncthreads();
  for (int e = tid; e < 32 * G; e += blockDim.x) {
    const int h = e >> 5, q4 = e & 31;
    const float* p = pr + (int64_t)h * kPartFloats + 4 + 4 * q4;
    const int64_t st = (int64_t)G * kPartFloats;
    f4 acc = {0.f, 0.f, 0.f, 0.f};
    int c = 0;
    for (; c + 15 < W; c += 16) {
      f4 v[16];
#pragma unroll
      for (int u = 0; u < 16; ++u) v[u] = *(const f4*)(p + (c + u) * st);
#pragma unroll
      for (int u = 0; u < 16; ++u) acc += wsh[(c + u) * G + h] * v[u];
    }
    for (; c < W; ++c) acc += wsh[c * G + h] * *(const f4*)(p + c * st);
    *(f4*)&y[h][4 * q4] = acc / hL[h];
  }
  __syncthreads();
  {
    const int wv = tid >> 6;
    for (int h = 0; h < G; ++h) {
      f4 o = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int u = 0; u < 16; ++u) o += rr[u] * y[h][16 * rb + u];
#pragma unroll
      for (int e = 0; e < 4; ++e) o[e] += shfl_xor(o[e], 32);  // the wave's two row blocks
      if ((tid & 32) == 0) *(f4*)&ob[wv][h][4 * j4] = o;
    }
  }
  __syncthreads();
  for (int e = tid; e < G * kD; e += blockDim.x) {
    const int h = e >> 7, j = e & (kD - 1);
    a.out[((int64_t)slot * G + h) * kD + j] =
        ldexpf((ob[0][h][j] + ob[1][h][j]) + (ob[2][h][j] + ob[3][h][j]), hE[h]);
  }
}

// ---------------------------------------------------------------------------
// plans and launchers
// ---------------------------------------------------------------------------

static int g_cus = 256;

// Scratch of tq_attend_noalloc, for callers that cannot allocate device
// memory: a file-scope device array (each GPU the library runs on holds its
// own copy until the process ends) standing in for the attend workspace.
// In host code `scratch` is only a host-side stand-in for the symbol; its
// device address comes from hipGetSymbolAddress, looked up once per device
// with that device current and kept per device.  Every call on one GPU
// shares the array, so calls that overlap on one GPU race.  Nothing in it
// needs clearing between calls: the query preparation writes the operands
// and norms, and the attend kernel writes every partial the combine reads.
static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};
}  // namespace

int noalloc_scratch_init(int device) {
  if (device < 0 || device >= kMaxDevices) return TQ_EDEVICE;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[device]) return 0;
  int cur = -1;
  if (hipGetDevice(&cur) != hipSuccess || cur != device) return TQ_EDEVICE;
  void* ptr = nullptr;
  if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) return TQ_EDEVICE;
  g_scratch_ptr[device] = ptr;
  return 0;
}

void* noalloc_scratch_ptr(int device) {
  if (device < 0 || device >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  return g_scratch_ptr[device];
}

int attention_device_init() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return -1;
  if (hipDeviceGetAttribute(&g_cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return -1;
  return 0;
}

AttnPlan plan_attention(int m, int n_seq, int G, int64_t n_tokens) {
  AttnPlan p;
  const int KBT = 4 + m / 32;
  const int64_t nblk = (n_tokens + kBlockTokens - 1) / kBlockTokens;
  const int64_t target_waves = kAttendWaves;
  int64_t bpw = (nblk * n_seq + target_waves - 1) / target_waves;
  if (bpw < 1) bpw = 1;
  // the combine kernel merges at most kMaxPartials partials per query head
  if ((nblk + bpw - 1) / bpw > kMaxPartials) bpw = (nblk + kMaxPartials - 1) / kMaxPartials;
  p.blocks_per_wave = (int)bpw;
  p.waves_per_slot = (int)((nblk + bpw - 1) / bpw);
  p.q_bytes = (size_t)n_seq * KBT * 64 * 8 * 2;
  p.qn_bytes = (size_t)n_seq * 16 * 4;
  p.part_bytes = (size_t)n_seq * p.waves_per_slot * G * kPartFloats * 4;
  p.sync_bytes = (size_t)n_seq * kSyncWords * 8 + 16;  // fused decode step: flags and counts, a status word
  p.group_bytes = (size_t)n_seq * (p.waves_per_slot / 4 + 2) * G * kPartFloats * 4;  // its workgroup partials
  p.total = ((p.q_bytes + 255) / 256 + (p.qn_bytes + 255) / 256 + (p.part_bytes + 255) / 256 +
             (p.sync_bytes + 255) / 256 + (p.group_bytes + 255) / 256) * 256;
  return p;
}

struct WsPtrs {
  uint16_t* wq;
  float* wqn;
  float* part;
  unsigned long long* sync;
  float* group;
};
static WsPtrs ws_ptrs(void* ws, const AttnPlan& p) {
  char* b = (char*)ws;
  WsPtrs w;
  w.wq = (uint16_t*)b;
  b += (p.q_bytes + 255) / 256 * 256;
  w.wqn = (float*)b;
  b += (p.qn_bytes + 255) / 256 * 256;
  w.part = (float*)b;
  b += (p.part_bytes + 255) / 256 * 256;
  w.sync = (unsigned long long*)b;
  b += (p.sync_bytes + 255) / 256 * 256;
  w.group = (float*)b;
  return w;
}


int launch_prep_queries(const Matrices& mats, int m, const AttnShape& s, void* ws, const AttnPlan& p,
                        void* stream) {
  // one workgroup per (slot, head), wave-parallel dot products (tq_general.hip);
  // with a single head group its operands have the layout read here
  const WsPtrs w = ws_ptrs(ws, p);
  return launch_gen_prep(mats, kD, m, s, 1, w.wq, w.wqn, stream);
}

static void fill_tables(const CodebookDev& cb, uint32_t* tlo, uint32_t* thi) {
  for (int i = 0; i < 4; ++i) { tlo[i] = cb.tlo[i]; thi[i] = cb.thi[i]; }
}

int launch_scores(const CodebookDev& cbk, int kbits, int m, const AttnShape& s, const void* key_records,
                  float* scores, void* ws, const AttnPlan& p, void* stream) {
  ScoreArgs a;
  const WsPtrs w = ws_ptrs(ws, p);
  a.rec = (const uint32_t*)key_records;
  a.scores = scores;
  a.wq = w.wq;
  a.wqn = w.wqn;
  a.n_tokens = s.n_tokens;
  a.capacity = s.capacity;
  a.n_seq = s.n_seq;
  a.G = s.G;
  a.rec_words = kbits * kD / 32 + m / 32 + 2;
  const int64_t ntile = (s.n_tokens + 15) / 16, total = ntile * s.n_seq;
  const int64_t tpw = std::max((total + kScoreWavesMax - 1) / kScoreWavesMax,
                               std::min(kScoreTilesPerWave, (total + kScoreWavesMin - 1) / kScoreWavesMin));
  a.tiles_per_wave = (int)tpw;
  a.waves_per_slot = (int)((ntile + tpw - 1) / tpw);
  a.kappa = (float)(1.2533141373155002512 / m);  // sqrt(pi/2) / m
  fill_tables(cbk, a.tlo, a.thi);
  const int64_t waves = (int64_t)a.waves_per_slot * s.n_seq;
  const dim3 grid((unsigned)((waves + 3) / 4)), block(256);
  hipStream_t st = (hipStream_t)stream;
#define TQ_SC(B, M) \
  if (kbits == B && m == M) { hipLaunchKernelGGL((scores_kernel<B, M>), grid, block, 0, st, a); goto done; }
  TQ_SC(0, 64) TQ_SC(1, 64) TQ_SC(2, 64) TQ_SC(3, 64) TQ_SC(4, 64)
  TQ_SC(0, 128) TQ_SC(1, 128) TQ_SC(2, 128) TQ_SC(3, 128) TQ_SC(4, 128)
#undef TQ_SC
  return TQ_EUNSUPPORTED;
done:
  return hipGetLastError() == hipSuccess ? 0 : TQ_EDEVICE;
}

static AttendArgs attend_args(const CodebookDev& cbk, int kbits, const CodebookDev& cbv, int vbits, int m,
                              const AttnShape& s, const void* key_records, const void* value_blocks, float scale,
                              const WsPtrs& w, const AttnPlan& p) {
  AttendArgs a;
  a.rec = (const uint32_t*)key_records;
  a.vblocks = (const uint32_t*)value_blocks;
  a.part = w.part;
  a.wq = w.wq;
  a.wqn = w.wqn;
  a.n_tokens = s.n_tokens;
  a.capacity = s.capacity;
  a.n_seq = s.n_seq;
  a.G = s.G;
  a.rec_words = kbits * kD / 32 + m / 32 + 2;
  a.block_words = 4 * vbits * kD + kBlockTokens;
  a.blocks_per_wave = p.blocks_per_wave;
  a.waves_per_slot = p.waves_per_slot;
  a.kappa = (float)(1.2533141373155002512 / m);
  a.scale2 = scale * kLog2e;
  fill_tables(cbk, a.tlo, a.thi);
  fill_tables(cbv, a.vtlo, a.vthi);
  return a;
}

static CombineArgs combine_args(const Matrices& mats, const AttnShape& s, float* out, const WsPtrs& w,
                                const AttnPlan& p) {
  CombineArgs c;
  c.part = w.part;
  c.out = out;
  c.r32 = mats.r32;
  c.n_seq = s.n_seq;
  c.G = s.G;
  c.waves_per_slot = p.waves_per_slot;
  return c;
}

int launch_attend(const Matrices& mats, const CodebookDev& cbk, int kbits, const CodebookDev& cbv, int vbits,
                  int m, const AttnShape& s, const void* key_records, const void* value_blocks, float scale,
                  float* out, void* ws, const AttnPlan& p, void* stream) {
  const WsPtrs w = ws_ptrs(ws, p);
  const AttendArgs a = attend_args(cbk, kbits, cbv, vbits, m, s, key_records, value_blocks, scale, w, p);
  const int64_t waves = (int64_t)a.waves_per_slot * s.n_seq;
  const dim3 grid((unsigned)((waves + 3) / 4)), block(256);
  hipStream_t st = (hipStream_t)stream;
  bool launched = false;
#define TQ_AT(BK, BV, M)                                                                   \
  if (!launched && kbits == BK && vbits == BV && m == M) {                                 \
    if (s.G <= 4) hipLaunchKernelGGL((attend_kernel<BK, BV, M, 4>), grid, block, 0, st, a); \
    else if (s.G <= 8) hipLaunchKernelGGL((attend_kernel<BK, BV, M, 2>), grid, block, 0, st, a); \
    else hipLaunchKernelGGL((attend_kernel<BK, BV, M, 1>), grid, block, 0, st, a);          \
    launched = true;                                                                       \
  }
#define TQ_AT_V(BK, M) TQ_AT(BK, 1, M) TQ_AT(BK, 2, M) TQ_AT(BK, 3, M) TQ_AT(BK, 4, M)
  TQ_AT_V(0, 64) TQ_AT_V(1, 64) TQ_AT_V(2, 64) TQ_AT_V(3, 64) TQ_AT_V(4, 64)
  TQ_AT_V(0, 128) TQ_AT_V(1, 128) TQ_AT_V(2, 128) TQ_AT_V(3, 128) TQ_AT_V(4, 128)
#undef TQ_AT_V
#undef TQ_AT
  if (!launched) return TQ_EUNSUPPORTED;
  if (hipGetLastError() != hipSuccess) return TQ_EDEVICE;
  const CombineArgs c = combine_args(mats, s, out, w, p);
  hipLaunchKernelGGL(combine_kernel, dim3((unsigned)(s.n_seq * s.G)), dim3(4 * kD), 0, st, c);
  return hipGetLastError() == hipSuccess ? 0 : TQ_EDEVICE;
}

// ---------------------------------------------------------------------------
// the fused decode step: appends, query preparation, attend and combine in
// one launch
// ---------------------------------------------------------------------------
//
// The grid's first workgroups are the producers of the step's inputs (the
// key appends, the value appends and the query preparation, one workgroup
// each, as in the separate small-append and preparation kernels); the rest
// run the attend waves, which issue the loads of their first block (if it
// predates the step) before they wait for the producers, then merge their
// partials and combine (see decode_step_kernel).
//
// The flags and counts live in the caller's workspace, which nobody clears:
// a flag is set to a 40-bit epoch that no earlier launch of the process
// used, so stale flags of earlier steps, or of other contexts sharing the
// workspace, are never mistaken for this step's.  (Uninitialised memory
// holding this launch's tag by chance is the one case not covered: odds of
// 2^-40 a word.)

constexpr int kWaitSpins = 1 << 20;  // polls of about 1 us (the flags' round trip and s_sleep(2)): about a second

// Wait (bounded) until the n flags at f all hold `tag`.  The spin reads
// relaxed (device-coherent loads, no cache maintenance per poll); the
// caller issues one acquire fence after the wait.
__device__ __forceinline__ bool flags_wait(const unsigned long long* f, int n, unsigned long long tag) {
  for (int i = 0; i < kWaitSpins; ++i) {
    bool all = true;
    for (int k = 0; k < n; ++k)
      all = (__hip_atomic_load(f + k, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == tag) && all;
    if (all) return true;
    __builtin_amdgcn_s_sleep(2);
  }
  return false;
}

struct StepArgs {
  DecodeArgs prep;             // producers: key appends, value appends, query preparation
  AttendArgs att;
  CombineArgs comb;
  unsigned long long* sync;    // [n_seq][kSyncWords]: producer flags, then the done count (word kSyncWords - 1)
  uint32_t* status;            // 1 after a wait gave up
  unsigned long long epoch;    // this launch's tag (1 .. 2^40 - 1)
  float* group;                // [n_seq][group_stride][G][kPartFloats] workgroup partials
  int group_stride;            // workgroup partials a slot has room for (waves_per_slot / 4 + 2)
  int64_t fresh_from;          // first new token (its block onwards is read only after the wait)
  int n_prod;                  // producer workgroups
  int prod_per_slot;           // producer workgroups of one slot
  int vblk_per_slot;           // value-append workgroups of one slot
};

// Synchronisation.  Producer k of slot s, once its stores are out, sets
// flag k of the slot to this launch's tag with a release store; producer 0
// also zeroes the slot's done count first.  An attend workgroup waits for
// all flags of the slots its waves cover (acquire), attends, merges its
// waves' partials into one, and adds 1 to each slot's done count; the add
// that completes a slot (acquire-release) makes its workgroup the one that
// combines the slot, after which it clears the slot's flags so that a
// replayed launch (a captured HIP graph keeps its arguments, tag included)
// waits again.  No count is shared by contending producers, and no
// workgroup waits for one of higher index, which the dispatcher starts
// later, so every wait ends.
template <int BK, int BV, int M, int GC>
__global__ __launch_bounds__(256) void decode_step_kernel(const StepArgs a) {
  __shared__ int flag[5];  // [0]: inputs missing; [1 + i]: this workgroup completes slot s_lo + i
  const int b = (int)blockIdx.x;
  if (b < a.n_prod) {
    const DecodeArgs& p = a.prep;
    int slot, k;
    if (b < p.nk) {
      small_keys_block(p.k, b);
      slot = (int)(b / p.k.n_new);
      k = (int)(b % p.k.n_new);
    } else if (b < p.nk + p.nv) {
      small_values_block(p.v, b - p.nk);
      slot = (b - p.nk) / a.vblk_per_slot;
      k = (int)p.k.n_new + (b - p.nk) % a.vblk_per_slot;
    } else {
      gen_prep_block(p.p, b - p.nk - p.nv);
      slot = (b - p.nk - p.nv) / 16;
      k = (int)p.k.n_new + a.vblk_per_slot + (b - p.nk - p.nv) % 16;
    }
    // The barrier waits for the workgroup's stores; the release store then
    // makes them visible device-wide (one L2 write-back for the workgroup).
    __syncthreads();
    if (threadIdx.x == 0) {
      unsigned long long* f = a.sync + (size_t)slot * kSyncWords;
      if (k == 0) __hip_atomic_store(f + kSyncWords - 1, 0ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __hip_atomic_store(f + k, a.epoch, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
    }
    return;
  }
  const int W = a.att.waves_per_slot;
  const int64_t gw0 = (int64_t)(b - a.n_prod) * 4;
  const int s_lo = (int)(gw0 / W);
  const int64_t s_end = (gw0 + 3) / W;
  const int s_hi = (int)(s_end < a.att.n_seq - 1 ? s_end : a.att.n_seq - 1);
  auto sync = [&]() {
    if (threadIdx.x == 0) {
      bool ok = true;
      for (int s = s_lo; s <= s_hi; ++s)
        ok = flags_wait(a.sync + (size_t)s * kSyncWords, a.prod_per_slot, a.epoch) && ok;
      if (!ok) __hip_atomic_store(a.status, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      flag[0] = ok ? 0 : 1;
      // acquire: this CU's caches drop lines older than the producers' stores
      // (the other waves read after the barrier below)
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
    }
    __syncthreads();
    return flag[0] != 0;
  };
  attend_body<BK, BV, M, GC>(a.att, gw0 + (threadIdx.x >> 6), sync, a.fresh_from);
  __syncthreads();  // the workgroup's wave partials written (read back below from this CU)
  // Merge the workgroup's waves of each slot into one workgroup partial
  // (the same log-sum-exp merge as the combine), so the slot's completing
  // workgroup reads a quarter as many.  Workgroup partial gi of slot s is
  // written by the workgroup whose first wave is 4 (gi + floor(s W / 4)).
  const int G = a.att.G;
  for (int s = s_lo; s <= s_hi; ++s) {
    const int64_t lo = (int64_t)s * W, hi = (int64_t)(s + 1) * W;
    const int c0 = (int)((gw0 > lo ? gw0 : lo) - lo), c1 = (int)((gw0 + 4 < hi ? gw0 + 4 : hi) - lo);
    const int gi = (int)(gw0 / 4 - lo / 4);
    const float* src = a.att.part + (int64_t)s * W * G * kPartFloats;
    float* dst = a.group + ((int64_t)s * a.group_stride + gi) * G * kPartFloats;
    for (int e = threadIdx.x; e < 32 * G; e += blockDim.x) {
      const int h = e >> 5, j4 = e & 31;
      float Mx = -INFINITY, VE = -INFINITY;
      for (int c = c0; c < c1; ++c) {
        const float* p = src + ((int64_t)c * G + h) * kPartFloats;
        Mx = fmaxf(Mx, p[0]);
        if (p[0] != -INFINITY) VE = fmaxf(VE, p[2]);
      }
      const int ve = VE == -INFINITY ? -1000 : (int)VE;
      float L = 0.f;
      f4 acc = {0.f, 0.f, 0.f, 0.f};
      for (int c = c0; c < c1; ++c) {
        const float* p = src + ((int64_t)c * G + h) * kPartFloats;
        const float e2 = p[0] == -INFINITY ? 0.f : exp2f(p[0] - Mx);
        L = fmaf(e2, p[1], L);
        acc += ldexpf(e2, (int)p[2] - ve) * *(const f4*)(p + 4 + 4 * j4);
      }
      float* d = dst + (int64_t)h * kPartFloats;
      *(f4*)(d + 4 + 4 * j4) = acc;
      if (j4 == 0) {
        d[0] = Mx;
        d[1] = L;
        d[2] = (float)ve;
      }
    }
  }
  __syncthreads();  // the workgroup partials written (the adds below release them)
  if (threadIdx.x == 0) {
    for (int s = s_lo; s <= s_hi; ++s) {
      const int64_t lo = (int64_t)s * W, hi = (int64_t)(s + 1) * W;
      const uint32_t n_groups = (uint32_t)((hi - 1) / 4 - lo / 4 + 1);
      unsigned long long* done = a.sync + (size_t)s * kSyncWords + kSyncWords - 1;
      const unsigned long long c = __hip_atomic_fetch_add(done, 1ull, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT);
      flag[1 + s - s_lo] = c + 1 == n_groups ? 1 : 0;
    }
  }
  __syncthreads();
  for (int s = s_lo; s <= s_hi; ++s) {
    if (flag[1 + s - s_lo]) {
      const int64_t lo = (int64_t)s * W, hi = (int64_t)(s + 1) * W;
      const int n_groups = (int)((hi - 1) / 4 - lo / 4 + 1);
      combine_slot(a.comb, s, a.group + (int64_t)s * a.group_stride * G * kPartFloats, n_groups);
      // every producer and attend workgroup of the slot is past its use of
      // the flags: clear them for a replay
      if (threadIdx.x < a.prod_per_slot)
        __hip_atomic_store(a.sync + (size_t)s * kSyncWords + threadIdx.x, 0ull, __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
    }
  }
}

static unsigned long long next_epoch() {
  // process-wide, distinct for 2^40 launches; the start is drawn at random so
  // that workspaces left by other processes hold other tags
  static std::atomic<unsigned long long> counter{0};
  static std::once_flag once;
  std::call_once(once, [] {
    std::random_device rd;
    const unsigned long long seed = ((unsigned long long)rd() << 32) ^ (unsigned long long)rd() ^
                                    (unsigned long long)std::chrono::steady_clock::now().time_since_epoch().count();
    counter.store(seed);
  });
  unsigned long long e;
  do {
    e = (counter.fetch_add(1) + 1) & ((1ull << 40) - 1);
  } while (e == 0);
  return e;
}

int launch_decode_step(const Matrices& mats, const CodebookDev& cbk, int kbits, const CodebookDev& cbv, int vbits,
                       int d, int m, const AppendShape& ks, const AppendShape& vs, const AttnShape& s,
                       void* key_records, void* value_blocks, float scale, float* out, void* ws, const AttnPlan& p,
                       void* stream) {
  if ((int64_t)(p.waves_per_slot / 4 + 2) * s.G > kStepMaxPartials) return TQ_EUNSUPPORTED;
  const WsPtrs w = ws_ptrs(ws, p);
  StepArgs a;
  a.prep = decode_args(mats, cbk, kbits, cbv, vbits, d, m, ks, vs, s, key_records, value_blocks, w.wq, w.wqn);
  a.att = attend_args(cbk, kbits, cbv, vbits, m, s, key_records, value_blocks, scale, w, p);
  a.comb = combine_args(mats, s, out, w, p);
  a.sync = w.sync;
  a.status = (uint32_t*)(w.sync + (size_t)kSyncWords * s.n_seq);
  a.fresh_from = ks.pos;
  a.epoch = next_epoch();
  a.group = w.group;
  a.group_stride = p.waves_per_slot / 4 + 2;
  const int np = a.prep.nk + a.prep.nv + s.n_seq * 16;
  a.n_prod = np;
  a.vblk_per_slot = a.prep.nv / s.n_seq;
  a.prod_per_slot = (int)ks.n_new + a.vblk_per_slot + 16;
  const int64_t waves = (int64_t)p.waves_per_slot * s.n_seq;
  const dim3 grid((unsigned)(np + (waves + 3) / 4)), block(256);
  const size_t lds = decode_lds_bytes(d, m);
  hipStream_t st = (hipStream_t)stream;
  bool launched = false;
#define TQ_DS(BK, BV, M)                                                                              \
  if (!launched && kbits == BK && vbits == BV && m == M) {                                            \
    if (s.G <= 4) hipLaunchKernelGGL((decode_step_kernel<BK, BV, M, 4>), grid, block, lds, st, a);      \
    else if (s.G <= 8) hipLaunchKernelGGL((decode_step_kernel<BK, BV, M, 2>), grid, block, lds, st, a); \
    else hipLaunchKernelGGL((decode_step_kernel<BK, BV, M, 1>), grid, block, lds, st, a);               \
    launched = true;                                                                                  \
  }
#define TQ_DS_V(BK, M) TQ_DS(BK, 1, M) TQ_DS(BK, 2, M) TQ_DS(BK, 3, M) TQ_DS(BK, 4, M)
  TQ_DS_V(0, 64) TQ_DS_V(1, 64) TQ_DS_V(2, 64) TQ_DS_V(3, 64) TQ_DS_V(4, 64)
  TQ_DS_V(0, 128) TQ_DS_V(1, 128) TQ_DS_V(2, 128) TQ_DS_V(3, 128) TQ_DS_V(4, 128)
#undef TQ_DS_V
#undef TQ_DS
  if (!launched) return TQ_EUNSUPPORTED;
  return hipGetLastError() == hipSuccess ? 0 : TQ_EDEVICE;
}

}  // namespace tq
