// Device code shared by the attention kernels (tq_attention.hip) and the
// fused decode step (tq_step.hip): key tiles and their decoding, the score
// kernel, the attend body with its hooks, and the host helpers that lay out
// the attention workspace.
#pragma once

#include <algorithm>
#include <type_traits>

#include "tq_device.h"

namespace tq {

constexpr int kPartFloats = 4 + kD;  // m, l, ve, pad, acc[d]
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

// Cache policy of the score kernel's record loads: each byte is read once,
// and nontemporal loads measured a few percent faster on this stream (the
// attend kernel, whose lanes read scattered words of lines other lanes also
// read, keeps the default policy).  The score stores keep the default
// policy: a wave writes 64-byte pieces of 16 head rows, and nontemporal
// stores of those moved 17% more bytes than they carry (WRITE_SIZE) for no
// gain in time.
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
          __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u4, v), ors, ob, 0, 0);
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
// under a workgroup barrier).  The hooks say where the query operands come
// from and where the partial goes:
//   prep()            called once by every wave (it may hold workgroup
//                     barriers) after the wave has issued the loads of its
//                     first key and value block and before it reads any
//                     query operand: the fused decode step prepares its
//                     queries there while those loads are in flight;
//   qop(slot, kb, l)  the fp16 B operand of K block kb for lane l;
//   qnorm(slot, i)    ||q|| of head lane i;
//   emit(slot, wc, h, q, m, l, ve, acc)  the partial of head h, called by
//                     the 4 lanes (q = 0..3) of the head's column.
// DEEP keeps the keys of all 4 steps of a block in flight at once (the
// decode step, one wave per SIMD and a block or two per wave, where the
// latency of each step's keys would otherwise add up); otherwise the keys
// are loaded one step ahead.
template <int BK, int BV, int M, int GC, bool DEEP, typename Prep, typename QOp, typename QNorm, typename Emit>
__device__ __forceinline__ void attend_body(const AttendArgs& a, int64_t gw, const Prep& prep, const QOp& qop,
                                            const QNorm& qnorm, const Emit& emit) {
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
    prep();
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
  constexpr int NK = DEEP ? 4 : 1;  // steps of keys held
  StepKeys<BK, BV, M> kq[NK];
  if (b_begin < b_end) {
    load_values(vcur, b_begin);
#pragma unroll
    for (int st = 0; st < NK; ++st) load_keys(kq[st], b_begin * kBlockTokens + 32 * st);
  }
  prep();
  h8 qb[KBT];
#pragma unroll
  for (int kb = 0; kb < KBT; ++kb) qb[kb] = qop(slot, kb, lane);
  if constexpr (KPT) {
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) qb[kb] = to_pair_order(qb[kb]);
  }
  const float qsc = qnorm(slot, r16 & (16 / GC - 1)) * a.scale2;
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
      StepKeys<BK, BV, M>& kcur = kq[DEEP ? step : 0];
      StepKeys<BK, BV, M> knext;
      if constexpr (!DEEP) {
        if (step < 3) load_keys(knext, tok0 + 32 * (step + 1));
        else if (more) load_keys(knext, tok0 + kBlockTokens);
      }
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
      if constexpr (DEEP) {
        if (more) load_keys(kcur, tok0 + kBlockTokens + 32 * step);  // this step of the next block
      } else {
        kcur = knext;
      }
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
  if (r16 < a.G) emit(slot, wc, r16, q, m_run, l_run, ve, acc);
}

// A partial in the layout [m, l, ve, pad, acc[128]] (acc column h of the
// wave's MFMA tiles: lane group q holds coordinates 16 nt + 4 q .. + 3).
__device__ __forceinline__ void store_partial(float* pr, int q, float m, float l, int ve, const f4 (&acc)[8]) {
  if (q == 0) {
    pr[0] = m;
    pr[1] = l;
    pr[2] = (float)ve;
  }
#pragma unroll
  for (int nt = 0; nt < 8; ++nt) *(f4*)(pr + 4 + 16 * nt + 4 * q) = acc[nt];
}

template <int BK, int BV, int M, int GC>
__global__ __launch_bounds__(256) void attend_kernel(const AttendArgs a) {
  constexpr int KBT = 4 + M / 32;
  attend_body<BK, BV, M, GC, false>(
      a, (int64_t)blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6), [] {},
      [&](int slot, int kb, int l) { return *(const h8*)(a.wq + (((int64_t)slot * KBT + kb) * 64 + l) * 8); },
      [&](int slot, int i) { return a.wqn[slot * 16 + i]; },
      [&](int slot, int wc, int h, int q, float m, float l, int ve, const f4 (&acc)[8]) {
        store_partial(a.part + (((int64_t)slot * a.waves_per_slot + wc) * a.G + h) * kPartFloats, q, m, l, ve, acc);
      });
}

// ---------------------------------------------------------------------------
// the attention workspace (host)
// ---------------------------------------------------------------------------

struct WsPtrs {
  uint16_t* wq;
  float* wqn;
  float* part;
  unsigned long long* sync;
  float* group;
};
// The decode step's arrival counts come first: the other regions move with
// the token count, but no call of this layout ever writes the counts' place.
inline WsPtrs ws_ptrs(void* ws, const AttnPlan& p) {
  char* b = (char*)ws;
  WsPtrs w;
  w.sync = (unsigned long long*)b;
  b += (p.sync_bytes + 255) / 256 * 256;
  w.wq = (uint16_t*)b;
  b += (p.q_bytes + 255) / 256 * 256;
  w.wqn = (float*)b;
  b += (p.qn_bytes + 255) / 256 * 256;
  w.part = (float*)b;
  b += (p.part_bytes + 255) / 256 * 256;
  w.group = (float*)b;
  return w;
}


inline void fill_tables(const CodebookDev& cb, uint32_t* tlo, uint32_t* thi) {
  for (int i = 0; i < 4; ++i) { tlo[i] = cb.tlo[i]; thi[i] = cb.thi[i]; }
}

inline AttendArgs attend_args(const CodebookDev& cbk, int kbits, const CodebookDev& cbv, int vbits, int m,
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

}  // namespace tq
