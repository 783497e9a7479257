// The whole decode step of a layer in one launch on gfx950 (tq_decode_step):
// the appends of the step's tokens, the query preparation, the attention
// over the cache and the merge of the partials, with no workgroup waiting for
// another (nav.superapi.store "turboquant-pytorch", 核心 API append_key /
// append_value and 常见使用模式 attention; the pages' streaming use, where
// each generated token is quantised as it arrives and attended at once:
// jansverre.net, Hva gjør Python-implementasjonen?).
#include <hip/hip_runtime.h>

#include "tq_attend.h"
#include "tq_small.h"

namespace tq {

// ---------------------------------------------------------------------------
// the fused decode step: appends, query preparation, attend and combine in
// one launch, with no workgroup waiting for another
// ---------------------------------------------------------------------------
//
// Workgroups (256 threads) per slot: n_plain attend workgroups, then one
// append workgroup.
//  * An attend workgroup takes 4 waves' ranges of the tokens before the
//    step (blocks_per_wave blocks each), exactly as the attend kernel does
//    with n_tokens = pos: the step's new tokens are not in its ranges, so it
//    reads nothing this launch writes.  It issues the loads of its first
//    block (all four steps' keys at once), prepares the slot's query
//    operands itself on the matrix cores (q~ = R q and p = (S R) q from the
//    split-fp16 images) while they are in flight, merges its waves'
//    partials in LDS and rotates the merged accumulator back (R^T on the
//    matrix cores) before writing one partial.
//  * The append workgroup compresses the step's tokens (stage 1 and 2 in
//    fp32 with R and S from L2, as the small appends do), writes their
//    records and value codes, and turns them into the softmax partial of the
//    new tokens directly: est = ||k|| (<q~, c[idx]> + gamma sqrt(pi/2)/m
//    <p, sign>), the estimator of the score kernels in fp32.
//  * Each workgroup adds 1 to its slot's arrival count after a release
//    fence; the one that completes the count merges the slot's n_plain + 1
//    partials (log-sum-exp with the value-norm exponents, as the combine
//    kernel) into the output and resets the count for the next launch.
// The count is a 64-bit word: a fixed 48-bit tag above a 16-bit count.  A
// word that is not of this form (a workspace never used by a decode step)
// is first set to (tag, 0) by compare-and-swap.  The counts sit at the start
// of the workspace, where no other call of the attention layout writes.
// (A word that holds the tag and a nonzero count by chance, odds 2^-48,
// would defeat this.)  Nothing else in the workspace needs clearing, and a
// replayed launch (a captured graph) finds the count reset.

constexpr unsigned long long kArriveTag = 0x7A3C5B1D96E4ull << 16;

// Dynamic LDS of the step kernel, in floats.
constexpr int kLdsQs = 0;                         // q shifted by 2^-e [16][128]; then merged accumulators
constexpr int kLdsQt = kLdsQs + 16 * kD;          // q~ = R q_shifted [16][128]; then per-head m, l, ve
constexpr int kLdsPp = kLdsQt + 16 * kD;          // p = S R q_shifted [16][128] (m <= 128)
constexpr int kLdsQn = kLdsPp + 16 * kD;          // ||q|| [16], shifted norms [16], exponents [16]
constexpr int kLdsOps = kLdsQn + 64;              // attend operands [KBT <= 8][64][8] fp16
constexpr int kLdsPm = kLdsOps + 8 * 64 * 8 / 2;  // wave partials [4][16][kPartFloats]; append scratch
constexpr int kLdsEnd = kLdsPm + 4 * 16 * kPartFloats;
constexpr size_t kStepLdsBytes = sizeof(float) * kLdsEnd;
static_assert(4 * kStepMaxPartials <= kLdsEnd, "the merge keeps every partial's header in LDS");

struct StepArgs {
  AttendArgs att;             // attention over tokens [0, pos): n_tokens = pos, waves_per_slot = 4 n_plain
  const uint16_t* r_hi;       // R * 2^8 hi / lo [128][kLdsStride]
  const uint16_t* r_lo;
  const uint16_t* rt_hi;      // R^T * 2^8 hi / lo
  const uint16_t* rt_lo;
  const uint16_t* p_hi;       // (S R) * 2^8 hi / lo [m][kLdsStride]
  const uint16_t* p_lo;
  const float* r32;           // R [128][128] fp32 (the appends)
  const float* s32;           // S [m][128] fp32
  const void* q;              // [n_seq][G][128]
  const void* k;              // new keys and values [n_seq][n_new][128]
  const void* v;
  uint32_t* rec;              // key records (as att.rec)
  uint32_t* vblk;             // value blocks (as att.vblocks)
  float* group;               // [n_seq][group_stride][G][kPartFloats] workgroup partials
  unsigned long long* count;  // [n_seq] arrival counts
  float* out;                 // [n_seq][G][128]
  int64_t pos, n_new;
  int dtype, n_plain, group_stride;
  float kbeta[16], kcent[16], vbeta[16], vcent[16];
};

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += shfl_xor(v, o);
  return v;
}

__device__ __forceinline__ float load_x(const void* p, int64_t i, int dtype) {
  return dtype == TQ_F32 ? ((const float*)p)[i] : (float)((const _Float16*)p)[i];
}

// 8 fp32 values as fp16 hi + lo operands (x = hi + lo to ~2^-22 relative
// for |x| < 1 and above the fp16 subnormals).
__device__ __forceinline__ void split8(const f4& x0, const f4& x1, h8& hi, h8& lo) {
  u4 h, l;
  HiLo t = split2(x0[0], x0[1]);
  h[0] = t.hi; l[0] = t.lo;
  t = split2(x0[2], x0[3]);
  h[1] = t.hi; l[1] = t.lo;
  t = split2(x1[0], x1[1]);
  h[2] = t.hi; l[2] = t.lo;
  t = split2(x1[2], x1[3]);
  h[3] = t.hi; l[3] = t.lo;
  hi = as_h8(h);
  lo = as_h8(l);
}

// The A operands of two 16-row tiles of an image (rows 16 (2 w + t) + r16,
// the 4 K steps, hi and lo), for wave w.
struct TileOps {
  h8 a[2][4][2];
};
__device__ __forceinline__ void load_tile_ops(TileOps& o, const uint16_t* hi, const uint16_t* lo, int wave, int lane) {
  const int r16 = lane & 15, q = lane >> 4;
#pragma unroll
  for (int t = 0; t < 2; ++t)
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      const int off = (16 * (2 * wave + t) + r16) * kLdsStride + 32 * ks + 8 * q;
      o.a[t][ks][0] = *(const h8*)(hi + off);
      o.a[t][ks][1] = *(const h8*)(lo + off);
    }
}

// The slot's query preparation by the whole workgroup on the matrix cores:
// per-head norms with a power-of-two shift (any finite query), then
// q~ = R q_shifted and p = (S R) q_shifted on the matrix cores (the fp16 hi
// images times q hi, + lo for fp32 queries), wave w forming rows 32 w .. +31
// of q~ and rows 16 (w + 4 u) .. of p for all 16 head lanes.  q~ and p go to
// LDS in fp32; with `plain` also the fp16 attend operands, the centroid
// part straight from the q~ tiles (their lane layout is the operand's).
template <int M>
__device__ __forceinline__ void step_prep(const StepArgs& a, int slot, float* L, bool plain) {
  constexpr int NP = M / 64;  // p tiles per wave
  constexpr int KBT = 4 + M / 32;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, r16 = lane & 15, q = lane >> 4, G = a.att.G;
  float* qs = L + kLdsQs;
  float* qt = L + kLdsQt;
  float* pp = L + kLdsPp;
  float* qn = L + kLdsQn;     // ||q|| per head lane (0 past G)
  float* qsn = qn + 16;       // norm of the shifted query
  int* qe = (int*)(qn + 32);  // its exponent
  uint16_t* ops = (uint16_t*)(L + kLdsOps);
  // image operands in flight first: the hi images only.  The query operands
  // are rounded to fp16 for the score products anyway, and R_hi q is within
  // ~2^-12 of R q, far inside the score tolerance (2e-3 of ||q|| ||k||);
  // the lo halves would double the bytes every workgroup loads before it
  // can start.
  h8 ra[2][4];
#pragma unroll
  for (int t = 0; t < 2; ++t)
#pragma unroll
    for (int ks = 0; ks < 4; ++ks)
      ra[t][ks] = *(const h8*)(a.r_hi + (16 * (2 * wave + t) + r16) * kLdsStride + 32 * ks + 8 * q);
  h8 pa[NP][4];
#pragma unroll
  for (int u = 0; u < NP; ++u)
#pragma unroll
    for (int ks = 0; ks < 4; ++ks)
      pa[u][ks] = *(const h8*)(a.p_hi + (16 * (wave + 4 * u) + r16) * kLdsStride + 32 * ks + 8 * q);
  // norms: thread (head h, seg) holds coordinates 8 seg .. + 7
  {
    const int h = tid >> 4, seg = tid & 15;
    float qv[8];
#pragma unroll
    for (int i = 0; i < 8; ++i)
      qv[i] = h < G ? load_x(a.q, ((int64_t)slot * G + h) * kD + 8 * seg + i, a.dtype) : 0.f;
    float mx = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) mx = fmaxf(mx, fabsf(qv[i]));
#pragma unroll
    for (int o = 1; o < 16; o <<= 1) mx = fmaxf(mx, shfl_xor(mx, o));
    const int e = pow2_exponent(mx);
    float ss = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      qv[i] = ldexpf(qv[i], -e);
      ss = fmaf(qv[i], qv[i], ss);
    }
    *(f4*)&qs[h * kD + 8 * seg] = f4{qv[0], qv[1], qv[2], qv[3]};
    *(f4*)&qs[h * kD + 8 * seg + 4] = f4{qv[4], qv[5], qv[6], qv[7]};
#pragma unroll
    for (int o = 1; o < 16; o <<= 1) ss += shfl_xor(ss, o);
    if (seg == 0) {
      qsn[h] = sqrtf(ss);
      qn[h] = h < G ? ldexpf(sqrtf(ss), e) : 0.f;
      qe[h] = e;
    }
  }
  __syncthreads();
  // B operands: head lane r16, K step ks = coordinates 32 ks + 8 q .. + 7
  h8 bh[4], bl[4];
#pragma unroll
  for (int ks = 0; ks < 4; ++ks)
    split8(*(const f4*)&qs[r16 * kD + 32 * ks + 8 * q], *(const f4*)&qs[r16 * kD + 32 * ks + 8 * q + 4], bh[ks],
           bl[ks]);
  const bool f32 = a.dtype == TQ_F32;  // (fp16 queries shifted by a power of two have no low part)
  f4 tq[2], tp[NP];
#pragma unroll
  for (int t = 0; t < 2; ++t) tq[t] = f4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int u = 0; u < NP; ++u) tp[u] = f4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) {
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      tq[t] = mfma(ra[t][ks], bh[ks], tq[t]);
      if (f32) tq[t] = mfma(ra[t][ks], bl[ks], tq[t]);
    }
#pragma unroll
    for (int u = 0; u < NP; ++u) {
      tp[u] = mfma(pa[u][ks], bh[ks], tp[u]);
      if (f32) tp[u] = mfma(pa[u][ks], bl[ks], tp[u]);
    }
  }
  const bool live = r16 < G;
  constexpr float kInvScale = 1.f / kRotScale;
#pragma unroll
  for (int t = 0; t < 2; ++t) tq[t] *= kInvScale;
#pragma unroll
  for (int u = 0; u < NP; ++u) tp[u] *= kInvScale;
  if (live) {
#pragma unroll
    for (int t = 0; t < 2; ++t) *(f4*)&qt[r16 * kD + 16 * (2 * wave + t) + 4 * q] = tq[t];
#pragma unroll
    for (int u = 0; u < NP; ++u) *(f4*)&pp[r16 * kD + 16 * (wave + 4 * u) + 4 * q] = tp[u];
  }
  if (plain) {
    // centroid operand of K block kb = wave: element e of lane 16 qq + h16 is
    // coordinate 32 kb + 16 (e / 4) + 4 qq + e % 4, i.e. tile 2 kb + e / 4, row 4 qq + e % 4
    const float inv = live && qsn[r16] > 0.f ? 1.f / qsn[r16] : 0.f;
    h8 v;
#pragma unroll
    for (int e = 0; e < 8; ++e) v[e] = (_Float16)(tq[e >> 2][e & 3] * inv);
    *(h8*)(ops + ((size_t)wave * 64 + lane) * 8) = v;
  }
  __syncthreads();
  if (plain) {
    // sign operands (layout of the query preparation kernels), from p in LDS
    for (int idx = tid; idx < (KBT - 4) * 64; idx += blockDim.x) {
      const int kbp = idx >> 6, l = idx & 63, qq = l >> 4, h16 = l & 15;
      const bool lv = h16 < G;
      const float inv = lv && qsn[h16] > 0.f ? 1.f / qsn[h16] : 0.f;
      h8 v;
#pragma unroll
      for (int e4 = 0; e4 < 4; ++e4)
#pragma unroll
        for (int half = 0; half < 2; ++half) {
          const int pe = 8 * (qq % 2) + 4 * (kbp % 2) + e4;
          const int t = 4 * (kbp / 2) + pe / 4, qsg = 2 * (qq / 2) + half;
          v[2 * e4 + half] = (_Float16)(lv ? pp[h16 * kD + 16 * t + 4 * qsg + pe % 4] * inv : 0.f);
        }
      *(h8*)(ops + ((size_t)(4 + kbp) * 64 + l) * 8) = v;
    }
    __syncthreads();
  }
}

// The workgroup's partial, rotated back on the matrix cores: out = R^T acc
// for the merged accumulators acc[h] (LDS [16][128], rotated domain, scaled
// into [-1, 1) by 2^-ve of the head), wave w forming coordinates
// 32 w .. + 31 of every head (R^T hi / lo x acc hi / lo, three products),
// written with the heads' (m, l, ve) as the slot's partial gi.
__device__ __forceinline__ void step_emit(const StepArgs& a, int slot, int gi, const float* acc, const float* hm,
                                          const float* hl, const int* hv, const TileOps& rt) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, r16 = lane & 15, q = lane >> 4, G = a.att.G;
  f4 o[2];
  o[0] = o[1] = f4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) {
    h8 bh, bl;
    split8(*(const f4*)&acc[r16 * kD + 32 * ks + 8 * q], *(const f4*)&acc[r16 * kD + 32 * ks + 8 * q + 4], bh, bl);
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      o[t] = mfma(rt.a[t][ks][0], bh, o[t]);
      o[t] = mfma(rt.a[t][ks][1], bh, o[t]);
      o[t] = mfma(rt.a[t][ks][0], bl, o[t]);
    }
  }
  if (r16 < G) {
    // written through to memory (cache policy sc0 sc1): the workgroup that
    // merges the slot may run on another XCD, and step_arrive then only
    // waits for these stores instead of writing back this XCD's L2
    // (the descriptor spans the partial's G heads: wave-uniform)
    constexpr int kSysCoherent = 1 | 16;
    const float* pg = a.group + ((int64_t)slot * a.group_stride + gi) * G * kPartFloats;
    const __amdgpu_buffer_rsrc_t prs = slot_rsrc(pg, 4u * (uint32_t)(G * kPartFloats));
    const uint32_t ph = 4u * (uint32_t)(r16 * kPartFloats);
#pragma unroll
    for (int t = 0; t < 2; ++t)
      __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u4, o[t] * (1.f / kRotScale)), prs,
                                             ph + 4u * (uint32_t)(4 + 16 * (2 * wave + t) + 4 * q), 0, kSysCoherent);
    if (wave == 0 && q == 0)
      __builtin_amdgcn_raw_buffer_store_b128(
          __builtin_bit_cast(u4, f4{hm[r16], hl[r16], (float)hv[r16], 0.f}), prs, ph, 0, kSysCoherent);
  }
}

// Per-head normalisation of a merged accumulator (thread (h, seg) holds
// coordinates 8 seg .. + 7 of head h in o): o scaled by 2^-ea, ea the
// exponent of the head's largest magnitude (so the split operands of the
// back-rotation stay in fp16 range), and the head's value exponent raised
// by ea.
__device__ __forceinline__ int normalise8(float (&o)[8]) {
  float mx = 0.f;
#pragma unroll
  for (int i = 0; i < 8; ++i) mx = fmaxf(mx, fabsf(o[i]));
#pragma unroll
  for (int s = 1; s < 16; s <<= 1) mx = fmaxf(mx, shfl_xor(mx, s));
  const int ea = pow2_exponent(mx);
#pragma unroll
  for (int i = 0; i < 8; ++i) o[i] = ldexpf(o[i], -ea);
  return ea;
}

// The merge of the slot's partials [gi][h][kPartFloats] (gi < n) into the
// output, by the workgroup that completed the slot's count.  Thread (h, j4)
// owns output coordinates 4 j4 .. 4 j4 + 3 of head h and merges every
// partial itself, kChunk at a time, carrying the running maximum, value
// exponent and sums from chunk to chunk (the softmax merge in its online
// form).  The partials' headers (m, l, ve) go to LDS once, and the loads of
// the first chunk's accumulator values are issued before them, so a slot of
// up to kChunk partials costs one round trip to memory.  The partials come
// from other XCDs: system-coherent loads (cache policy sc0 sc1) read them
// past this XCD's caches.
__device__ __forceinline__ void step_combine(const StepArgs& a, int slot, int n, float* L) {
  constexpr int kChunk = 24;
  constexpr int kSysCoherent = 1 | 16;
  const int G = a.att.G, tid = threadIdx.x;
  const float* gp = a.group + (int64_t)slot * a.group_stride * G * kPartFloats;
  const __amdgpu_buffer_rsrc_t prs = slot_rsrc(gp, (uint32_t)(n * G * kPartFloats * 4));
  auto ld4 = [&](int c, int h, int off) {
    return __builtin_bit_cast(
        f4, __builtin_amdgcn_raw_buffer_load_b128(prs, 4u * (uint32_t)((c * G + h) * kPartFloats + off), 0,
                                                  kSysCoherent));
  };
  f4* hdr = (f4*)L;  // [n][G] headers (n G <= kStepMaxPartials fits the step's LDS)
  const bool own0 = tid < G * (kD / 4);
  f4 av0[kChunk];    // this thread's first element, first chunk: in flight with the headers
#pragma unroll
  for (int u = 0; u < kChunk; ++u)
    av0[u] = own0 && u < n ? ld4(u, tid >> 5, 4 + 4 * (tid & 31)) : f4{0.f, 0.f, 0.f, 0.f};
  for (int i = tid; i < n * G; i += blockDim.x) hdr[i] = ld4(i / G, i % G, 0);
  __syncthreads();
  constexpr int kNoExp = -100000;  // value exponent before any partial with weight
  for (int e = tid; e < G * (kD / 4); e += blockDim.x) {
    const int h = e >> 5, j4 = e & 31;
    float M = -INFINITY, Lh = 0.f;
    int VE = kNoExp;
    f4 o = {0.f, 0.f, 0.f, 0.f};  // sum of weight x acc, in the scale 2^-VE
    for (int c0 = 0; c0 < n; c0 += kChunk) {
      f4 av[kChunk];
#pragma unroll
      for (int u = 0; u < kChunk; ++u)
        av[u] = e == tid && c0 == 0 ? av0[u]
                : c0 + u < n        ? ld4(c0 + u, h, 4 + 4 * j4)
                                    : f4{0.f, 0.f, 0.f, 0.f};
      float Mc = M;
      int Vc = VE;
#pragma unroll
      for (int u = 0; u < kChunk; ++u) {
        if (c0 + u < n) {
          const f4 hd = hdr[(c0 + u) * G + h];
          Mc = fmaxf(Mc, hd[0]);
          if (hd[0] != -INFINITY) Vc = max(Vc, (int)hd[2]);
        }
      }
      if (Mc == -INFINITY) continue;  // no partial with weight yet
      // the running sums move to the chunk's maximum and exponent
      const float f = M == -INFINITY ? 0.f : exp2f(M - Mc);
      Lh *= f;
      o *= ldexpf(f, max(VE - Vc, -1000));
#pragma unroll
      for (int u = 0; u < kChunk; ++u) {
        if (c0 + u < n) {
          const f4 hd = hdr[(c0 + u) * G + h];
          const float w = hd[0] == -INFINITY ? 0.f : exp2f(hd[0] - Mc);
          Lh = fmaf(w, hd[1], Lh);
          o += ldexpf(w, (int)hd[2] - Vc) * av[u];
        }
      }
      M = Mc;
      VE = Vc;
    }
    const float inv = Lh > 0.f ? 1.f / Lh : 0.f;
    f4 r;
#pragma unroll
    for (int i = 0; i < 4; ++i) r[i] = VE == kNoExp ? 0.f : ldexpf(o[i] * inv, VE);
    *(f4*)(a.out + ((int64_t)slot * G + h) * kD + 4 * j4) = r;
  }
}

// Arrival at the slot's count (after this workgroup's partial is written);
// true in the workgroup that completes it, whose reads then see every
// partial.  One fetch-and-add; a count without the tag (a workspace never
// used by a decode step) is first set to (tag, 0) by compare-and-swap and
// the arrival repeated.
__device__ __forceinline__ bool step_arrive(const StepArgs& a, int slot, int* flag) {
  // Every wave waits for its own partial stores (written through to memory
  // by step_emit) to complete before the barrier: a wait in one wave does
  // not cover the stores of the others.  The workgroups of a slot run on
  // different XCDs, each with an L2 of its own: the counts are only ever
  // read by atomics, and the merge reads the partials with system-coherent
  // loads, which bypass this XCD's caches.  Nothing else this launch writes
  // is read by another workgroup of it, so no L2 write-back is needed.
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_waitcnt(0);
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __syncthreads();
  if (threadIdx.x == 0) {
    unsigned long long* cnt = a.count + slot;
    // a count is (tag, n) with n below 2^16 (a slot has at most 4096
    // workgroups); anything else was never a count of this protocol
    auto valid = [](unsigned long long w) { return (w & ~0xFFFFull) == kArriveTag; };
    unsigned long long c = __hip_atomic_fetch_add(cnt, 1ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
    // A word that is not a count: start the count with (tag, 1) by
    // compare-and-swap, this workgroup being arrival 0, unless another
    // workgroup started it first (then arrive again).  Only atomics read
    // the word: they are performed where the adds are, while a load may be
    // served by a stale line in this XCD's cache.  (Bounded: the workgroups
    // of a slot settle this within a few tries.)
    unsigned long long expect = c + 1ull;  // the word as this add left it
    for (int tries = 0; !valid(c) && tries < 4096; ++tries) {
      unsigned long long seen = expect;
      if (__hip_atomic_compare_exchange_strong(cnt, &seen, kArriveTag | 1ull, __ATOMIC_RELAXED, __ATOMIC_RELAXED,
                                               __HIP_MEMORY_SCOPE_SYSTEM)) {
        c = kArriveTag;
      } else if (valid(seen)) {
        c = __hip_atomic_fetch_add(cnt, 1ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
        expect = c + 1ull;
      } else {
        expect = seen;  // the current value, from the failed compare-and-swap
      }
    }
    const bool last = (c & 0xFFFFull) == (unsigned long long)a.n_plain;
    if (last) {
      // the next launch's start
      (void)__hip_atomic_exchange(cnt, kArriveTag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
    }
    *flag = last ? 1 : 0;
  }
  __syncthreads();
  return *flag != 0;
}

// The append workgroup of a slot: the step's new tokens, one after the
// other (threads 0..127: key coordinate j, 128..255: value coordinate j),
// in fp32 with R and S from L2 (each thread's half row of R and its S rows
// loaded once), then their partial.
template <int BK, int BV, int M>
__device__ __forceinline__ void step_append(const StepArgs& a, int slot, float* L, const TileOps& rt) {
  constexpr int RW = rec_words<BK, M>();
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, G = a.att.G;
  const int j = tid & (kD - 1), hf = tid >> 7;
  const bool isv = tid >= kD;
  const float* qt = L + kLdsQt;
  const float* pp = L + kLdsPp;
  const int* qe = (const int*)(L + kLdsQn + 32);
  float* xs = L + kLdsPm;             // [2][128] shifted inputs
  float* yp = xs + 2 * kD;            // [2 halves][2 vectors][128] partial rows of R x
  float* rs = yp + 4 * kD;            // [128] key residual
  float* zs = rs + kD;                // [128] S r (m <= 128)
  int* kidx = (int*)(zs + kD);        // [128] key cells
  float* red = (float*)(kidx + kD);   // [16] reductions
  float* tn = red + 16;               // [4]: shifted norms of k, v
  int* te = (int*)(tn + 4);           // [4]: their exponents
  uint8_t* vcell = (uint8_t*)(te + 4);          // [16][128] value cells of the step's tokens
  float* vnorm = (float*)(vcell + 16 * kD);     // [16] value norms
  float* acc = vnorm + 16;                      // [16][128] the new tokens' accumulators (rotated domain)
  float* hm = acc + 16 * kD;                    // [16] per head: m, l, ve
  float* hl = hm + 16;
  int* hv = (int*)(hl + 16);
  __shared__ float kct[16], vct[16];  // centroids of the key and value codebooks
  if (tid < 16) {
    kct[tid] = a.kcent[tid];
    vct[tid] = a.vcent[tid];
  }
  float beta[15];
#pragma unroll
  for (int i = 0; i < 15; ++i) beta[i] = isv ? a.vbeta[i] : a.kbeta[i];
  // R: half row hf of row j; S: rows si + 64 u, columns 32 sc ..
  f4 rr[16];
#pragma unroll
  for (int u = 0; u < 16; ++u) rr[u] = *(const f4*)(a.r32 + (size_t)j * kD + 64 * hf + 4 * u);
  const int si = tid >> 2, sc = tid & 3;
  f4 sr[M / 64][8];
#pragma unroll
  for (int u = 0; u < M / 64; ++u)
#pragma unroll
    for (int e = 0; e < 8; ++e) sr[u][e] = *(const f4*)(a.s32 + (size_t)(si + 64 * u) * kD + 32 * sc + 4 * e);
  // per-head online softmax state: thread (h, seg) keeps coordinates 8 seg .. + 7
  const int h = tid >> 4, seg = tid & 15;
  float m_h = -INFINITY, l_h = 0.f, a8[8];
  int ve = -1000;
#pragma unroll
  for (int i = 0; i < 8; ++i) a8[i] = 0.f;
  const float kappa = a.att.kappa;
  float xn = load_x(isv ? a.v : a.k, ((int64_t)slot * a.n_new) * kD + j, a.dtype);
  for (int t = 0; t < (int)a.n_new; ++t) {
    float x = xn;
    if (t + 1 < (int)a.n_new) xn = load_x(isv ? a.v : a.k, ((int64_t)slot * a.n_new + t + 1) * kD + j, a.dtype);
    // norm with the power-of-two shift: two waves per vector
    float mx = wave_max(fabsf(x));
    if (lane == 0) red[wave] = mx;
    __syncthreads();
    mx = fmaxf(red[2 * isv], red[2 * isv + 1]);
    const int e = mx > 0.f ? pow2_exponent(mx) : 0;
    x = ldexpf(x, -e);
    const float s2 = wave_sum(x * x);
    if (lane == 0) red[8 + wave] = s2;
    xs[isv * kD + j] = x;
    __syncthreads();
    const float ns = sqrtf(red[8 + 2 * isv] + red[8 + 2 * isv + 1]);
    if (j == 0) {
      tn[isv] = ns;
      te[isv] = e;
    }
    // R x for both vectors: this thread's half row against each
    {
      float yk0 = 0.f, yk1 = 0.f, yv0 = 0.f, yv1 = 0.f;
#pragma unroll
      for (int u = 0; u < 16; u += 2) {
        const f4 xk0 = *(const f4*)&xs[64 * hf + 4 * u], xk1 = *(const f4*)&xs[64 * hf + 4 * u + 4];
        const f4 xv0 = *(const f4*)&xs[kD + 64 * hf + 4 * u], xv1 = *(const f4*)&xs[kD + 64 * hf + 4 * u + 4];
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          yk0 = fmaf(rr[u][c], xk0[c], yk0);
          yk1 = fmaf(rr[u + 1][c], xk1[c], yk1);
          yv0 = fmaf(rr[u][c], xv0[c], yv0);
          yv1 = fmaf(rr[u + 1][c], xv1[c], yv1);
        }
      }
      yp[(2 * hf) * kD + j] = yk0 + yk1;
      yp[(2 * hf + 1) * kD + j] = yv0 + yv1;
    }
    __syncthreads();
    const float y = yp[isv * kD + j] + yp[(2 + isv) * kD + j];
    const float u = ns > 0.f ? y / ns : 0.f;
    int idx = 0;
#pragma unroll
    for (int i = 0; i < 15; ++i) idx += beta[i] < u ? 1 : 0;
    float g2 = 0.f;
    if (!isv) {
      const float r = u - kct[idx];
      rs[j] = r;
      kidx[j] = idx;
      g2 = r * r;
    } else {
      vcell[t * kD + j] = (uint8_t)idx;
    }
    g2 = wave_sum(g2);
    if (lane == 0) red[4 + wave] = g2;
    __syncthreads();
    const float gamma = sqrtf(red[4] + red[5]);
    // z = S r: S row si + 64 u2 against the residual, quarters by lane exchange
#pragma unroll
    for (int u2 = 0; u2 < M / 64; ++u2) {
      float zz = 0.f;
#pragma unroll
      for (int e4 = 0; e4 < 8; ++e4) {
        const f4 rv = *(const f4*)&rs[32 * sc + 4 * e4];
        zz = fmaf(sr[u2][e4][0], rv[0], fmaf(sr[u2][e4][1], rv[1], fmaf(sr[u2][e4][2], rv[2], fmaf(sr[u2][e4][3], rv[3], zz))));
      }
      zz += shfl_xor(zz, 1);
      zz += shfl_xor(zz, 2);
      if (sc == 0) zs[si + 64 * u2] = zz;
    }
    __syncthreads();
    const float kn = ldexpf(tn[0], te[0]);
    // the key record (layout v2, as the small appends write it)
    uint32_t* rec = a.rec + ((int64_t)slot * a.att.capacity + a.pos + t) * RW;
    {
      constexpr int code_words = BK * kD / 32;
      const int wi = tid >> 3, sl = tid & 7;
      uint32_t part = 0u;
      if (wi < code_words) {
        const int grp = wi / (BK > 0 ? BK : 1), w = wi % (BK > 0 ? BK : 1);
#pragma unroll
        for (int i = 0; i < 4; ++i) part |= code_bits(BK, w, sl, i, (uint32_t)kidx[16 * sl + 4 * grp + i]);
      }
      part |= __shfl_xor(part, 1, 64);
      part |= __shfl_xor(part, 2, 64);
      part |= __shfl_xor(part, 4, 64);
      if (wi < code_words && sl == 0) rec[wi] = part;
      // sign words: projection 16 tt + 4 q + i is bit 16 (q%2) + 4 (tt%4) + i of word 2 (tt/4) + q/2
      const int sw = tid >> 5, bit = tid & 31;
      bool on = false;
      if (sw < M / 32) {
        const int hb = bit >> 4, tt = 4 * (sw >> 1) + ((bit >> 2) & 3), q = 2 * (sw & 1) + hb, i = bit & 3;
        on = zs[16 * tt + 4 * q + i] >= 0.f;
      }
      const uint64_t mask = __ballot(on);
      if (sw < M / 32 && bit == 0) rec[code_words + sw] = (uint32_t)(mask >> (tid & 32));
      if (tid == 0) {
        rec[RW - 2] = __float_as_uint(kn);
        rec[RW - 1] = __float_as_uint(gamma);
      }
    }
    // the token's share of each head's softmax:
    // est = ||k|| 2^e_q (<q~, c[idx]> + gamma sqrt(pi/2)/m <p, 2s - 1>)
    {
      float d1 = 0.f, d2 = 0.f;
      if (h < G) {
#pragma unroll
        for (int i = 0; i < 8; ++i) d1 = fmaf(qt[h * kD + 8 * seg + i], kct[kidx[8 * seg + i]], d1);
#pragma unroll
        for (int i = 0; i < M / 16; ++i) {
          const int pi = (M / 16) * seg + i;
          d2 += zs[pi] >= 0.f ? pp[h * kD + pi] : -pp[h * kD + pi];
        }
      }
#pragma unroll
      for (int o = 1; o < 16; o <<= 1) {
        d1 += shfl_xor(d1, o);
        d2 += shfl_xor(d2, o);
      }
      const float vn = ldexpf(tn[1], te[1]);
      if (tid == 0) vnorm[t] = vn;
      if (h < G) {
        const float logit = ldexpf(kn * fmaf(gamma * kappa, d2, d1), qe[h]) * a.att.scale2;
        int e_blk = 0;
        frexpf(vn, &e_blk);
        if (vn > 0.f && e_blk > ve) {
          const float f = ldexpf(1.f, ve - e_blk);
#pragma unroll
          for (int i = 0; i < 8; ++i) a8[i] *= f;
          ve = e_blk;
        }
        const float m_new = fmaxf(m_h, logit);
        const float alpha = m_h == -INFINITY ? 0.f : exp2f(m_h - m_new);
        const float p = exp2f(logit - m_new);
        const float pv = p * ldexpf(vn, -ve);
#pragma unroll
        for (int i = 0; i < 8; ++i) a8[i] = fmaf(a8[i], alpha, pv * vct[vcell[t * kD + 8 * seg + i]]);
        l_h = fmaf(l_h, alpha, p);
        m_h = m_new;
      }
    }
    __syncthreads();  // before the next token re-uses xs, yp, rs, zs, kidx, red
  }
  // value codes: the words of the touched blocks that hold a code of a new
  // token are read together, merged and written back (one thread a word)
  {
    constexpr int BWV = 4 * BV * kD + kBlockTokens;
    constexpr int NWV = (4 * BV * kD + 255) / 256;
    const int64_t blk0 = a.pos / kBlockTokens, blk1 = (a.pos + a.n_new - 1) / kBlockTokens;
    for (int64_t blk = blk0; blk <= blk1; ++blk) {
      uint32_t* vb = a.vblk + ((int64_t)slot * (a.att.capacity / kBlockTokens) + blk) * BWV;
      const int64_t t_lo = max(a.pos, blk * kBlockTokens), t_hi = min(a.pos + a.n_new, (blk + 1) * kBlockTokens);
      uint32_t keep[NWV], bits[NWV], old[NWV];
#pragma unroll
      for (int k = 0; k < NWV; ++k) {
        const int e = tid + 256 * k;
        keep[k] = 0xFFFFFFFFu;
        bits[k] = 0u;
        if (e < 4 * BV * kD) {
          const int c = e % kD, wq = e / kD, q = wq % 4, w = wq / 4;
          for (int64_t tk = t_lo; tk < t_hi; ++tk) {
            const int tau = (int)(tk - blk * kBlockTokens);
            if (((tau >> 2) & 3) != q) continue;
            const int sl = tau >> 4, i = tau & 3;
            keep[k] &= ~code_mask(BV, w, sl, i);
            bits[k] |= code_bits(BV, w, sl, i, (uint32_t)vcell[(tk - a.pos) * kD + c]);
          }
        }
        old[k] = keep[k] != 0xFFFFFFFFu ? vb[e] : 0u;
      }
#pragma unroll
      for (int k = 0; k < NWV; ++k)
        if (keep[k] != 0xFFFFFFFFu) vb[tid + 256 * k] = (old[k] & keep[k]) | bits[k];
      float* vn = (float*)(vb + 4 * BV * kD);
      if (tid >= t_lo - a.pos && tid < t_hi - a.pos) vn[(int)(a.pos + tid - blk * kBlockTokens)] = vnorm[tid];
    }
  }
  // the new tokens' partial per head, rotated back
  if (h < G) {
    const int ea = normalise8(a8);
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[h * kD + 8 * seg + i] = a8[i];
    if (seg == 0) {
      hm[h] = m_h;
      hl[h] = l_h;
      hv[h] = ve + ea;
    }
  }
  __syncthreads();
  step_emit(a, slot, a.n_plain, acc, hm, hl, hv, rt);
}

template <int BK, int BV, int M, int GC>
__global__ __launch_bounds__(256, 1) void decode_step_kernel(const StepArgs a) {
  extern __shared__ __align__(16) float L[];
  __shared__ int flag;
  const int per = a.n_plain + 1;
  const int slot = (int)blockIdx.x / per, r = (int)blockIdx.x % per;
  const int tid = threadIdx.x, wave = tid >> 6, G = a.att.G;
  if (r == a.n_plain) {
    step_prep<M>(a, slot, L, false);
    TileOps rt;
    load_tile_ops(rt, a.rt_hi, a.rt_lo, wave, tid & 63);
    step_append<BK, BV, M>(a, slot, L, rt);
  } else {
    float* pm = L + kLdsPm;
    const uint16_t* ops = (const uint16_t*)(L + kLdsOps);
    const float* qn = L + kLdsQn;
    attend_body<BK, BV, M, GC, true>(
        a.att, (int64_t)slot * a.att.waves_per_slot + 4 * r + wave, [&] { step_prep<M>(a, slot, L, true); },
        [&](int, int kb, int l) { return *(const h8*)(ops + ((size_t)kb * 64 + l) * 8); },
        [&](int, int i) { return qn[i]; },
        [&](int, int, int h, int q, float m, float l, int ve, const f4 (&acc)[8]) {
          store_partial(pm + (wave * 16 + h) * kPartFloats, q, m, l, ve, acc);
        });
    TileOps rt;  // R^T operands, in flight during the merge
    load_tile_ops(rt, a.rt_hi, a.rt_lo, wave, tid & 63);
    __syncthreads();
    // merge the 4 waves' partials of each head: thread (h, seg), coordinates 8 seg ..
    float* acc = L + kLdsQs;
    float* hm = L + kLdsQt;  // (q~ is no longer read)
    float* hl = hm + 16;
    int* hv = (int*)(hl + 16);
    const int h = tid >> 4, seg = tid & 15;
    if (h < G) {
      float M_ = -INFINITY, VE = -INFINITY;
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        const float mw = pm[(w * 16 + h) * kPartFloats];
        M_ = fmaxf(M_, mw);
        if (mw != -INFINITY) VE = fmaxf(VE, pm[(w * 16 + h) * kPartFloats + 2]);
      }
      const int ve = VE == -INFINITY ? -1000 : (int)VE;
      float Lh = 0.f, o[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) o[i] = 0.f;
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        const float* p = pm + (w * 16 + h) * kPartFloats;
        const float e2 = p[0] == -INFINITY ? 0.f : exp2f(p[0] - M_);
        Lh = fmaf(e2, p[1], Lh);
        const float f = ldexpf(e2, (int)p[2] - ve);
#pragma unroll
        for (int i = 0; i < 8; ++i) o[i] = fmaf(f, p[4 + 8 * seg + i], o[i]);
      }
      const int ea = normalise8(o);
#pragma unroll
      for (int i = 0; i < 8; ++i) acc[h * kD + 8 * seg + i] = o[i];
      if (seg == 0) {
        hm[h] = M_;
        hl[h] = Lh;
        hv[h] = ve + ea;
      }
    }
    __syncthreads();
    step_emit(a, slot, r, acc, hm, hl, hv, rt);
  }
  if (step_arrive(a, slot, &flag)) step_combine(a, slot, per, L);
}

// Query preparation for the attend kernel on the single-kernel shapes: one
// workgroup per slot runs the decode step's preparation (the fp16 hi images
// on the matrix cores; the attend operands are fp16, so R_hi q, within
// ~2^-12 of R q, loses nothing they keep) and writes the operands and norms
// where the attend kernel reads them ([n_seq][KBT][64][8] fp16, [n_seq][16]).
template <int M>
__global__ __launch_bounds__(256) void prep_step_kernel(const StepArgs a, uint16_t* wq, float* wqn) {
  extern __shared__ __align__(16) float L[];
  constexpr int KBT = 4 + M / 32;
  const int slot = blockIdx.x;
  step_prep<M>(a, slot, L, true);  // (ends with a barrier: operands and norms complete)
  const u4* ops = (const u4*)(L + kLdsOps);
  u4* dst = (u4*)(wq + (int64_t)slot * KBT * 64 * 8);
  for (int i = threadIdx.x; i < KBT * 64; i += blockDim.x) dst[i] = ops[i];
  if (threadIdx.x < 16) wqn[(int64_t)slot * 16 + threadIdx.x] = L[kLdsQn + threadIdx.x];
}

int launch_prep_step(const Matrices& mats, int m, const AttnShape& s, uint16_t* wq, float* wqn, void* stream) {
  StepArgs a{};
  a.att.G = s.G;
  a.q = s.q;
  a.dtype = s.dtype;
  a.r_hi = mats.r_hi;
  a.p_hi = mats.p_hi;
  if (!a.r_hi || !a.p_hi) return TQ_EUNSUPPORTED;
  const dim3 grid((unsigned)s.n_seq), block(256);
  const size_t lds = sizeof(float) * kLdsPm;  // query, q~, p, norms, operands
  hipStream_t st = (hipStream_t)stream;
  if (m == 64) hipLaunchKernelGGL(prep_step_kernel<64>, grid, block, lds, st, a, wq, wqn);
  else if (m == 128) hipLaunchKernelGGL(prep_step_kernel<128>, grid, block, lds, st, a, wq, wqn);
  else return TQ_EUNSUPPORTED;
  return hipGetLastError() == hipSuccess ? 0 : TQ_EDEVICE;
}

int launch_decode_step(const Matrices& mats, const CodebookDev& cbk, int kbits, const CodebookDev& cbv, int vbits,
                       int d, int m, const AppendShape& ks, const AppendShape& vs, const AttnShape& s,
                       void* key_records, void* value_blocks, float scale, float* out, void* ws, const AttnPlan& p,
                       void* stream) {
  (void)d;
  (void)vs;
  const WsPtrs w = ws_ptrs(ws, p);
  // attend workgroups of 4 waves over the tokens before the step, with the
  // plan's blocks per wave (its workgroup-partial room holds them and the
  // append workgroup's)
  const int64_t nblk_old = (ks.pos + kBlockTokens - 1) / kBlockTokens;
  const int bpw = p.blocks_per_wave;
  const int n_plain = (int)std::max<int64_t>(1, (nblk_old + 4 * bpw - 1) / (4 * bpw));
  const int group_stride = p.waves_per_slot / 4 + 2;
  if (n_plain + 1 > group_stride || (int64_t)(n_plain + 1) * s.G > kStepMaxPartials) return TQ_EUNSUPPORTED;
  StepArgs a;
  AttnShape so = s;
  so.n_tokens = ks.pos;
  a.att = attend_args(cbk, kbits, cbv, vbits, m, so, key_records, value_blocks, scale, w, p);
  a.att.waves_per_slot = 4 * n_plain;
  a.att.blocks_per_wave = bpw;
  a.r_hi = mats.r_hi;
  a.r_lo = mats.r_lo;
  a.rt_hi = mats.rt_hi;
  a.rt_lo = mats.rt_lo;
  a.p_hi = mats.p_hi;
  a.p_lo = mats.p_lo;
  a.r32 = mats.r32;
  a.s32 = mats.s32;
  if (!a.rt_hi || !a.p_hi) return TQ_EUNSUPPORTED;
  a.q = s.q;
  a.k = ks.x;
  a.v = vs.x;
  a.rec = (uint32_t*)key_records;
  a.vblk = (uint32_t*)value_blocks;
  a.group = w.group;
  a.count = w.sync;
  a.out = out;
  a.pos = ks.pos;
  a.n_new = ks.n_new;
  a.dtype = ks.dtype;
  a.n_plain = n_plain;
  a.group_stride = group_stride;
  for (int i = 0; i < 16; ++i) {
    a.kbeta[i] = cbk.beta[i];
    a.kcent[i] = cbk.cent[i];
    a.vbeta[i] = cbv.beta[i];
    a.vcent[i] = cbv.cent[i];
  }
  const dim3 grid((unsigned)(s.n_seq * (n_plain + 1))), block(256);
  hipStream_t st = (hipStream_t)stream;
  bool launched = false;
#define TQ_DS(BK, BV, M)                                                                                        \
  if (!launched && kbits == BK && vbits == BV && m == M) {                                                      \
    if (s.G <= 4) hipLaunchKernelGGL((decode_step_kernel<BK, BV, M, 4>), grid, block, kStepLdsBytes, st, a);      \
    else if (s.G <= 8) hipLaunchKernelGGL((decode_step_kernel<BK, BV, M, 2>), grid, block, kStepLdsBytes, st, a); \
    else hipLaunchKernelGGL((decode_step_kernel<BK, BV, M, 1>), grid, block, kStepLdsBytes, st, a);               \
    launched = true;                                                                                            \
  }
#define TQ_DS_V(BK, M) TQ_DS(BK, 1, M) TQ_DS(BK, 2, M) TQ_DS(BK, 3, M) TQ_DS(BK, 4, M)
  TQ_DS_V(0, 64) TQ_DS_V(1, 64) TQ_DS_V(2, 64) TQ_DS_V(3, 64) TQ_DS_V(4, 64)
  TQ_DS_V(0, 128) TQ_DS_V(1, 128) TQ_DS_V(2, 128) TQ_DS_V(3, 128) TQ_DS_V(4, 128)
#undef TQ_DS_V
#undef TQ_DS
  if (!launched) return TQ_EUNSUPPORTED;
  return hipGetLastError() == hipSuccess ? 0 : TQ_EDEVICE;
}

// The step kernel's dynamic LDS (above the 64 KB default), set once.
int decode_step_device_init() {
  int rc = 0;
#define TQ_DSA1(BK, BV, M, GC)                                                                     \
  rc |= hipFuncSetAttribute((const void*)decode_step_kernel<BK, BV, M, GC>,                        \
                            hipFuncAttributeMaxDynamicSharedMemorySize, (int)kStepLdsBytes);
#define TQ_DSA(BK, BV, M) TQ_DSA1(BK, BV, M, 1) TQ_DSA1(BK, BV, M, 2) TQ_DSA1(BK, BV, M, 4)
#define TQ_DSA_V(BK, M) TQ_DSA(BK, 1, M) TQ_DSA(BK, 2, M) TQ_DSA(BK, 3, M) TQ_DSA(BK, 4, M)
  TQ_DSA_V(0, 64) TQ_DSA_V(1, 64) TQ_DSA_V(2, 64) TQ_DSA_V(3, 64) TQ_DSA_V(4, 64)
  TQ_DSA_V(0, 128) TQ_DSA_V(1, 128) TQ_DSA_V(2, 128) TQ_DSA_V(3, 128) TQ_DSA_V(4, 128)
#undef TQ_DSA_V
#undef TQ_DSA
#undef TQ_DSA1
  return rc == hipSuccess ? 0 : -1;
}

}  // namespace tq
