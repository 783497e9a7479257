// C ABI of libtq.so: argument checking, context set-up and launch dispatch.
// Every argument is checked on the host before any HIP call, so errors never
// reach the device and never leave partial writes.
#include <hip/hip_runtime_api.h>

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <mutex>
#include <vector>

#include "tq_internal.h"

namespace tq {

static thread_local char g_err[512] = "";

int fail(int code, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return code;
}

void clear_error() { g_err[0] = 0; }

// Round to the nearest fp16 (ties to even), returned as raw bits.
static uint16_t to_half_bits(float f) {
  _Float16 h = (_Float16)f;
  uint16_t b;
  std::memcpy(&b, &h, 2);
  return b;
}
static float half_to_float(uint16_t b) {
  _Float16 h;
  std::memcpy(&h, &b, 2);
  return (float)h;
}

static bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

// Shape checks shared by tq_create and the size queries.  Returns TQ_OK,
// TQ_EINVAL or TQ_EUNSUPPORTED.
static int check_config(const tq_config* c) {
  if (!c) return fail(TQ_EINVAL, "config is NULL");
  if (c->head_dim < 64 || c->head_dim > 1024 || c->head_dim % 64)
    return fail(TQ_EINVAL, "head_dim %d: need a multiple of 64 in [64, 1024]", c->head_dim);
  if (c->proj_dim < 32 || c->proj_dim > 512 || c->proj_dim % 32)
    return fail(TQ_EINVAL, "proj_dim %d: need a multiple of 32 in [32, 512]", c->proj_dim);
  if (c->key_bits < 0 || c->key_bits > 4 || c->value_bits < 1 || c->value_bits > 4)
    return fail(TQ_EINVAL, "key_bits %d / value_bits %d: need 0..4 / 1..4", c->key_bits, c->value_bits);
  return TQ_OK;
}

// Shapes with the single-kernel compress / attention path; every other valid
// shape runs on the general path (tq_general.hip).  Keys of 0 bits (signs
// and norms only) are compressed by the 32 x 32-tile or the small kernel
// (tq_append_key) and scored and attended on the single-kernel path.
static bool fast_shape(const tq_config& c) { return c.head_dim == kD && (c.proj_dim == 64 || c.proj_dim == 128); }
static bool fast_keys(const tq_config& c) { return fast_shape(c) && c.key_bits > 0; }
static bool fast_values(const tq_config& c) { return c.head_dim == kD; }
static bool fast_attn(const tq_config& c, int G) { return fast_shape(c) && G <= 16; }
constexpr int64_t kScratchRows = 32768;  // general-path rows per launch

// 128-coordinate chunks and 64-projection tiles of the general path (the
// last one possibly half full).
static int key_chunks(int d) { return (d + 127) / 128; }
static int sign_blocks(int m) { return (m + 63) / 64; }

static size_t key_rec_bytes(const tq_config& c) { return 4u * (c.key_bits * c.head_dim / 32 + c.proj_dim / 32 + 2); }
static size_t val_blk_bytes(const tq_config& c) { return 4u * (4 * c.value_bits * c.head_dim + kBlockTokens); }

}  // namespace tq

using namespace tq;

struct tq_ctx {
  tq_config cfg;
  int device;
  void* dev_mem;       // one allocation holding every device image below (and the general-path scratch)
  Matrices mats;
  GenMats gen;         // general path: the same images plus scratch
  CodebookDev cb[5];   // indexed by bits
  bool loaded[5];
};

static std::once_flag g_init_flag;
static int g_init_rc = 0;

extern "C" {

const char* tq_last_error(void) { return g_err; }

size_t tq_config_key_record_bytes(const tq_config* cfg) {
  if (check_config(cfg) == TQ_EINVAL) return 0;
  return key_rec_bytes(*cfg);
}

size_t tq_value_block_bytes(const tq_config* cfg) {
  if (check_config(cfg) == TQ_EINVAL) return 0;
  return val_blk_bytes(*cfg);
}

size_t tq_cache_key_bytes(const tq_config* cfg, int32_t n_seq, int64_t capacity) {
  if (check_config(cfg) == TQ_EINVAL || n_seq < 1 || capacity < 1 || capacity % kBlockTokens) return 0;
  return key_rec_bytes(*cfg) * (size_t)n_seq * (size_t)capacity;
}

size_t tq_cache_value_bytes(const tq_config* cfg, int32_t n_seq, int64_t capacity) {
  if (check_config(cfg) == TQ_EINVAL || n_seq < 1 || capacity < 1 || capacity % kBlockTokens) return 0;
  return val_blk_bytes(*cfg) * (size_t)n_seq * (size_t)(capacity / kBlockTokens);
}

size_t tq_workspace_bytes(const tq_config* cfg, int32_t n_seq, int32_t G, int64_t n_tokens) {
  if (check_config(cfg) == TQ_EINVAL || n_seq < 1 || G < 1 || G > kMaxGeneralHeads || n_tokens < 1) return 0;
  if (fast_attn(*cfg, G)) return plan_attention(cfg->proj_dim, n_seq, G, n_tokens).total;
  if (G <= 16) return general_attend_plan(cfg->head_dim, cfg->proj_dim, n_seq, G, n_tokens).total;
  return general_scores_workspace(cfg->head_dim, cfg->proj_dim, n_seq, G);
}

size_t tq_key_record_bytes(const tq_ctx* ctx) { return ctx ? key_rec_bytes(ctx->cfg) : 0; }

size_t tq_value_record_bytes(const tq_ctx* ctx) { return ctx ? val_blk_bytes(ctx->cfg) / kBlockTokens : 0; }

size_t tq_attend_workspace_bytes(const tq_ctx* ctx, int32_t n_seq, int32_t G, int64_t n_tokens) {
  return ctx ? tq_workspace_bytes(&ctx->cfg, n_seq, G, n_tokens) : 0;
}

int tq_create(const tq_config* cfg, const double* R, const double* S, tq_ctx** out) {
  clear_error();
  if (!out) return fail(TQ_EINVAL, "tq_create: out is NULL");
  *out = nullptr;
  int rc = check_config(cfg);
  if (rc != TQ_OK) return rc;
  if (!R || !S) return fail(TQ_EINVAL, "tq_create: R or S is NULL");
  const int d = cfg->head_dim, m = cfg->proj_dim;
  for (size_t i = 0; i < (size_t)d * d; ++i)
    if (!std::isfinite(R[i])) return fail(TQ_EINVAL, "tq_create: R has a non-finite entry");
  for (size_t i = 0; i < (size_t)m * d; ++i)
    if (!std::isfinite(S[i])) return fail(TQ_EINVAL, "tq_create: S has a non-finite entry");

  // Host images.  R and S are scaled by 2^8 and split into fp16 high and low
  // parts (hi = fp16(x), lo = fp16(x - hi)), so hi + lo carries ~22 bits.
  // Rows are padded to ld = d + 8 halves.  S's columns are stored in "slot
  // order" per 128-coordinate chunk: column 128 u + 32 kb + 8 q + e holds
  // rotated coordinate 128 u + 16 (2 kb + e/4) + 4 q + e%4, the order in which
  // a key lane holds its residual after the rotation.
  // The d = 128 key kernel built on 32 x 32 matrix-core tiles holds its
  // residual in another order and takes a second copy of S: column
  // 16 kk + 8 g + e holds coordinate 16 kk + 8 (e/4) + 4 g + e%4 (bits 2 and
  // 3 of the coordinate swapped).
  // The images have d rounded up to 128 rows (R) and m rounded up to 64 rows
  // (S), the extra rows zero: the general-path kernels work on whole 128-
  // coordinate chunks and 64-projection tiles, and a zero row gives a zero
  // coordinate that is never stored.
  const int ld = d + 8;
  const size_t r_img = (size_t)(128 * key_chunks(d)) * ld, s_img = (size_t)(64 * sign_blocks(m)) * ld;
  std::vector<uint16_t> rh(r_img, 0), rl(r_img, 0), sh(s_img, 0), sl(s_img, 0), sh32(s_img, 0), sl32(s_img, 0);
  std::vector<float> r32((size_t)d * d), s32((size_t)m * d);
  auto split = [](double x, uint16_t& hi, uint16_t& lo) {
    const double xs = x * (double)kRotScale;
    hi = to_half_bits((float)xs);
    lo = to_half_bits((float)(xs - (double)half_to_float(hi)));
  };
  for (int i = 0; i < d; ++i)
    for (int k = 0; k < d; ++k) {
      split(R[(size_t)i * d + k], rh[(size_t)i * ld + k], rl[(size_t)i * ld + k]);
      r32[(size_t)i * d + k] = (float)R[(size_t)i * d + k];
    }
  // The fused decode step (head_dim 128 with proj_dim 64 or 128) prepares
  // its queries and rotates its partials back on the matrix cores: R^T and
  // P = S R (the query's projection p = S R q in one product) as the same
  // scaled hi / lo fp16 images, P formed in fp64.
  const bool step_imgs = fast_shape(*cfg);
  const size_t t_img = step_imgs ? (size_t)d * ld : 0, p_img = step_imgs ? (size_t)m * ld : 0;
  std::vector<uint16_t> rth(t_img, 0), rtl(t_img, 0), ph(p_img, 0), pl(p_img, 0);
  if (step_imgs) {
    for (int i = 0; i < d; ++i)
      for (int k = 0; k < d; ++k) split(R[(size_t)k * d + i], rth[(size_t)i * ld + k], rtl[(size_t)i * ld + k]);
    std::vector<double> P((size_t)m * d, 0.0);
    for (int i = 0; i < m; ++i)
      for (int j = 0; j < d; ++j) {
        const double sij = S[(size_t)i * d + j];
        for (int k = 0; k < d; ++k) P[(size_t)i * d + k] += sij * R[(size_t)j * d + k];
      }
    for (int i = 0; i < m; ++i)
      for (int k = 0; k < d; ++k) split(P[(size_t)i * d + k], ph[(size_t)i * ld + k], pl[(size_t)i * ld + k]);
  }
  for (int i = 0; i < m; ++i) {
    for (int col = 0; col < d; ++col) {
      const int u = col / 128, c = col % 128, kb = c / 32, q = (c % 32) / 8, e = c % 8;
      const int coord = 128 * u + 16 * (2 * kb + e / 4) + 4 * q + e % 4;
      split(S[(size_t)i * d + coord], sh[(size_t)i * ld + col], sl[(size_t)i * ld + col]);
    }
    for (int k = 0; k < d; ++k) s32[(size_t)i * d + k] = (float)S[(size_t)i * d + k];
    for (int col = 0; col < d; ++col) {
      const int coord = (col & ~12) | ((col & 4) << 1) | ((col & 8) >> 1);
      split(S[(size_t)i * d + coord], sh32[(size_t)i * ld + col], sl32[(size_t)i * ld + col]);
    }
  }

  std::call_once(g_init_flag, [] { g_init_rc = compress_device_init() | attention_device_init() | dequant_device_init() |
                                     topk_device_init() | small_device_init(); });
  if (g_init_rc != 0) return fail(TQ_EDEVICE, "tq_create: HIP device initialisation failed");

  tq_ctx* c = new tq_ctx();
  c->cfg = *cfg;
  if (hipGetDevice(&c->device) != hipSuccess) {
    delete c;
    return fail(TQ_EDEVICE, "tq_create: hipGetDevice failed");
  }
  // set-up of tq_attend_noalloc's scratch on this device (once per device)
  if (noalloc_scratch_init(c->device) != 0) {
    delete c;
    return fail(TQ_EDEVICE, "tq_create: device address of the no-allocation scratch not found");
  }
  const size_t b_rimg = r_img * 2, b_simg = s_img * 2;
  const size_t off_rl = b_rimg, off_sh = 2 * b_rimg, off_sl = off_sh + b_simg, off_sh32 = off_sl + b_simg;
  const size_t off_sl32 = off_sh32 + b_simg, off_r32 = off_sl32 + b_simg;
  const size_t off_s32 = off_r32 + r32.size() * 4, off_rth = off_s32 + s32.size() * 4;
  const size_t off_rtl = off_rth + t_img * 2, off_ph = off_rtl + t_img * 2, off_pl = off_ph + p_img * 2;
  const size_t end_imgs = off_pl + p_img * 2;
  // general-path scratch (row norms, key residual hi/lo, residual square sums)
  const bool gen = (!fast_keys(*cfg) && cfg->key_bits > 0) || !fast_values(*cfg);
  const int64_t srows = gen ? kScratchRows : 0;
  auto up = [](size_t x) { return (x + 255) / 256 * 256; };
  const size_t off_nrm = up(end_imgs), off_rh = off_nrm + up((size_t)srows * 8);  // (norm, exponent) pairs
  const size_t off_rlo = off_rh + up((size_t)srows * d * 2), off_g2 = off_rlo + up((size_t)srows * d * 2);
  const size_t total = off_g2 + up((size_t)srows * key_chunks(d) * 4);
  if (hipMalloc(&c->dev_mem, total) != hipSuccess) {
    delete c;
    return fail(TQ_ENOMEM, "tq_create: hipMalloc of %zu bytes failed", total);
  }
  char* base = (char*)c->dev_mem;
  bool ok = hipMemcpy(base, rh.data(), b_rimg, hipMemcpyHostToDevice) == hipSuccess &&
            hipMemcpy(base + off_rl, rl.data(), b_rimg, hipMemcpyHostToDevice) == hipSuccess &&
            hipMemcpy(base + off_sh, sh.data(), b_simg, hipMemcpyHostToDevice) == hipSuccess &&
            hipMemcpy(base + off_sl, sl.data(), b_simg, hipMemcpyHostToDevice) == hipSuccess &&
            hipMemcpy(base + off_sh32, sh32.data(), b_simg, hipMemcpyHostToDevice) == hipSuccess &&
            hipMemcpy(base + off_sl32, sl32.data(), b_simg, hipMemcpyHostToDevice) == hipSuccess &&
            hipMemcpy(base + off_r32, r32.data(), r32.size() * 4, hipMemcpyHostToDevice) == hipSuccess &&
            hipMemcpy(base + off_s32, s32.data(), s32.size() * 4, hipMemcpyHostToDevice) == hipSuccess &&
            (!step_imgs ||
             (hipMemcpy(base + off_rth, rth.data(), t_img * 2, hipMemcpyHostToDevice) == hipSuccess &&
              hipMemcpy(base + off_rtl, rtl.data(), t_img * 2, hipMemcpyHostToDevice) == hipSuccess &&
              hipMemcpy(base + off_ph, ph.data(), p_img * 2, hipMemcpyHostToDevice) == hipSuccess &&
              hipMemcpy(base + off_pl, pl.data(), p_img * 2, hipMemcpyHostToDevice) == hipSuccess));
  if (!ok) {
    (void)hipFree(c->dev_mem);
    delete c;
    return fail(TQ_EDEVICE, "tq_create: hipMemcpy failed");
  }
  c->mats.r_hi = (const uint16_t*)base;
  c->mats.r_lo = (const uint16_t*)(base + off_rl);
  c->mats.s_hi = (const uint16_t*)(base + off_sh);
  c->mats.s_lo = (const uint16_t*)(base + off_sl);
  c->mats.s_hi32 = (const uint16_t*)(base + off_sh32);
  c->mats.s_lo32 = (const uint16_t*)(base + off_sl32);
  c->mats.r32 = (const float*)(base + off_r32);
  c->mats.s32 = (const float*)(base + off_s32);
  c->mats.rt_hi = step_imgs ? (const uint16_t*)(base + off_rth) : nullptr;
  c->mats.rt_lo = step_imgs ? (const uint16_t*)(base + off_rtl) : nullptr;
  c->mats.p_hi = step_imgs ? (const uint16_t*)(base + off_ph) : nullptr;
  c->mats.p_lo = step_imgs ? (const uint16_t*)(base + off_pl) : nullptr;
  c->gen.mats = c->mats;
  c->gen.ld = ld;
  c->gen.scratch_rows = srows;
  c->gen.nrm = gen ? (float*)(base + off_nrm) : nullptr;
  c->gen.res_hi = gen ? (uint16_t*)(base + off_rh) : nullptr;
  c->gen.res_lo = gen ? (uint16_t*)(base + off_rlo) : nullptr;
  c->gen.g2p = gen ? (float*)(base + off_g2) : nullptr;
  for (int b = 0; b < 5; ++b) c->loaded[b] = false;
  *out = c;
  return TQ_OK;
}

int tq_destroy(tq_ctx* ctx) {
  clear_error();
  if (!ctx) return TQ_OK;
  int rc = TQ_OK;
  if (ctx->dev_mem && hipFree(ctx->dev_mem) != hipSuccess) rc = fail(TQ_EDEVICE, "tq_destroy: hipFree failed");
  delete ctx;
  return rc;
}

int tq_codebook_load(tq_ctx* ctx, int32_t bits, const double* centroids, const double* boundaries) {
  clear_error();
  if (!ctx) return fail(TQ_EINVAL, "tq_codebook_load: ctx is NULL");
  if (bits < 0 || bits > 4) return fail(TQ_EINVAL, "tq_codebook_load: bits %d not in 0..4", bits);
  if (!centroids || (bits > 0 && !boundaries)) return fail(TQ_EINVAL, "tq_codebook_load: NULL table");
  const int L = 1 << bits;
  for (int i = 0; i < L; ++i) {
    if (!std::isfinite(centroids[i])) return fail(TQ_EINVAL, "tq_codebook_load: non-finite centroid %d", i);
    if (i && !(centroids[i] > centroids[i - 1])) return fail(TQ_EINVAL, "tq_codebook_load: centroids not ascending");
    if (std::fabs(centroids[i]) > 60000.0) return fail(TQ_EINVAL, "tq_codebook_load: centroid out of fp16 range");
  }
  for (int i = 0; i < L - 1; ++i) {
    if (!std::isfinite(boundaries[i])) return fail(TQ_EINVAL, "tq_codebook_load: non-finite boundary %d", i);
    if (!(boundaries[i] > centroids[i] && boundaries[i] < centroids[i + 1]))
      return fail(TQ_EINVAL, "tq_codebook_load: boundary %d not between its centroids", i);
  }
  // The kernels bucket |y| against the positive boundaries, which needs a
  // codebook symmetric about 0 (every Lloyd-Max codebook of N(0, 1/d) is).
  double cmax = 0.0;
  for (int i = 0; i < L; ++i) cmax = std::fmax(cmax, std::fabs(centroids[i]));
  const double tol = 1e-9 * cmax;
  for (int i = 0; i < L; ++i)
    if (std::fabs(centroids[i] + centroids[L - 1 - i]) > tol)
      return fail(TQ_EINVAL, "tq_codebook_load: centroids not symmetric about 0 (c_i != -c_{L-1-i})");
  for (int i = 0; i < L - 1; ++i)
    if (std::fabs(boundaries[i] + boundaries[L - 2 - i]) > tol)
      return fail(TQ_EINVAL, "tq_codebook_load: boundaries not symmetric about 0");
  CodebookDev cb;
  std::memset(&cb, 0, sizeof(cb));
  for (int i = 0; i < 16; ++i) {
    // exact symmetry in fp32 (the middle boundary is 0)
    cb.beta[i] = i < L - 1 ? (float)(0.5 * (boundaries[i] - boundaries[L - 2 - i])) : INFINITY;
    const double ci = i < L ? 0.5 * (centroids[i] - centroids[L - 1 - i]) : 0.0;
    cb.cent[i] = (float)ci;
    const uint16_t h = i < L ? to_half_bits((float)ci) : 0;
    cb.tlo[i / 4] |= (uint32_t)(h & 0xFF) << (8 * (i % 4));
    cb.thi[i / 4] |= (uint32_t)(h >> 8) << (8 * (i % 4));
  }
  ctx->cb[bits] = cb;
  ctx->loaded[bits] = true;
  return TQ_OK;
}

static int check_cache(const tq_ctx* ctx, const tq_cache_view* cache, const char* fn) {
  if (!ctx) return fail(TQ_EINVAL, "%s: ctx is NULL", fn);
  if (!cache) return fail(TQ_EINVAL, "%s: cache is NULL", fn);
  if (cache->n_seq < 1) return fail(TQ_EINVAL, "%s: n_seq %d < 1", fn, cache->n_seq);
  if (cache->capacity < kBlockTokens || cache->capacity % kBlockTokens || cache->capacity > kMaxCapacity)
    return fail(TQ_EINVAL, "%s: capacity %lld is not a multiple of 128 in [128, 2^24]", fn,
                (long long)cache->capacity);
  if (!cache->key_records || !cache->value_blocks) return fail(TQ_EINVAL, "%s: NULL cache buffer", fn);
  if (!aligned16(cache->key_records) || !aligned16(cache->value_blocks))
    return fail(TQ_EINVAL, "%s: cache buffers must be 16-byte aligned", fn);
  return TQ_OK;
}

static int append_common(tq_ctx* ctx, const tq_cache_view* cache, const void* x, int32_t dtype, int64_t pos,
                         int64_t n_new, int bits, const char* fn) {
  int rc = check_cache(ctx, cache, fn);
  if (rc) return rc;
  if (dtype != TQ_F16 && dtype != TQ_F32) return fail(TQ_EINVAL, "%s: dtype %d", fn, dtype);
  if (n_new < 0) return fail(TQ_EINVAL, "%s: n_new %lld < 0", fn, (long long)n_new);
  if (pos < 0 || pos > cache->capacity || n_new > cache->capacity - pos)
    return fail(TQ_ECAPACITY, "%s: tokens [%lld, %lld) exceed capacity %lld", fn, (long long)pos,
                (long long)(pos + n_new), (long long)cache->capacity);
  if (n_new > 0 && !x) return fail(TQ_EINVAL, "%s: input is NULL", fn);
  if (n_new > 0 && !aligned16(x)) return fail(TQ_EINVAL, "%s: input must be 16-byte aligned", fn);
  if (!ctx->loaded[bits]) return fail(TQ_ENOCODEBOOK, "%s: no %d-bit codebook loaded", fn, bits);
  return TQ_OK;
}

// Whether a general-path append of n_new tokens per slot runs the tiled
// kernels, which keep the row norms and the key residual in a scratch
// buffer between launches (the context's, or a caller's workspace).
static bool keys_use_scratch(const tq_config& c, int64_t n_new) {
  return !fast_keys(c) && c.key_bits > 0 && n_new > kSmallAppend;
}
static bool values_use_scratch(const tq_config& c, int64_t n_new) {
  return !fast_values(c) && n_new > kSmallAppend;
}

// A caller's workspace laid out as the context's scratch: rows of
// (norm, exponent), key residual hi / lo and residual square sums per chunk,
// for n_seq slots x sub tokens, sub = n_new rounded up to 128 tokens and
// capped at the context's 32768 rows (at least 128 tokens a slot).
static int64_t ws_rows(int32_t n_seq, int64_t n_new) {
  int64_t cap = kScratchRows / n_seq;
  cap -= cap % kBlockTokens;
  if (cap < kBlockTokens) cap = kBlockTokens;
  const int64_t sub = std::min<int64_t>((n_new + kBlockTokens - 1) / kBlockTokens * kBlockTokens, cap);
  return (int64_t)n_seq * sub;
}
static size_t ws_layout(int d, int64_t rows, size_t off[4]) {
  auto up = [](size_t x) { return (x + 255) / 256 * 256; };
  off[0] = 0;
  off[1] = up((size_t)rows * 8);
  off[2] = off[1] + up((size_t)rows * d * 2);
  off[3] = off[2] + up((size_t)rows * d * 2);
  return off[3] + up((size_t)rows * key_chunks(d) * 4);
}

static int append_key_impl(tq_ctx* ctx, const tq_cache_view* cache, const void* k, int32_t dtype, int64_t pos,
                           int64_t n_new, const GenMats* scratch, void* stream, const char* fn) {
  AppendShape s{k, dtype, n_new, pos, cache->capacity, cache->n_seq};
  if (hipSetDevice(ctx->device) != hipSuccess) return fail(TQ_EDEVICE, "%s: hipSetDevice failed", fn);
  // A decode step on the general path takes one launch of the small kernel
  // instead of the tiled norm / rotation / projection kernels (with head_dim
  // 128 the single matrix-core kernel is as quick for a few tokens).  0-bit
  // keys (no codes) take the 32 x 32-tile kernel for bulk fp16 appends at
  // head_dim 128 and proj_dim 64, and the small kernel otherwise.
  const tq_config& c = ctx->cfg;
  const bool zero_tiles = c.key_bits == 0 && c.head_dim == kD && c.proj_dim == 64 && dtype == TQ_F16;
  int rc;
  if (fast_keys(c) || (zero_tiles && n_new > kSmallAppend))
    rc = launch_compress_keys(ctx->mats, ctx->cb[c.key_bits], c.key_bits, c.proj_dim, s, cache->key_records,
                              stream);
  else if (!keys_use_scratch(c, n_new))
    rc = launch_small_keys(ctx->mats, ctx->cb[c.key_bits], c.key_bits, c.head_dim, c.proj_dim, s,
                           cache->key_records, stream);
  else
    rc = launch_general_keys(*scratch, ctx->cb[c.key_bits], c.key_bits, c.head_dim, c.proj_dim, s,
                             cache->key_records, stream);
  if (rc == TQ_EUNSUPPORTED)
    return fail(rc, "%s: a bulk append into %d slots needs more rows than the context's scratch holds "
                    "(tq_append_key_ws takes a workspace of any size)", fn, cache->n_seq);
  return rc ? fail(rc, "%s: launch failed (%d)", fn, rc) : TQ_OK;
}

static int append_value_impl(tq_ctx* ctx, const tq_cache_view* cache, const void* v, int32_t dtype, int64_t pos,
                             int64_t n_new, const GenMats* scratch, void* stream, const char* fn) {
  AppendShape s{v, dtype, n_new, pos, cache->capacity, cache->n_seq};
  if (hipSetDevice(ctx->device) != hipSuccess) return fail(TQ_EDEVICE, "%s: hipSetDevice failed", fn);
  const tq_config& c = ctx->cfg;
  int rc;
  if (n_new <= kSmallAppend)  // a decode step: no tile set-up
    rc = launch_small_values(ctx->mats, ctx->cb[c.value_bits], c.value_bits, c.head_dim, s, cache->value_blocks,
                             stream);
  else if (fast_values(c))
    rc = launch_compress_values(ctx->mats, ctx->cb[c.value_bits], c.value_bits, s, cache->value_blocks, stream);
  else
    rc = launch_general_values(*scratch, ctx->cb[c.value_bits], c.value_bits, c.head_dim, s, cache->value_blocks,
                               stream);
  if (rc == TQ_EUNSUPPORTED)
    return fail(rc, "%s: a bulk append into %d slots needs more rows than the context's scratch holds "
                    "(tq_append_value_ws takes a workspace of any size)", fn, cache->n_seq);
  return rc ? fail(rc, "%s: launch failed (%d)", fn, rc) : TQ_OK;
}

// The scratch view of a caller's workspace (checked against its size).
static int ws_scratch(const tq_ctx* ctx, int32_t n_seq, int64_t n_new, void* ws, size_t ws_bytes, GenMats* g,
                      const char* fn) {
  *g = ctx->gen;
  const int64_t rows = ws_rows(n_seq, n_new);
  size_t off[4];
  const size_t need = ws_layout(ctx->cfg.head_dim, rows, off);
  if (!ws) return fail(TQ_EINVAL, "%s: workspace is NULL (%zu bytes needed)", fn, need);
  if (!aligned16(ws)) return fail(TQ_EINVAL, "%s: workspace must be 16-byte aligned", fn);
  if (ws_bytes < need) return fail(TQ_EWORKSPACE, "%s: workspace %zu < %zu bytes", fn, ws_bytes, need);
  char* b = (char*)ws;
  g->nrm = (float*)(b + off[0]);
  g->res_hi = (uint16_t*)(b + off[1]);
  g->res_lo = (uint16_t*)(b + off[2]);
  g->g2p = (float*)(b + off[3]);
  g->scratch_rows = rows;
  return TQ_OK;
}

int tq_append_key(tq_ctx* ctx, const tq_cache_view* cache, const void* k, int32_t dtype, int64_t pos,
                  int64_t n_new, void* stream) {
  clear_error();
  int rc = append_common(ctx, cache, k, dtype, pos, n_new, ctx ? ctx->cfg.key_bits : 1, "tq_append_key");
  if (rc) return rc;
  if (n_new == 0) return TQ_OK;
  return append_key_impl(ctx, cache, k, dtype, pos, n_new, &ctx->gen, stream, "tq_append_key");
}

int tq_append_value(tq_ctx* ctx, const tq_cache_view* cache, const void* v, int32_t dtype, int64_t pos,
                    int64_t n_new, void* stream) {
  clear_error();
  int rc = append_common(ctx, cache, v, dtype, pos, n_new, ctx ? ctx->cfg.value_bits : 1, "tq_append_value");
  if (rc) return rc;
  if (n_new == 0) return TQ_OK;
  return append_value_impl(ctx, cache, v, dtype, pos, n_new, &ctx->gen, stream, "tq_append_value");
}

size_t tq_append_workspace_bytes(const tq_ctx* ctx, int32_t n_seq, int64_t n_new) {
  if (!ctx || n_seq < 1 || n_new < 1) return 0;
  if (!keys_use_scratch(ctx->cfg, n_new) && !values_use_scratch(ctx->cfg, n_new)) return 0;
  size_t off[4];
  return ws_layout(ctx->cfg.head_dim, ws_rows(n_seq, n_new), off);
}

int tq_append_key_ws(tq_ctx* ctx, const tq_cache_view* cache, const void* k, int32_t dtype, int64_t pos,
                     int64_t n_new, void* workspace, size_t workspace_bytes, void* stream) {
  clear_error();
  int rc = append_common(ctx, cache, k, dtype, pos, n_new, ctx ? ctx->cfg.key_bits : 1, "tq_append_key_ws");
  if (rc) return rc;
  if (n_new == 0) return TQ_OK;
  GenMats g;
  if (keys_use_scratch(ctx->cfg, n_new)) {
    rc = ws_scratch(ctx, cache->n_seq, n_new, workspace, workspace_bytes, &g, "tq_append_key_ws");
    if (rc) return rc;
  }
  return append_key_impl(ctx, cache, k, dtype, pos, n_new, &g, stream, "tq_append_key_ws");
}

int tq_append_value_ws(tq_ctx* ctx, const tq_cache_view* cache, const void* v, int32_t dtype, int64_t pos,
                       int64_t n_new, void* workspace, size_t workspace_bytes, void* stream) {
  clear_error();
  int rc = append_common(ctx, cache, v, dtype, pos, n_new, ctx ? ctx->cfg.value_bits : 1, "tq_append_value_ws");
  if (rc) return rc;
  if (n_new == 0) return TQ_OK;
  GenMats g;
  if (values_use_scratch(ctx->cfg, n_new)) {
    rc = ws_scratch(ctx, cache->n_seq, n_new, workspace, workspace_bytes, &g, "tq_append_value_ws");
    if (rc) return rc;
  }
  return append_value_impl(ctx, cache, v, dtype, pos, n_new, &g, stream, "tq_append_value_ws");
}

static int attn_common(tq_ctx* ctx, const tq_cache_view* cache, const void* q, int32_t dtype, int32_t G,
                       int64_t n_tokens, const void* outp, void* ws, size_t ws_bytes, bool need_values,
                       const char* fn, AttnPlan* plan) {
  int rc = check_cache(ctx, cache, fn);
  if (rc) return rc;
  if (dtype != TQ_F16 && dtype != TQ_F32) return fail(TQ_EINVAL, "%s: dtype %d", fn, dtype);
  const int gmax = need_values ? 16 : kMaxGeneralHeads;
  if (G < 1 || G > gmax) return fail(TQ_EINVAL, "%s: G %d not in 1..%d", fn, G, gmax);
  if (n_tokens < 1 || n_tokens > cache->capacity)
    return fail(TQ_EINVAL, "%s: n_tokens %lld not in [1, capacity]", fn, (long long)n_tokens);
  if (!q || !outp || !ws) return fail(TQ_EINVAL, "%s: NULL q, output or workspace", fn);
  if (!aligned16(q) || !aligned16(outp) || !aligned16(ws))
    return fail(TQ_EINVAL, "%s: q, output and workspace must be 16-byte aligned", fn);
  if (!ctx->loaded[ctx->cfg.key_bits])
    return fail(TQ_ENOCODEBOOK, "%s: no %d-bit key codebook loaded", fn, ctx->cfg.key_bits);
  if (need_values && !ctx->loaded[ctx->cfg.value_bits])
    return fail(TQ_ENOCODEBOOK, "%s: no %d-bit value codebook loaded", fn, ctx->cfg.value_bits);
  size_t need;
  if (fast_attn(ctx->cfg, G))
    need = (*plan = plan_attention(ctx->cfg.proj_dim, cache->n_seq, G, n_tokens)).total;
  else if (need_values)
    need = general_attend_plan(ctx->cfg.head_dim, ctx->cfg.proj_dim, cache->n_seq, G, n_tokens).total;
  else
    need = general_scores_workspace(ctx->cfg.head_dim, ctx->cfg.proj_dim, cache->n_seq, G);
  if (ws_bytes < need) return fail(TQ_EWORKSPACE, "%s: workspace %zu < %zu bytes", fn, ws_bytes, need);
  return TQ_OK;
}

int tq_attention_scores(tq_ctx* ctx, const tq_cache_view* cache, const void* q, int32_t dtype, int32_t G,
                        int64_t n_tokens, float* scores, void* workspace, size_t workspace_bytes, void* stream) {
  clear_error();
  AttnPlan plan;
  int rc = attn_common(ctx, cache, q, dtype, G, n_tokens, scores, workspace, workspace_bytes, false,
                       "tq_attention_scores", &plan);
  if (rc) return rc;
  if (hipSetDevice(ctx->device) != hipSuccess) return fail(TQ_EDEVICE, "tq_attention_scores: hipSetDevice");
  AttnShape s{q, dtype, G, n_tokens, cache->capacity, cache->n_seq};
  if (fast_attn(ctx->cfg, G)) {
    rc = launch_prep_queries(ctx->mats, ctx->cfg.proj_dim, s, workspace, plan, stream);
    if (!rc)
      rc = launch_scores(ctx->cb[ctx->cfg.key_bits], ctx->cfg.key_bits, ctx->cfg.proj_dim, s, cache->key_records,
                         scores, workspace, plan, stream);
  } else {
    rc = launch_general_scores(ctx->mats, ctx->cb[ctx->cfg.key_bits], ctx->cfg.key_bits, ctx->cfg.head_dim,
                               ctx->cfg.proj_dim, s, cache->key_records, scores, workspace, stream);
  }
  return rc ? fail(rc, "tq_attention_scores: launch failed (%d)", rc) : TQ_OK;
}

int tq_attend(tq_ctx* ctx, const tq_cache_view* cache, const void* q, int32_t dtype, int32_t G, int64_t n_tokens,
              float scale, float* out, void* workspace, size_t workspace_bytes, void* stream) {
  clear_error();
  AttnPlan plan;
  int rc = attn_common(ctx, cache, q, dtype, G, n_tokens, out, workspace, workspace_bytes, true, "tq_attend",
                       &plan);
  if (rc) return rc;
  if (!std::isfinite(scale)) return fail(TQ_EINVAL, "tq_attend: scale is not finite");
  if (scale <= 0.f) scale = 1.f / std::sqrt((float)ctx->cfg.head_dim);
  if (hipSetDevice(ctx->device) != hipSuccess) return fail(TQ_EDEVICE, "tq_attend: hipSetDevice");
  AttnShape s{q, dtype, G, n_tokens, cache->capacity, cache->n_seq};
  if (fast_attn(ctx->cfg, G)) {
    rc = launch_prep_queries(ctx->mats, ctx->cfg.proj_dim, s, workspace, plan, stream);
    if (!rc)
      rc = launch_attend(ctx->mats, ctx->cb[ctx->cfg.key_bits], ctx->cfg.key_bits, ctx->cb[ctx->cfg.value_bits],
                         ctx->cfg.value_bits, ctx->cfg.proj_dim, s, cache->key_records, cache->value_blocks, scale,
                         out, workspace, plan, stream);
  } else {
    rc = launch_general_attend(ctx->mats, ctx->cb[ctx->cfg.key_bits], ctx->cfg.key_bits,
                               ctx->cb[ctx->cfg.value_bits], ctx->cfg.value_bits, ctx->cfg.head_dim,
                               ctx->cfg.proj_dim, s, cache->key_records, cache->value_blocks, scale, out,
                               workspace, stream);
  }
  return rc ? fail(rc, "tq_attend: launch failed (%d)", rc) : TQ_OK;
}

int tq_attend_noalloc(tq_ctx* ctx, const tq_cache_view* cache, const void* q, int32_t dtype, int32_t G,
                      int64_t n_tokens, float scale, float* out, void* stream) {
  clear_error();
  const char* fn = "tq_attend_noalloc";
  if (!ctx) return fail(TQ_EINVAL, "%s: ctx is NULL", fn);
  void* ws = noalloc_scratch_ptr(ctx->device);
  if (!ws) return fail(TQ_EDEVICE, "%s: no scratch address for device %d", fn, ctx->device);
  // the checks of tq_attend, against the scratch's fixed size
  AttnPlan plan;
  int rc = attn_common(ctx, cache, q, dtype, G, n_tokens, out, ws, kNoAllocScratchBytes, true, fn, &plan);
  if (rc) return rc;
  return tq_attend(ctx, cache, q, dtype, G, n_tokens, scale, out, ws, kNoAllocScratchBytes, stream);
}

int tq_decode_step(tq_ctx* ctx, const tq_cache_view* cache, const void* k, const void* v, int32_t dtype,
                   int64_t pos, int64_t n_new, const void* q, int32_t G, float scale, float* out, void* workspace,
                   size_t workspace_bytes, void* stream) {
  clear_error();
  const char* fn = "tq_decode_step";
  if (n_new < 1) return fail(TQ_EINVAL, "%s: n_new %lld < 1", fn, (long long)n_new);
  // every argument of the three operations is checked before anything runs
  int rc = append_common(ctx, cache, k, dtype, pos, n_new, ctx ? ctx->cfg.key_bits : 1, fn);
  if (rc) return rc;
  rc = append_common(ctx, cache, v, dtype, pos, n_new, ctx->cfg.value_bits, fn);
  if (rc) return rc;
  AttnPlan plan;
  rc = attn_common(ctx, cache, q, dtype, G, pos + n_new, out, workspace, workspace_bytes, true, fn, &plan);
  if (rc) return rc;
  if (!std::isfinite(scale)) return fail(TQ_EINVAL, "%s: scale is not finite", fn);
  if (!(fast_attn(ctx->cfg, G) && n_new <= kSmallAppend &&
        (int64_t)(plan.waves_per_slot / 4 + 2) * G <= kStepMaxPartials)) {
    // other shapes or longer appends: the three calls, in order
    rc = tq_append_key(ctx, cache, k, dtype, pos, n_new, stream);
    if (!rc) rc = tq_append_value(ctx, cache, v, dtype, pos, n_new, stream);
    if (!rc) rc = tq_attend(ctx, cache, q, dtype, G, pos + n_new, scale, out, workspace, workspace_bytes, stream);
    return rc;
  }
  if (scale <= 0.f) scale = 1.f / std::sqrt((float)ctx->cfg.head_dim);
  if (hipSetDevice(ctx->device) != hipSuccess) return fail(TQ_EDEVICE, "%s: hipSetDevice failed", fn);
  const AppendShape ks{k, dtype, n_new, pos, cache->capacity, cache->n_seq};
  const AppendShape vs{v, dtype, n_new, pos, cache->capacity, cache->n_seq};
  const AttnShape s{q, dtype, G, pos + n_new, cache->capacity, cache->n_seq};
  rc = launch_decode_step(ctx->mats, ctx->cb[ctx->cfg.key_bits], ctx->cfg.key_bits, ctx->cb[ctx->cfg.value_bits],
                          ctx->cfg.value_bits, ctx->cfg.head_dim, ctx->cfg.proj_dim, ks, vs, s, cache->key_records,
                          cache->value_blocks, scale, out, workspace, plan, stream);
  return rc ? fail(rc, "%s: launch failed (%d)", fn, rc) : TQ_OK;
}

static int get_common(tq_ctx* ctx, const tq_cache_view* cache, int64_t pos, int64_t n_tokens, const float* out,
                      int bits, const char* fn) {
  int rc = check_cache(ctx, cache, fn);
  if (rc) return rc;
  if (n_tokens < 0) return fail(TQ_EINVAL, "%s: n_tokens %lld < 0", fn, (long long)n_tokens);
  if (pos < 0 || pos > cache->capacity || n_tokens > cache->capacity - pos)
    return fail(TQ_ECAPACITY, "%s: tokens [%lld, %lld) exceed capacity %lld", fn, (long long)pos,
                (long long)(pos + n_tokens), (long long)cache->capacity);
  if (n_tokens > 0 && !out) return fail(TQ_EINVAL, "%s: out is NULL", fn);
  if (n_tokens > 0 && !aligned16(out)) return fail(TQ_EINVAL, "%s: out must be 16-byte aligned", fn);
  if (!ctx->loaded[bits]) return fail(TQ_ENOCODEBOOK, "%s: no %d-bit codebook loaded", fn, bits);
  return TQ_OK;
}

static int get_vectors(tq_ctx* ctx, const tq_cache_view* cache, int64_t pos, int64_t n_tokens, float* out,
                       void* stream, bool keys, const char* fn) {
  clear_error();
  const int bits = ctx ? (keys ? ctx->cfg.key_bits : ctx->cfg.value_bits) : 1;
  int rc = get_common(ctx, cache, pos, n_tokens, out, bits, fn);
  if (rc) return rc;
  if (n_tokens == 0) return TQ_OK;
  if (hipSetDevice(ctx->device) != hipSuccess) return fail(TQ_EDEVICE, "%s: hipSetDevice failed", fn);
  rc = launch_dequant(ctx->mats, ctx->cb[bits], bits, ctx->cfg.head_dim, ctx->cfg.proj_dim, keys,
                      cache->key_records, cache->value_blocks, cache->capacity, cache->n_seq, pos, n_tokens, out,
                      stream);
  return rc ? fail(rc, "%s: launch failed (%d)", fn, rc) : TQ_OK;
}

size_t tq_topk_workspace_bytes(const tq_config* cfg, int32_t n_seq, int32_t G, int64_t n_tokens, int32_t k) {
  if (!cfg || check_config(cfg) != TQ_OK || n_seq < 1 || G < 1 || G > kMaxGeneralHeads || n_tokens < 1 || k < 1 ||
      k > kTopkMax)
    return 0;
  return topk_plan(cfg->head_dim, cfg->proj_dim, n_seq, G, n_tokens, k).total;
}

int tq_topk_scores(tq_ctx* ctx, const tq_cache_view* cache, const void* q, int32_t dtype, int32_t G,
                   int64_t n_tokens, int32_t k, float* top_scores, int32_t* top_index, void* workspace,
                   size_t workspace_bytes, void* stream) {
  clear_error();
  const char* fn = "tq_topk_scores";
  int rc = check_cache(ctx, cache, fn);
  if (rc) return rc;
  if (dtype != TQ_F16 && dtype != TQ_F32) return fail(TQ_EINVAL, "%s: dtype %d", fn, dtype);
  if (G < 1 || G > kMaxGeneralHeads) return fail(TQ_EINVAL, "%s: G %d not in 1..%d", fn, G, kMaxGeneralHeads);
  if (k < 1 || k > kTopkMax) return fail(TQ_EINVAL, "%s: k %d not in 1..%d", fn, k, kTopkMax);
  if (n_tokens < 1 || n_tokens > cache->capacity)
    return fail(TQ_EINVAL, "%s: n_tokens %lld not in [1, capacity]", fn, (long long)n_tokens);
  if (!q || !top_scores || !top_index || !workspace) return fail(TQ_EINVAL, "%s: NULL pointer", fn);
  if (!aligned16(q) || !aligned16(top_scores) || !aligned16(top_index) || !aligned16(workspace))
    return fail(TQ_EINVAL, "%s: q, outputs and workspace must be 16-byte aligned", fn);
  if (!ctx->loaded[ctx->cfg.key_bits])
    return fail(TQ_ENOCODEBOOK, "%s: no %d-bit key codebook loaded", fn, ctx->cfg.key_bits);
  const size_t need = topk_plan(ctx->cfg.head_dim, ctx->cfg.proj_dim, cache->n_seq, G, n_tokens, k).total;
  if (workspace_bytes < need) return fail(TQ_EWORKSPACE, "%s: workspace %zu < %zu bytes", fn, workspace_bytes, need);
  if (hipSetDevice(ctx->device) != hipSuccess) return fail(TQ_EDEVICE, "%s: hipSetDevice failed", fn);
  AttnShape s{q, dtype, G, n_tokens, cache->capacity, cache->n_seq};
  rc = launch_topk(ctx->mats, ctx->cb[ctx->cfg.key_bits], ctx->cfg.key_bits, ctx->cfg.head_dim, ctx->cfg.proj_dim,
                   s, k, cache->key_records, top_scores, top_index, workspace, stream);
  return rc ? fail(rc, "%s: launch failed (%d)", fn, rc) : TQ_OK;
}

int tq_get_values(tq_ctx* ctx, const tq_cache_view* cache, int64_t pos, int64_t n_tokens, float* out,
                  void* stream) {
  return get_vectors(ctx, cache, pos, n_tokens, out, stream, false, "tq_get_values");
}

int tq_get_keys(tq_ctx* ctx, const tq_cache_view* cache, int64_t pos, int64_t n_tokens, float* out,
                void* stream) {
  return get_vectors(ctx, cache, pos, n_tokens, out, stream, true, "tq_get_keys");
}

int tq_hbm_stream(const void* src, size_t read_bytes, void* dst, size_t write_bytes, uint32_t* sink,
                  int32_t waves_per_cu, int32_t flags, void* stream) {
  clear_error();
  const int nl = (flags >> 8) & 0xFF;
  const int loads = nl == 0 ? 4 : nl;
  if ((flags & ~0xFF01) != 0 || !(loads == 4 || loads == 8 || loads == 16))
    return fail(TQ_EINVAL, "tq_hbm_stream: flags 0x%x: bit 0 and loads in flight 4, 8 or 16 in bits 8-15", flags);
  if (!src || ((uintptr_t)src & 15u)) return fail(TQ_EINVAL, "tq_hbm_stream: src must be a 16-byte aligned device pointer");
  const size_t group = 1024u * (size_t)loads;
  if (read_bytes == 0 || read_bytes % group != 0)
    return fail(TQ_EINVAL, "tq_hbm_stream: read_bytes must be a positive multiple of %zu", group);
  if (write_bytes != 0) {
    if (!dst || ((uintptr_t)dst & 15u))
      return fail(TQ_EINVAL, "tq_hbm_stream: dst must be a 16-byte aligned device pointer");
    if (!(write_bytes == read_bytes || 2 * write_bytes == read_bytes || 4 * write_bytes == read_bytes))
      return fail(TQ_EINVAL, "tq_hbm_stream: write_bytes must be 0 or read_bytes / 1, / 2 or / 4");
  }
  if (!sink || ((uintptr_t)sink & 3u)) return fail(TQ_EINVAL, "tq_hbm_stream: sink must be a 4-byte aligned device pointer");
  if (waves_per_cu < 0 || waves_per_cu > 64 || waves_per_cu % 4)
    return fail(TQ_EINVAL, "tq_hbm_stream: waves_per_cu %d: need 0 or a multiple of 4 up to 64", waves_per_cu);
  if (waves_per_cu == 0) waves_per_cu = 16;
  static std::once_flag once;
  static int init_rc = 0;
  std::call_once(once, [] { init_rc = stream_device_init(); });
  if (init_rc != 0) return fail(TQ_EDEVICE, "tq_hbm_stream: HIP device query failed");
  const int rc = launch_stream(src, read_bytes, dst, write_bytes, sink, waves_per_cu, loads, (flags & 1) != 0, stream);
  return rc == 0 ? TQ_OK : fail(rc, "tq_hbm_stream: kernel launch failed");
}

}  // extern "C"
