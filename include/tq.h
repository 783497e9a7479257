/*
 * tq.h -- TurboQuant KV-cache compression and attention over the packed
 * cache, for AMD Instinct MI355X (gfx950).  C ABI of libtq.so.
 *
 * What is computed (sources: the "turboquant-pytorch" skill pages on
 * nav.superapi.store -- sections 主要能力, 核心 API, 常见使用模式, 算法细节,
 * 限制与注意事项 -- and on atskills.one -- "What this skill does": Stage 1,
 * Stage 2, Why Random Rotation?, Why QJL for Keys but Not Values?):
 *
 *   keys   k (d floats): n = ||k||, y = R k / n, idx_j = #{i : beta_i < y_j}
 *          (Lloyd-Max cell of each rotated coordinate), r = y - c[idx],
 *          gamma = ||r||, sign bits s = [S r >= 0] (1-bit QJL projection of
 *          the residual).  Stored: idx, s, n, gamma.
 *   values v: n = ||v||, y = R v / n, idx as above.  Stored: idx, n.
 *   score  est(q, k) = n * ( <R q, c[idx]> + gamma * sqrt(pi/2)/m * <S R q, 2s-1> )
 *          (asymmetric: full-precision query against the packed key; unscaled).
 *   attend out = R^T sum_t softmax_t(scale * est_t) * n_t^v * c[idx_t^v].
 *
 * R (d x d, orthogonal) and S (m x d, Gaussian) are fixed per (dim, seed) and
 * handed in by the caller; c (2^b centroids) and beta (2^b - 1 boundaries)
 * are the Lloyd-Max codebook of N(0, 1/d).
 *
 * Conventions for every call:
 *  - Return 0 (TQ_OK) or a negative tq_status.  Nothing throws.  On an
 *    argument error nothing is launched and no output is written;
 *    tq_last_error() then holds a message (thread-local).
 *  - "device" pointers are HIP device memory owned by the caller.  The
 *    library allocates device memory only in tq_create (its own copies of R,
 *    S and the codebooks: d^2 + m d fp32 plus the same again as fp16 halves;
 *    for shapes on the general path, see below, also a scratch buffer of
 *    32768 rows x (4 d + 8 + 4 ceil(d/128)) bytes, 128 MB at d = 1024) and frees it
 *    in tq_destroy.
 *  - Calls that take a stream enqueue work on it and return at once; they
 *    are ordered with other work on that stream.  stream == NULL means the
 *    default stream.  The argument is a hipStream_t passed as void*.
 *  - A context is read-only after its codebooks are loaded, so calls on
 *    different streams may run concurrently; tq_codebook_load must not run
 *    concurrently with calls that use the same context.  Exception: on the
 *    general path the appends of one context share its scratch buffer, so
 *    its tq_append_key / tq_append_value calls must be ordered (one stream,
 *    or one context per stream); tq_append_key_ws / tq_append_value_ws take
 *    the scratch from a caller-owned workspace instead and have no such
 *    restriction.
 *  - Shapes.  head_dim 128 with proj_dim 64 or 128 runs single-kernel
 *    compress and attention paths; every other valid shape (head_dim a
 *    multiple of 64 up to 1024, proj_dim a multiple of 32 up to 512) runs
 *    the general path: tiled rotation / projection kernels for the appends,
 *    a chunked score kernel, and an attend that materialises the scores in
 *    the workspace and merges per-range softmax partials.  0-bit keys are
 *    appended by the single-kernel key path (fp16, proj_dim 64) or by one
 *    workgroup per token, and scored and attended as above.
 *  - Device pointers must be 16-byte aligned.
 */
#ifndef TQ_H
#define TQ_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Version of the packed record layout described below.  Version 1 was the
 * planned bit-plane layout (index bit p of 32 consecutive coordinates in one
 * word); it was never built.  Version 2 is the matrix-core operand layout
 * below, whose code groups decode straight into MFMA operands. */
#define TQ_LAYOUT_VERSION 2

typedef enum {
  TQ_OK = 0,
  TQ_EINVAL = -1,       /* bad argument: size, bits, dtype, null/misaligned pointer */
  TQ_ECAPACITY = -2,    /* pos + n_new exceeds the cache capacity */
  TQ_ENOCODEBOOK = -3,  /* no codebook loaded for the bits this call needs */
  TQ_ENOMEM = -4,       /* device allocation failed (tq_create only) */
  TQ_EDEVICE = -5,      /* a HIP call or kernel launch failed */
  TQ_EUNSUPPORTED = -6, /* valid but not built (a bulk general-path append into more than 256
                           slots through the context's scratch: see tq_append_key_ws) */
  TQ_EWORKSPACE = -7    /* workspace smaller than tq_attend_workspace_bytes / tq_workspace_bytes */
} tq_status;

typedef enum { TQ_F16 = 1, TQ_F32 = 2 } tq_dtype;

typedef struct tq_ctx tq_ctx;

/* Static shape of a compressed cache.  head_dim d: multiple of 64 in
 * [64, 1024].  proj_dim m: multiple of 32 in [32, 512] (default d/2, so
 * 64 -> 32 and 128 -> 64: nav.superapi.store 算法细节 / proj_dim 选择).  value_bits in 1..4 and
 * key_bits in 0..4 (the pages use 2-4; 1 is the 1-bit limit).  key_bits 0
 * is the bit budget of (b - 1)-bit codes plus QJL signs at b = 1: one cell
 * whose centroid is 0, so a key keeps only its m sign bits of S R k/||k||
 * and its norms, and its score is the plain QJL estimate (atskills.one,
 * Stage 2 applied to the whole rotated direction). */
typedef struct {
  int32_t head_dim;
  int32_t proj_dim;
  int32_t key_bits;
  int32_t value_bits;
} tq_config;

/* Caller-owned packed cache of n_seq slots (one slot = one KV head of one
 * sequence/layer), each holding up to `capacity` tokens (a multiple of 128,
 * at most 2^24).
 *
 * key_records: device, n_seq * capacity * tq_key_record_bytes(ctx) bytes.
 *   Slot s, token t starts at byte (s * capacity + t) * tq_key_record_bytes(ctx).
 * value_blocks: device, n_seq * capacity * tq_value_record_bytes(ctx) bytes
 *   (= n_seq * (capacity/128) * tq_value_block_bytes(cfg)); block (s, t/128)
 *   starts at byte (s * capacity/128 + t/128) * tq_value_block_bytes(cfg).
 * Zero-fill both buffers before first use if tokens will be read before
 * they are written.
 *
 * Record layout v2 (32-bit little-endian words; b = bits, d = head_dim):
 *  Code groups.  b consecutive words hold 32 b-bit codes as 8 slots s x 4
 *  byte lanes i; byte lane i of every word belongs to code (s, i):
 *    b=1: bit s;  b=2: word s/4, bits 2(s%4)..;  b=4: word s/2, bits 4(s%2)..;
 *    b=3: s<6: word s/2, bits 3(s%2)..; s=6: code bits 0-1 at bits 6-7 of
 *         word 0, bit 2 at bit 6 of word 2; s=7: bits 0-1 at bits 6-7 of
 *         word 1, bit 2 at bit 7 of word 2   (bit numbers within the byte).
 *  Key record, n = floor(d/128) full chunks: 4 n code groups (q, g),
 *    q = 0..3, g = 0..n - 1, at words b (q n + g) .. + b - 1; group (q, g),
 *    slot s, byte lane i is the code of rotated coordinate
 *    128 g + 16 s + 4 q + i.  If d % 128 == 64, two more groups p = 0, 1
 *    (the half chunk) at words b (4 n + p) .. + b - 1; slot s, byte lane i
 *    of group p is coordinate 128 n + 16 (s%4) + 4 (p + 2 (s/4)) + i.
 *    Then m/32 sign words, n' = floor(m/64): projection coordinate
 *    16 t + 4 q + i < 64 n' is bit 16 (q%2) + 4 (t%4) + i of word
 *    2 (t/4) + q/2; if m % 64 == 32, projection 64 n' + j is bit j of word
 *    2 n' (1 = projection >= 0).
 *    Then fp32 ||k||, then fp32 gamma.  Size 4 (b d/32 + m/32 + 2) bytes
 *    (b = 0: no code groups, the sign words start the record).
 *  Value block (128 tokens): for w = 0..b-1, q = 0..3, coordinate c =
 *    0..d-1, word (w * 4 + q) * d + c; the b words (w = 0..b-1) of (q, c)
 *    form a code group whose slot s, byte lane i is the code of coordinate c
 *    of block token 16 s + 4 q + i.  Then 128 fp32 norms ||v|| in token
 *    order.  Size 4 (4 b d + 128) bytes.
 * Codes are idx = #{i : beta_i < y} of the rotated, normalised coordinate.
 * Keys are grouped by token and values by coordinate because those are the
 * contraction orders of the score and the weighted-sum matrix products. */
typedef struct {
  void* key_records;
  void* value_blocks;
  int64_t capacity;
  int32_t n_seq;
} tq_cache_view;

/* ---- host-only helpers (no device work) ---------------------------------- */

/* Lloyd-Max codebook for coordinates ~ N(0, 1/head_dim) with 2^bits levels
 * (nav.superapi.store 核心 API build_lloyd_max_codebook(dim, bits) ->
 * (boundaries, centroids); 限制与注意事项: computed once per (dim, bits)).
 * Writes 2^bits ascending centroids and 2^bits - 1 ascending boundaries
 * (host arrays owned by the caller).  bits in 0..4, head_dim >= 1; at 0 bits
 * the one centroid is 0 and boundaries may be NULL.
 * Returns TQ_EINVAL on bad arguments. */
int tq_lloyd_max_codebook(int32_t head_dim, int32_t bits, double* centroids, double* boundaries);

/* Sizes for a configuration, usable before any context exists (to size the
 * caller's buffers): bytes of one key record / one 128-token value block / a
 * whole cache of n_seq slots x capacity tokens.  0 if cfg is NULL or invalid
 * (the same checks as tq_create) or capacity is not a positive multiple of
 * 128. */
size_t tq_config_key_record_bytes(const tq_config* cfg);
size_t tq_value_block_bytes(const tq_config* cfg);
size_t tq_cache_key_bytes(const tq_config* cfg, int32_t n_seq, int64_t capacity);
size_t tq_cache_value_bytes(const tq_config* cfg, int32_t n_seq, int64_t capacity);

/* Device workspace bytes needed by tq_attention_scores, tq_attend and
 * tq_decode_step for this shape (query operands, query norms, per-wave
 * attention partials; on the general path also the materialised scores of
 * tq_attend).  0 on invalid arguments (cfg NULL/invalid, n_seq < 1, G not in
 * 1..512, n_tokens < 1). */
size_t tq_workspace_bytes(const tq_config* cfg, int32_t n_seq, int32_t G, int64_t n_tokens);

/* Thread-local message describing the last failure of this thread. */
const char* tq_last_error(void);

/* ---- context ---------------------------------------------------------------- */

/* Create a context on the current HIP device.  R: host, d x d row-major
 * (rotation y = R x), S: host, m x d row-major (QJL matrix, applied to the
 * rotated residual).  Both are copied before return.  R should be orthogonal
 * (nav.superapi.store 算法细节 / 随机旋转); this is not checked.  Returns
 * TQ_EINVAL (bad config or null pointers), TQ_ENOMEM or TQ_EDEVICE.
 * Arguments are checked before any HIP call. */
int tq_create(const tq_config* cfg, const double* R, const double* S, tq_ctx** out);

/* Free the context's device memory.  NULL is accepted.  Work still queued
 * that uses the context must have finished. */
int tq_destroy(tq_ctx* ctx);

/* Size queries of a context (the sizes behind TurboQuantKVCache's buffers,
 * nav.superapi.store 核心 API).  Host-only; 0 if ctx is NULL or an argument
 * is out of range.
 *   tq_key_record_bytes:   one token's key record, 4 (b d/32 + m/32 + 2)
 *                          bytes (b = key_bits).
 *   tq_value_record_bytes: one token's share of a 128-token value block,
 *                          4 (b d/32 + 1) bytes (b = value_bits): the block
 *                          is 128 times this.
 *   tq_attend_workspace_bytes: the workspace tq_attention_scores, tq_attend
 *                          and tq_decode_step need for n_seq slots, G query
 *                          heads per slot and n_tokens attended tokens; the
 *                          same value as tq_workspace_bytes for the
 *                          context's configuration (n_seq >= 1, 1 <= G <= 512,
 *                          n_tokens >= 1). */
size_t tq_key_record_bytes(const tq_ctx* ctx);
size_t tq_value_record_bytes(const tq_ctx* ctx);
size_t tq_attend_workspace_bytes(const tq_ctx* ctx, int32_t n_seq, int32_t G, int64_t n_tokens);

/* Load the codebook for `bits` (host arrays, copied): 2^bits strictly
 * ascending finite centroids and 2^bits - 1 strictly ascending finite
 * boundaries, each boundary strictly between its two centroids, and the
 * codebook symmetric about 0 within 1e-9 of its largest centroid (as every
 * Lloyd-Max codebook of the centred Gaussian is); TQ_EINVAL otherwise.  Needed for
 * key_bits and value_bits before any append or attention call.  Host-only:
 * the codebook travels to the kernels as launch arguments. */
int tq_codebook_load(tq_ctx* ctx, int32_t bits, const double* centroids, const double* boundaries);
/* (bits 0..4; at 0 bits the single centroid must be 0 and boundaries may be
 * NULL.) */

/* ---- hot path ---------------------------------------------------------------- */

/* Compress n_new keys per slot and write them at token positions
 * [pos, pos + n_new) of every slot (append_key of TurboQuantKVCache,
 * nav.superapi.store 核心 API; stage 1 + stage 2, atskills.one Stage 2).
 * k: device, [n_seq][n_new][d] contiguous, dtype TQ_F16 or TQ_F32, finite.
 * fp32 rows may have any magnitude whose norm fits fp32, subnormal
 * coordinates included: norms are taken over rows shifted by a power of two.
 * A zero vector is encoded with direction 0 and scores 0.
 * Errors: TQ_EINVAL, TQ_ECAPACITY (pos < 0 or pos + n_new > capacity),
 * TQ_ENOCODEBOOK, TQ_EDEVICE.  n_new == 0 is a no-op. */
int tq_append_key(tq_ctx* ctx, const tq_cache_view* cache, const void* k, int32_t dtype,
                  int64_t pos, int64_t n_new, void* stream);

/* Compress n_new values per slot (stage 1 only: TurboQuantCompressorMSE,
 * nav.superapi.store 核心 API; values need no QJL, 算法细节) into token
 * positions [pos, pos + n_new).  Codes of other tokens sharing a 128-token
 * block are preserved.  Same arguments and errors as tq_append_key. */
int tq_append_value(tq_ctx* ctx, const tq_cache_view* cache, const void* v, int32_t dtype,
                    int64_t pos, int64_t n_new, void* stream);

/* The appends with a caller-owned device workspace in place of the
 * context's scratch buffer (the same results, bit for bit), so that appends
 * of one context may run on several streams at once: each concurrent call
 * needs a workspace of its own.  Only general-path appends of more than 16
 * tokens per slot use it (the tiled rotation / projection kernels keep the
 * key residual and the row norms there between launches);
 * tq_append_workspace_bytes gives its size, 0 when the append of n_new
 * tokens into n_seq slots uses no workspace (then workspace may be NULL)
 * or when an argument is invalid (the append itself reports which).  The
 * size is at most that of the context's scratch for n_seq <= 256 (4 d + 8 +
 * 4 ceil(d/128) bytes a row, 32768 rows), and n_seq x 128 rows beyond: with
 * a workspace, general-path appends of any slot count are built, while the
 * context's scratch serves bulk appends into at most 256 slots
 * (tq_append_key / tq_append_value return TQ_EUNSUPPORTED beyond).
 * workspace: device, 16-byte aligned, owned by the caller; it is free again
 * once the call's work on `stream` has finished.  Extra error:
 * TQ_EWORKSPACE if workspace_bytes < tq_append_workspace_bytes. */
size_t tq_append_workspace_bytes(const tq_ctx* ctx, int32_t n_seq, int64_t n_new);
int tq_append_key_ws(tq_ctx* ctx, const tq_cache_view* cache, const void* k, int32_t dtype, int64_t pos,
                     int64_t n_new, void* workspace, size_t workspace_bytes, void* stream);
int tq_append_value_ws(tq_ctx* ctx, const tq_cache_view* cache, const void* v, int32_t dtype, int64_t pos,
                       int64_t n_new, void* workspace, size_t workspace_bytes, void* stream);

/* Asymmetric attention scores straight from the packed keys
 * (asymmetric_attention_scores / attention_scores, nav.superapi.store
 * 常见使用模式 and 核心 API): scores[s][h][t] = est(q[s][h], k[s][t]),
 * unscaled, for t < n_tokens.
 * q: device [n_seq][G][d] (query head h of slot s uses KV slot s; GQA groups
 * of G contiguous heads), dtype TQ_F16 or TQ_F32.  1 <= G <= 512 (a
 * vector-search batch of queries against one slot is G queries, n_seq = 1).
 * scores: device fp32 [n_seq][G][n_tokens].
 * workspace: device, >= tq_attend_workspace_bytes(ctx, n_seq, G, n_tokens).
 * The call takes a workspace because each query is rotated and projected
 * once per call (q~ = R q, p = S q~, as split-fp16 matrix-core operands) into
 * device memory that the score kernel then streams the keys against; the
 * library allocates no device memory after tq_create, so that memory is the
 * caller's.
 * Errors: TQ_EINVAL (n_tokens <= 0 or > capacity, G out of range, ...),
 * TQ_ENOCODEBOOK, TQ_EWORKSPACE, TQ_EDEVICE. */
int tq_attention_scores(tq_ctx* ctx, const tq_cache_view* cache, const void* q, int32_t dtype,
                        int32_t G, int64_t n_tokens, float* scores, void* workspace,
                        size_t workspace_bytes, void* stream);

/* Attention over the packed cache: softmax over the first n_tokens of
 * scale * est, then the weighted sum of the dequantised values, rotated
 * back (nav.superapi.store 常见使用模式: scores from compressed keys,
 * softmax, weighted sum of the decompressed values).  scale <= 0 means
 * 1/sqrt(d).  No causal mask.  out: device fp32 [n_seq][G][d].
 * Same q/workspace rules and errors as tq_attention_scores, with
 * 1 <= G <= 16. */
int tq_attend(tq_ctx* ctx, const tq_cache_view* cache, const void* q, int32_t dtype, int32_t G,
              int64_t n_tokens, float scale, float* out, void* workspace, size_t workspace_bytes,
              void* stream);

/* tq_attend without the workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation).  The same results as tq_attend with the
 * same arguments.  The workspace is a static device array of 32 MiB that
 * the library holds on each GPU it runs on until the process ends (its
 * address is looked up when a context is created on that device); shapes
 * whose tq_attend_workspace_bytes exceeds 32 MiB are rejected with
 * TQ_EWORKSPACE before anything is launched.  Nothing is allocated.  Every
 * call on one GPU shares that array, so calls that overlap on one GPU (on
 * different streams, or from several threads or contexts) race; serialise
 * them.  Errors as tq_attend, plus TQ_EWORKSPACE for a shape too large and
 * TQ_EDEVICE if the scratch address is unknown for ctx's device. */
int tq_attend_noalloc(tq_ctx* ctx, const tq_cache_view* cache, const void* q, int32_t dtype, int32_t G,
                      int64_t n_tokens, float scale, float* out, void* stream);

/* One decode step: append n_new tokens' keys and values at token slots
 * [pos, pos + n_new) of every slot, then attend with q over the whole cache
 * [0, pos + n_new) -- the same results as tq_append_key, tq_append_value and
 * tq_attend called in that order (the streaming use of the cache,
 * nav.superapi.store 常见使用模式: append_key / append_value per token, then
 * attention over the compressed cache).  k, v: device [n_seq][n_new][d]; q:
 * device [n_seq][G][d]; all three of type dtype.  scale, out, workspace as
 * for tq_attend with n_tokens = pos + n_new (workspace >=
 * tq_attend_workspace_bytes(ctx, n_seq, G, pos + n_new)).  On the
 * single-kernel shapes (head_dim 128, proj_dim 64 or 128, G <= 16) with
 * n_new <= 16 (and at most 4096 partials per slot: attention workgroups +
 * 1, times G) the whole step is one kernel launch in which no workgroup
 * waits for another: attention workgroups over the tokens before pos (each
 * preparing the queries itself), one workgroup per slot that appends the
 * new tokens and forms their share of the softmax, and the merge, done by
 * the workgroup that completes the slot's arrival count at the start of the
 * workspace (a tagged word that the step sets up itself, so the workspace
 * needs no clearing; a replayed graph of the call works too).  The new
 * tokens' scores are taken in fp32, the others' as tq_attend does, so the
 * output equals the three calls' up to rounding.  Otherwise the three calls
 * run in order.  Calls that overlap on one workspace race.
 * Every argument is checked before anything is launched.  Errors: TQ_EINVAL
 * (including n_new < 1), TQ_ECAPACITY, TQ_ENOCODEBOOK, TQ_EWORKSPACE,
 * TQ_EDEVICE. */
int tq_decode_step(tq_ctx* ctx, const tq_cache_view* cache, const void* k, const void* v, int32_t dtype,
                   int64_t pos, int64_t n_new, const void* q, int32_t G, float scale, float* out, void* workspace,
                   size_t workspace_bytes, void* stream);

/* ---- vector search ----------------------------------------------------------- */

/* Device workspace bytes tq_topk_scores needs (query operands and per-wave
 * candidate lists).  0 on invalid arguments (cfg NULL/invalid, n_seq < 1,
 * G not in 1..512, n_tokens < 1, k not in 1..16). */
size_t tq_topk_workspace_bytes(const tq_config* cfg, int32_t n_seq, int32_t G, int64_t n_tokens, int32_t k);

/* The k best tokens of each query by the asymmetric score estimate, without
 * writing the n_seq x G x n_tokens scores (inner-product search over a
 * compressed database: ai-manual.ru article, Где TurboQuant выстреливает;
 * jansverre.net post, Hvem er dette nyttig for?).  The estimate is the one
 * tq_attention_scores returns.  top_scores: device fp32 [n_seq][G][k],
 * top_index: device int32 [n_seq][G][k] (token positions in the slot),
 * ordered by score descending, equal scores by position ascending; when
 * n_tokens < k the rest is (-inf, -1).  q as for tq_attention_scores,
 * 1 <= G <= 512, 1 <= k <= 16.  workspace >= tq_topk_workspace_bytes.
 * Errors: TQ_EINVAL, TQ_ENOCODEBOOK, TQ_EWORKSPACE, TQ_EDEVICE. */
int tq_topk_scores(tq_ctx* ctx, const tq_cache_view* cache, const void* q, int32_t dtype, int32_t G,
                   int64_t n_tokens, int32_t k, float* top_scores, int32_t* top_index, void* workspace,
                   size_t workspace_bytes, void* stream);

/* ---- reconstruction (not on the attention path) --------------------------- */

/* Stage-1 reconstruction of cached values, x^ = ||v|| R^T c[idx]
 * (TurboQuantKVCache.get_values and TurboQuantMSE.dequantize,
 * nav.superapi.store 核心 API; the value compressor keeps only this MSE
 * reconstruction, 生产级压缩器).  Tokens [pos, pos + n_tokens) of every slot.
 * out: device fp32 [n_seq][n_tokens][d], 16-byte aligned.  Computed in fp32
 * from the stored codes and norms.  Errors: TQ_EINVAL, TQ_ECAPACITY
 * (pos < 0 or pos + n_tokens > capacity), TQ_ENOCODEBOOK, TQ_EDEVICE.
 * n_tokens == 0 is a no-op. */
int tq_get_values(tq_ctx* ctx, const tq_cache_view* cache, int64_t pos, int64_t n_tokens, float* out,
                  void* stream);

/* The same reconstruction of cached keys from their stage-1 codes and norms,
 * ||k|| R^T c[idx] (the MSE part; the QJL sign bits estimate inner products
 * and do not reconstruct the residual; with key_bits 0 it is all zeros).
 * Same arguments and errors. */
int tq_get_keys(tq_ctx* ctx, const tq_cache_view* cache, int64_t pos, int64_t n_tokens, float* out,
                void* stream);

/* ---- measurement ------------------------------------------------------------ */

/* The HBM ceiling for the bandwidth-bound kernels above: stream read_bytes
 * from src and, if write_bytes > 0, write write_bytes of a constant fp32
 * pattern (1.0f) to dst, interleaved with the reads in their ratio; every
 * wave reads and writes contiguous spans, as the score and attend kernels
 * do.  The words read are XOR-folded into *sink (the caller initialises it;
 * the value only proves the reads happened).  Not part of the method: it
 * measures what a plain stream reaches on the device (the reported
 * baseline beside the theoretical peak).  src, dst: device, 16-byte aligned;
 * write_bytes 0, read_bytes, read_bytes / 2 or read_bytes / 4; sink: device
 * uint32; waves_per_cu: the grid's waves per compute unit, a multiple of 4
 * up to 64 (0: 16), since the best count depends on the read/write mix.
 * flags: bit 0 (TQ_STREAM_NONTEMPORAL) makes every load and store
 * nontemporal; bits 8-15 give the 16-byte loads each lane keeps in flight,
 * 4, 8 or 16 (0: 4); read_bytes must be a positive multiple of that many
 * KiB.  Errors: TQ_EINVAL, TQ_EDEVICE. */
#define TQ_STREAM_NONTEMPORAL 1
#define TQ_STREAM_LOADS(n) ((n) << 8)
int tq_hbm_stream(const void* src, size_t read_bytes, void* dst, size_t write_bytes, uint32_t* sink,
                  int32_t waves_per_cu, int32_t flags, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* TQ_H */
