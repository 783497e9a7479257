// Internal declarations shared by the host API and the kernel launchers.
#pragma once

#include <cstddef>
#include <cstdint>

#include "../../include/tq.h"

namespace tq {

// Record failure `code` with a printf-style message; returns code.
int fail(int code, const char* fmt, ...);
void clear_error();

bool lloyd_max_standard(int bits, double* c, double* beta);

constexpr int kD = 128;          // head_dim of the built fast path
constexpr int kLdsStride = 136;  // padded fp16 row stride of R / S images (conflict-free b128 reads)
constexpr int kBlockTokens = 128;
constexpr int64_t kMaxCapacity = int64_t(1) << 24;  // tokens per slot: in-slot word offsets fit 32 bits
constexpr float kRotScale = 256.0f;   // R and S images are scaled by 2^8 before the hi/lo fp16 split
constexpr float kResScale = 4096.0f;  // residual scaled by 2^12 before its hi/lo split

// Per-bits codebook as the kernels consume it.
struct CodebookDev {
  float beta[16];   // boundaries, +inf past the last
  float cent[16];   // centroids fp32
  uint32_t tlo[4];  // low bytes of fp16(centroid v) at byte v (16 entries)
  uint32_t thi[4];  // high bytes
};

struct Matrices {
  const uint16_t* r_hi;  // [d][kLdsStride] fp16 bits, R * 2^8 high part (row = output coordinate)
  const uint16_t* r_lo;
  const uint16_t* s_hi;  // [m][kLdsStride] fp16 bits, S * 2^8 high part, columns in slot order
  const uint16_t* s_lo;
  const uint16_t* s_hi32;  // the same for d = 128 with columns in 32-lane slot order
  const uint16_t* s_lo32;
  const float* r32;      // [d][d] fp32 R
  const float* s32;      // [m][d] fp32 S (natural column order)
  const uint16_t* rt_hi;  // [d][kLdsStride] R^T * 2^8 hi / lo (d = 128, m in {64, 128}: the fused decode step)
  const uint16_t* rt_lo;
  const uint16_t* p_hi;   // [m][kLdsStride] (S R) * 2^8 hi / lo (the same shapes)
  const uint16_t* p_lo;
};

// ---- launchers (defined in the .hip files) -----------------------------------

struct AppendShape {
  const void* x;
  int dtype;         // TQ_F16 / TQ_F32
  int64_t n_new, pos, capacity;
  int n_seq;
};

int launch_compress_keys(const Matrices& mats, const CodebookDev& cb, int bits, int m,
                         const AppendShape& s, void* key_records, void* stream);
int launch_dequant(const Matrices& mats, const CodebookDev& cb, int bits, int d, int m, bool keys,
                   const void* key_records, const void* value_blocks, int64_t capacity, int n_seq, int64_t pos,
                   int64_t n_tokens, float* out, void* stream);
int dequant_device_init();
int launch_compress_values(const Matrices& mats, const CodebookDev& cb, int bits,
                           const AppendShape& s, void* value_blocks, void* stream);

struct AttnShape {
  const void* q;
  int dtype;
  int G;
  int64_t n_tokens, capacity;
  int n_seq;
};

// Workspace partition for the attention calls.
struct AttnPlan {
  int waves_per_slot;      // split of the token axis for tq_attend
  int blocks_per_wave;
  size_t q_bytes;          // prepared query operands
  size_t qn_bytes;         // query norms
  size_t part_bytes;       // attend partials
  size_t sync_bytes;       // counters and status word of the fused decode step
  size_t group_bytes;      // the fused decode step's workgroup partials
  size_t total;
};
AttnPlan plan_attention(int m, int n_seq, int G, int64_t n_tokens);
int attention_device_init();

int launch_prep_queries(const Matrices& mats, int m, const AttnShape& s, void* ws, const AttnPlan& p,
                        void* stream);
// Query preparation on the matrix cores for one head group at head_dim 128
// (the decode step's preparation, one workgroup per slot; tq_step.hip).
int launch_prep_step(const Matrices& mats, int m, const AttnShape& s, uint16_t* wq, float* wqn, void* stream);
int launch_scores(const CodebookDev& cbk, int kbits, int m, const AttnShape& s, const void* key_records,
                  float* scores, void* ws, const AttnPlan& p, void* stream);
int launch_attend(const Matrices& mats, const CodebookDev& cbk, int kbits, const CodebookDev& cbv, int vbits,
                  int m, const AttnShape& s, const void* key_records, const void* value_blocks, float scale,
                  float* out, void* ws, const AttnPlan& p, void* stream);
int compress_device_init();

// General-shape path (tq_general.hip): head_dim a multiple of 64 up to 1024,
// proj_dim a multiple of 32 up to 512.
constexpr int kMaxGeneralHeads = 512;   // query heads per KV slot for general scores
struct GenMats {
  Matrices mats;         // R / S images (row stride ld halves) and fp32 copies
  int ld;                // d + 8
  float* nrm;            // scratch: [scratch_rows] (shifted norm, exponent) pairs
  uint16_t* res_hi;      // scratch: [scratch_rows][d] key residual, fp16 high part
  uint16_t* res_lo;      //          and low part
  float* g2p;            // scratch: [scratch_rows][d/128] residual square sums
  int64_t scratch_rows;
};
int launch_general_keys(const GenMats& g, const CodebookDev& cb, int bits, int d, int m, const AppendShape& s,
                        void* key_records, void* stream);
int launch_general_values(const GenMats& g, const CodebookDev& cb, int bits, int d, const AppendShape& s,
                          void* value_blocks, void* stream);
size_t general_scores_workspace(int d, int m, int n_seq, int G);
// Query operands for HG groups of 16 heads: wq [n_seq][HG][d/32 + m/32][64][8] fp16, wqn [n_seq][16 HG]
// (with HG = 1 the layout the single-kernel score and attend kernels read).
int launch_gen_prep(const Matrices& mats, int d, int m, const AttnShape& s, int HG, uint16_t* wq, float* wqn,
                    void* stream);
struct GenAttnPlan {
  int blocks_per_wave, ranges;  // split of each slot's token axis for the value accumulation
  size_t off_scores;            // materialised scores [n_seq][G][n_tokens] fp32
  size_t off_part;              // partials [n_seq][ranges][d/128][G][132] fp32
  size_t total;
};
GenAttnPlan general_attend_plan(int d, int m, int n_seq, int G, int64_t n_tokens);
int launch_general_attend(const Matrices& mats, const CodebookDev& cbk, int kbits, const CodebookDev& cbv, int vbits,
                          int d, int m, const AttnShape& s, const void* key_records, const void* value_blocks,
                          float scale, float* out, void* ws, void* stream);
int launch_general_scores(const Matrices& mats, const CodebookDev& cbk, int kbits, int d, int m,
                          const AttnShape& s, const void* key_records, float* scores, void* ws, void* stream);

// Appends of at most kSmallAppend tokens per slot (tq_small.hip): fp32
// vector arithmetic with R and S from L2, for any shape.
constexpr int kSmallAppend = 16;
int small_device_init();
int launch_small_keys(const Matrices& mats, const CodebookDev& cb, int bits, int d, int m, const AppendShape& s,
                      void* key_records, void* stream);
int launch_small_values(const Matrices& mats, const CodebookDev& cb, int bits, int d, const AppendShape& s,
                        void* value_blocks, void* stream);

// The whole decode step in one launch (tq_step.hip) serves shapes whose
// workgroup partials per slot (attend workgroups + 1, x G) are at most this
// many: one workgroup merges them, and beyond this the merge would take
// longer than the separate launches of the three calls.
constexpr int kStepMaxPartials = 4096;
int decode_step_device_init();  // (tq_step.hip; called by attention_device_init)
// The whole decode step in one launch (tq_step.hip): the appends, the query
// preparation, the attention over the cache and the merge of the partials,
// ordered by one arrival count per slot in the workspace.
int launch_decode_step(const Matrices& mats, const CodebookDev& cbk, int kbits, const CodebookDev& cbv, int vbits,
                       int d, int m, const AppendShape& ks, const AppendShape& vs, const AttnShape& s,
                       void* key_records, void* value_blocks, float scale, float* out, void* ws, const AttnPlan& p,
                       void* stream);

// Device scratch of tq_attend_noalloc (tq_attention.hip): a static device
// array of kNoAllocScratchBytes per GPU.  noalloc_scratch_init looks up its
// address on `device` (which must be current) once; noalloc_scratch_ptr
// returns it (nullptr before the look-up).
constexpr size_t kNoAllocScratchBytes = size_t(32) << 20;
int noalloc_scratch_init(int device);
void* noalloc_scratch_ptr(int device);

// HBM stream for measuring the memory ceiling (tq_stream.hip).
int stream_device_init();
int launch_stream(const void* src, size_t read_bytes, void* dst, size_t write_bytes, uint32_t* sink,
                  int waves_per_cu, int loads_in_flight, bool nontemporal, void* stream);

// Fused inner-product top-k over the packed keys (tq_topk.hip).
constexpr int kTopkMax = 16;  // largest k of tq_topk_scores
struct TopkPlan {
  int HG, n_qblk, n_ranges, n_lists;
  int64_t tiles_per_range;
  size_t q_bytes, qn_bytes, cand_bytes, total;
};
TopkPlan topk_plan(int d, int m, int n_seq, int G, int64_t n_tokens, int k);
int topk_device_init();
int launch_topk(const Matrices& mats, const CodebookDev& cbk, int kbits, int d, int m, const AttnShape& s, int k,
                const void* key_records, float* top_s, int32_t* top_i, void* ws, void* stream);

}  // namespace tq
