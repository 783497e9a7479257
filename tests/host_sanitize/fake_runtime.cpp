// Host-only stand-ins for the HIP runtime calls and the kernel launchers that
// tq_api.cpp makes, so that the C ABI's host logic (argument checks, size
// queries, the R / S images built in tq_create, codebook tables, workspace
// partitions) runs under AddressSanitizer and UndefinedBehaviorSanitizer on
// a machine without a GPU.  "Device" memory is host memory; a launcher
// records the call and checks the buffers it was handed lie inside the
// allocations the caller made (each launch touches the first and the last
// byte of its output buffers, which ASan turns into an error if a size
// query and the call disagree).
#include <hip/hip_runtime_api.h>

#include <algorithm>
#include <cstdint>
#include <cstdlib>
#include <cstring>

#include "../../kv_cache_vector_compress_amd/csrc/tq_internal.h"

int g_launches = 0;

extern "C" {
hipError_t hipSetDevice(int device) { return device == 0 ? hipSuccess : hipErrorInvalidDevice; }
hipError_t hipGetDevice(int* device) {
  *device = 0;
  return hipSuccess;
}
hipError_t hipMalloc(void** ptr, size_t size) {  // exactly `size` bytes, 256-byte aligned
  *ptr = nullptr;
  return posix_memalign(ptr, 256, size ? size : 1) == 0 ? hipSuccess : hipErrorOutOfMemory;
}
hipError_t hipFree(void* ptr) {
  std::free(ptr);
  return hipSuccess;
}
hipError_t hipMemcpy(void* dst, const void* src, size_t n, hipMemcpyKind) {
  std::memcpy(dst, src, n);
  return hipSuccess;
}
}

namespace tq {

static unsigned char g_scratch[kNoAllocScratchBytes];

// The first and last byte of [p, p + n): ASan reports an access outside the
// allocation p came from.
static void touch(const void* p, size_t n) {
  if (!p || !n) return;
  volatile const unsigned char* b = (const unsigned char*)p;
  (void)b[0];
  (void)b[n - 1];
}
static int launched() {
  ++g_launches;
  return 0;
}

int compress_device_init() { return 0; }
int attention_device_init() { return 0; }
int dequant_device_init() { return 0; }
int topk_device_init() { return 0; }
int small_device_init() { return 0; }
int stream_device_init() { return 0; }
int noalloc_scratch_init(int device) { return device == 0 ? 0 : -1; }
void* noalloc_scratch_ptr(int device) { return device == 0 ? g_scratch : nullptr; }

// Workspace plans: fixed partitions that grow with every argument (the real
// ones live with their kernels).
AttnPlan plan_attention(int m, int n_seq, int G, int64_t n_tokens) {
  AttnPlan p{};
  p.waves_per_slot = 64;
  p.blocks_per_wave = (int)((n_tokens + 64 * 128 - 1) / (64 * 128));
  p.q_bytes = (size_t)n_seq * (4 + m / 32) * 64 * 8 * 2;
  p.qn_bytes = (size_t)n_seq * 16 * 4;
  p.part_bytes = (size_t)n_seq * 64 * G * 132 * 4;
  p.sync_bytes = (size_t)n_seq * 40 * 8 + 16;
  p.group_bytes = (size_t)n_seq * 18 * G * 132 * 4;
  p.total = p.q_bytes + p.qn_bytes + p.part_bytes + p.sync_bytes + p.group_bytes;
  return p;
}
size_t general_scores_workspace(int d, int m, int n_seq, int G) {
  return (size_t)n_seq * ((G + 15) / 16) * ((d / 32 + m / 32) * 64 * 8 * 2 + 16 * 4);
}
GenAttnPlan general_attend_plan(int d, int m, int n_seq, int G, int64_t n_tokens) {
  GenAttnPlan p{};
  p.blocks_per_wave = 4;
  p.ranges = (int)((n_tokens + 511) / 512);
  p.off_scores = general_scores_workspace(d, m, n_seq, G);  // the score workspace is the plan's prefix
  p.off_part = p.off_scores + (size_t)n_seq * G * n_tokens * 4;
  p.total = p.off_part + (size_t)n_seq * p.ranges * ((d + 127) / 128) * G * 132 * 4;
  return p;
}
TopkPlan topk_plan(int d, int m, int n_seq, int G, int64_t n_tokens, int k) {
  TopkPlan p{};
  p.HG = (G + 15) / 16;
  p.n_qblk = (p.HG + 1) / 2;
  p.n_ranges = (int)((n_tokens + 1023) / 1024);
  p.n_lists = p.n_ranges * 8;
  p.tiles_per_range = 64;
  p.q_bytes = (size_t)n_seq * p.HG * (d / 32 + m / 32) * 64 * 8 * 2;
  p.qn_bytes = (size_t)n_seq * p.HG * 16 * 4;
  p.cand_bytes = (size_t)n_seq * G * p.n_lists * k * 4;
  p.total = p.q_bytes + p.qn_bytes + 2 * p.cand_bytes;
  return p;
}

// Launchers: touch the buffers the caller sized, then count the launch.
static size_t rec_bytes(int bits, int d, int m) { return 4u * (bits * d / 32 + m / 32 + 2); }

int launch_compress_keys(const Matrices& mats, const CodebookDev&, int bits, int m, const AppendShape& s,
                         void* key_records, void*) {
  touch(mats.r_hi, 2);
  touch(key_records, (size_t)s.n_seq * s.capacity * rec_bytes(bits, 128, m));
  touch(s.x, (size_t)s.n_seq * s.n_new * 128 * (s.dtype == TQ_F32 ? 4 : 2));
  return launched();
}
int launch_compress_values(const Matrices&, const CodebookDev&, int bits, const AppendShape& s, void* value_blocks,
                           void*) {
  touch(value_blocks, (size_t)s.n_seq * (s.capacity / 128) * 4 * (4 * bits * 128 + 128));
  return launched();
}
int launch_small_keys(const Matrices& mats, const CodebookDev&, int bits, int d, int m, const AppendShape& s,
                      void* key_records, void*) {
  touch(mats.r32, (size_t)d * d * 4);
  touch(mats.s32, (size_t)m * d * 4);
  touch(key_records, (size_t)s.n_seq * s.capacity * rec_bytes(bits, d, m));
  touch(s.x, (size_t)s.n_seq * s.n_new * d * (s.dtype == TQ_F32 ? 4 : 2));
  return launched();
}
int launch_small_values(const Matrices& mats, const CodebookDev&, int bits, int d, const AppendShape& s,
                        void* value_blocks, void*) {
  touch(mats.r32, (size_t)d * d * 4);
  touch(value_blocks, (size_t)s.n_seq * (s.capacity / 128) * 4 * (4 * bits * d + 128));
  return launched();
}
int launch_general_keys(const GenMats& g, const CodebookDev&, int bits, int d, int m, const AppendShape& s,
                        void* key_records, void*) {
  int64_t sub = g.scratch_rows / s.n_seq;
  sub -= sub % 128;
  if (sub < 128) sub = 128;
  if (sub * s.n_seq > g.scratch_rows) return TQ_EUNSUPPORTED;
  const int64_t rows = std::min<int64_t>(sub, s.n_new) * s.n_seq;
  touch(g.nrm, (size_t)rows * 8);
  touch(g.res_hi, (size_t)rows * d * 2);
  touch(g.res_lo, (size_t)rows * d * 2);
  touch(g.g2p, (size_t)rows * ((d + 127) / 128) * 4);
  // the padded images: 128 ceil(d / 128) rows of R, 64 ceil(m / 64) rows of S
  touch(g.mats.r_hi, (size_t)128 * ((d + 127) / 128) * g.ld * 2);
  touch(g.mats.s_hi, (size_t)64 * ((m + 63) / 64) * g.ld * 2);
  touch(key_records, (size_t)s.n_seq * s.capacity * rec_bytes(bits, d, m));
  return launched();
}
int launch_general_values(const GenMats& g, const CodebookDev&, int bits, int d, const AppendShape& s,
                          void* value_blocks, void*) {
  int64_t sub = g.scratch_rows / s.n_seq;
  sub -= sub % 128;
  if (sub < 128) sub = 128;
  if (sub * s.n_seq > g.scratch_rows) return TQ_EUNSUPPORTED;
  touch(g.nrm, (size_t)std::min<int64_t>(sub, s.n_new) * s.n_seq * 8);
  touch(value_blocks, (size_t)s.n_seq * (s.capacity / 128) * 4 * (4 * bits * d + 128));
  return launched();
}
int launch_prep_queries(const Matrices&, int, const AttnShape&, void* ws, const AttnPlan& p, void*) {
  touch(ws, p.total);
  return launched();
}
int launch_scores(const CodebookDev&, int, int, const AttnShape& s, const void*, float* scores, void* ws,
                  const AttnPlan& p, void*) {
  touch(ws, p.total);
  touch(scores, (size_t)s.n_seq * s.G * s.n_tokens * 4);
  return launched();
}
int launch_attend(const Matrices&, const CodebookDev&, int, const CodebookDev&, int, int, const AttnShape& s,
                  const void*, const void*, float, float* out, void* ws, const AttnPlan& p, void*) {
  touch(ws, p.total);
  touch(out, (size_t)s.n_seq * s.G * 128 * 4);
  return launched();
}
int launch_general_attend(const Matrices&, const CodebookDev&, int, const CodebookDev&, int, int d, int m,
                          const AttnShape& s, const void*, const void*, float, float* out, void* ws, void*) {
  touch(ws, general_attend_plan(d, m, s.n_seq, s.G, s.n_tokens).total);
  touch(out, (size_t)s.n_seq * s.G * d * 4);
  return launched();
}
int launch_general_scores(const Matrices&, const CodebookDev&, int, int d, int m, const AttnShape& s, const void*,
                          float* scores, void* ws, void*) {
  touch(ws, general_scores_workspace(d, m, s.n_seq, s.G));
  touch(scores, (size_t)s.n_seq * s.G * s.n_tokens * 4);
  return launched();
}
int launch_decode_step(const Matrices&, const CodebookDev&, int, const CodebookDev&, int, int d, int,
                       const AppendShape& ks, const AppendShape& vs, const AttnShape& s, void*, void*, float,
                       float* out, void* ws, const AttnPlan& p, void*) {
  touch(ws, p.total);
  touch(out, (size_t)s.n_seq * s.G * d * 4);
  touch(ks.x, (size_t)ks.n_seq * ks.n_new * d * (ks.dtype == TQ_F32 ? 4 : 2));
  touch(vs.x, (size_t)vs.n_seq * vs.n_new * d * (vs.dtype == TQ_F32 ? 4 : 2));
  return launched();
}
int launch_topk(const Matrices&, const CodebookDev&, int, int d, int m, const AttnShape& s, int k, const void*,
                float* top_s, int32_t* top_i, void* ws, void*) {
  touch(ws, topk_plan(d, m, s.n_seq, s.G, s.n_tokens, k).total);
  touch(top_s, (size_t)s.n_seq * s.G * k * 4);
  touch(top_i, (size_t)s.n_seq * s.G * k * 4);
  return launched();
}
int launch_dequant(const Matrices&, const CodebookDev&, int, int d, int, bool, const void*, const void*, int64_t,
                   int n_seq, int64_t, int64_t n_tokens, float* out, void*) {
  touch(out, (size_t)n_seq * n_tokens * d * 4);
  return launched();
}
int launch_stream(const void* src, size_t read_bytes, void* dst, size_t write_bytes, uint32_t* sink, int, int, bool,
                  void*) {
  touch(src, read_bytes);
  touch(dst, write_bytes);
  touch(sink, 4);
  return launched();
}

}  // namespace tq
