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
#include <mutex>
#include <type_traits>

#include "tq_attend.h"

namespace tq {

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
  return decode_step_device_init();
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
  p.sync_bytes = (size_t)n_seq * 8;  // fused decode step: an arrival count per slot
  p.group_bytes = (size_t)n_seq * (p.waves_per_slot / 4 + 2) * G * kPartFloats * 4;  // its workgroup partials
  p.total = ((p.q_bytes + 255) / 256 + (p.qn_bytes + 255) / 256 + (p.part_bytes + 255) / 256 +
             (p.sync_bytes + 255) / 256 + (p.group_bytes + 255) / 256) * 256;
  return p;
}

int launch_prep_queries(const Matrices& mats, int m, const AttnShape& s, void* ws, const AttnPlan& p,
                        void* stream) {
  // one workgroup per (slot, head), wave-parallel dot products (tq_general.hip);
  // with a single head group its operands have the layout read here
  const WsPtrs w = ws_ptrs(ws, p);
  return launch_gen_prep(mats, kD, m, s, 1, w.wq, w.wqn, stream);
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

}  // namespace tq
