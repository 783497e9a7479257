// Appends of a few tokens per slot (a decode step appends one), for any
// shape of the layout.  The bulk kernels stage R (and S) images in LDS and
// fill whole 16- to 64-token matrix-core tiles; for a handful of tokens that
// set-up is most of their time.  Here the arithmetic runs in fp32 on the
// vector units with R and S read from L2 (they are shared by every
// workgroup): stage 1 (nav.superapi.store "turboquant-pytorch", 主要能力;
// atskills.one Stage 1): n = ||x||, y = R x / n, idx = #{i : beta_i < y};
// keys also take stage 2 (atskills.one Stage 2): r = y - c[idx],
// gamma = ||r||, s = [S r >= 0].  fp32 dot products of d terms are within
// about 1e-7 of the exact values, inside the tolerance of the codes.
//
//   small_keys_kernel:   one workgroup per (slot, new token); writes the
//                        token's record.
//   small_values_kernel: one workgroup per (slot, touched 128-token block);
//                        the block's new tokens are coded one after the
//                        other and each code word is read, merged and
//                        written by one thread (words are shared by tokens).
#include <algorithm>

#include "tq_small.h"

namespace tq {

__global__ __launch_bounds__(kSmallThreads) void small_keys_kernel(const SmallArgs a) {
  small_keys_block(a, a.bid0 + blockIdx.x);
}

__global__ __launch_bounds__(kSmallThreads) void small_values_kernel(const SmallArgs a) {
  small_values_block(a, blockIdx.x);
}


int small_device_init() {
  // up to head_dim 1024: values keep 16 x d cells plus 2 d floats in LDS
  const int lds = (int)(sizeof(float) * (2 * 1024 + 16 * 1024));
  const bool ok =
      hipFuncSetAttribute((const void*)small_values_kernel, hipFuncAttributeMaxDynamicSharedMemorySize, lds) ==
          hipSuccess;
  return ok ? 0 : -1;
}

int launch_small_keys(const Matrices& mats, const CodebookDev& cb, int bits, int d, int m, const AppendShape& s,
                      void* key_records, void* stream) {
  SmallArgs a = small_args(mats, cb, bits, d, m, s, key_records);
  const size_t lds = sizeof(float) * (size_t)(4 * d + m);
  // one workgroup per (slot, token); launches of at most 2^23 workgroups
  // keep the grid's thread count within 32 bits
  const int64_t total = (int64_t)s.n_seq * s.n_new, chunk = (int64_t)1 << 23;
  for (a.bid0 = 0; a.bid0 < total; a.bid0 += chunk) {
    const int64_t nb = std::min(chunk, total - a.bid0);
    hipLaunchKernelGGL(small_keys_kernel, dim3((unsigned)nb), dim3(kSmallThreads), lds, (hipStream_t)stream, a);
    if (hipGetLastError() != hipSuccess) return TQ_EDEVICE;
  }
  return 0;
}

int launch_small_values(const Matrices& mats, const CodebookDev& cb, int bits, int d, const AppendShape& s,
                        void* value_blocks, void* stream) {
  const SmallArgs a = small_args(mats, cb, bits, d, 64, s, value_blocks);
  const int64_t nblk = (s.pos + s.n_new - 1) / kBlockTokens - s.pos / kBlockTokens + 1;
  const size_t lds = sizeof(float) * (size_t)(2 * d + kSmallAppend * d);
  hipLaunchKernelGGL(small_values_kernel, dim3((unsigned)(s.n_seq * nblk)), dim3(kSmallThreads), lds,
                     (hipStream_t)stream, a);
  return hipGetLastError() == hipSuccess ? 0 : TQ_EDEVICE;
}

}  // namespace tq
