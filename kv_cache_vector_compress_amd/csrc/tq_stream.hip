// HBM stream kernel for gfx950: the memory ceiling the bandwidth-bound
// kernels of the attention path are measured against.  Not part of the
// method; it moves bytes the way those kernels do and nothing else.
//
// Each wave owns a contiguous span of the source and reads it in groups of
// NL 1 KB blocks (one 16-byte load per lane per block, NL loads in flight),
// folding the words into one XOR so the loads cannot be dropped.  With
// writes, after each group it stores NL / rpw blocks of the matching
// contiguous span of the destination (rpw = read bytes per written byte: 1,
// 2 or 4), interleaving reads and writes in the ratio of the score kernel
// (64 B of key record read per 16 B of scores written at G = 4).  NT makes
// every load and store nontemporal (streamed past the caches' normal
// retention), which on this chip moves a plain stream closer to the
// datasheet bandwidth.
#include "tq_device.h"

namespace tq {

struct StreamArgs {
  const u4* src;
  u4* dst;
  int64_t groups;  // NL KB read groups
  int rpw;         // read bytes per written byte; 0: no writes
  uint32_t* sink;
};

template <int NL, bool NT>
__global__ __launch_bounds__(256) void stream_kernel(const StreamArgs a) {
  const int lane = threadIdx.x & 63;
  const int64_t waves = (int64_t)gridDim.x * (blockDim.x >> 6);
  const int64_t gw = (int64_t)blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6);
  const int64_t g0 = gw * a.groups / waves, g1 = (gw + 1) * a.groups / waves;
  const u4 fill = {0x3F800000u, 0x3F800000u, 0x3F800000u, 0x3F800000u};
  uint32_t acc = 0u;
  for (int64_t g = g0; g < g1; ++g) {
    const u4* s = a.src + g * (64 * NL) + lane;  // 64 NL u4 = NL KB
    u4 v[NL];
#pragma unroll
    for (int j = 0; j < NL; ++j) v[j] = NT ? __builtin_nontemporal_load(s + 64 * j) : s[64 * j];
#pragma unroll
    for (int j = 0; j < NL; ++j) acc ^= (v[j][0] ^ v[j][1]) ^ (v[j][2] ^ v[j][3]);
    if (a.rpw > 0) {
      const int nb = NL / a.rpw;  // 1 KB blocks written per group
      u4* d = a.dst + (g * nb) * 64 + lane;
      for (int j = 0; j < nb; ++j) {
        if (NT) __builtin_nontemporal_store(fill, d + 64 * j);
        else d[64 * j] = fill;
      }
    }
  }
  // fold the wave's words into the sink (a device word the caller reads)
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) acc ^= (uint32_t)__shfl_xor((int)acc, o, 64);
  if (lane == 0) atomicXor(a.sink, acc);
}

static int g_stream_cus = 0;

int stream_device_init() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return -1;
  return hipDeviceGetAttribute(&g_stream_cus, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess ? 0 : -1;
}

int launch_stream(const void* src, size_t read_bytes, void* dst, size_t write_bytes, uint32_t* sink,
                  int waves_per_cu, int loads_in_flight, bool nontemporal, void* stream) {
  StreamArgs a;
  a.src = (const u4*)src;
  a.dst = (u4*)dst;
  a.groups = (int64_t)(read_bytes / (1024 * (size_t)loads_in_flight));
  a.rpw = write_bytes == 0 ? 0 : (int)(read_bytes / write_bytes);
  a.sink = sink;
  const int64_t waves = (int64_t)(g_stream_cus > 0 ? g_stream_cus : 256) * waves_per_cu;
  const dim3 grid((unsigned)(waves / 4)), block(256);
  hipStream_t st = (hipStream_t)stream;
#define TQ_ST(NL, NT) \
  if (loads_in_flight == NL && nontemporal == NT) hipLaunchKernelGGL((stream_kernel<NL, NT>), grid, block, 0, st, a);
  TQ_ST(4, false) TQ_ST(8, false) TQ_ST(16, false) TQ_ST(4, true) TQ_ST(8, true) TQ_ST(16, true)
#undef TQ_ST
  return hipGetLastError() == hipSuccess ? 0 : TQ_EDEVICE;
}

}  // namespace tq
