// Streaming-read probe: the read bandwidth the partial kernels' loads can
// reach on this device, reported next to the published HBM peak.  Every
// thread streams 16-byte non-temporal loads over a grid-strided range of the
// buffer (the load form the KV gather uses) and folds them into one word,
// which is stored only if it equals a value it never takes in practice, so
// the loads cannot be dropped and nothing is written.
#include "pa_device.h"
#include "pa_launch.h"

namespace pa {
namespace {

constexpr int kProbeThreads = 256;
constexpr int kProbeUnroll = 8;   // loads in flight per thread

__global__ __launch_bounds__(kProbeThreads) void stream_read(const u32x4* src, size_t n16,
                                                             uint32_t* sink) {
  const size_t stride = (size_t)gridDim.x * kProbeThreads;
  size_t i = (size_t)blockIdx.x * kProbeThreads + threadIdx.x;
  uint32_t acc = 0;
  for (; i + (kProbeUnroll - 1) * stride < n16; i += kProbeUnroll * stride) {
    u32x4 v[kProbeUnroll];
#pragma unroll
    for (int u = 0; u < kProbeUnroll; ++u) v[u] = __builtin_nontemporal_load(src + i + u * stride);
#pragma unroll
    for (int u = 0; u < kProbeUnroll; ++u) acc ^= v[u][0] ^ v[u][1] ^ v[u][2] ^ v[u][3];
  }
  for (; i < n16; i += stride) {
    const u32x4 v = __builtin_nontemporal_load(src + i);
    acc ^= v[0] ^ v[1] ^ v[2] ^ v[3];
  }
  if (acc == 0x9E3779B9u) sink[0] = acc;
}

}  // namespace

hipError_t launch_stream_read(const void* src, size_t bytes, uint32_t* sink, int cus,
                              hipStream_t st) {
  const size_t n16 = bytes / 16;
  // 8 workgroups of 4 waves per CU keep enough loads in flight to saturate HBM
  const size_t want = (size_t)(cus > 0 ? cus : 256) * 8;
  const size_t per_wg = (size_t)kProbeThreads * kProbeUnroll;
  size_t blocks = (n16 + per_wg - 1) / per_wg;
  if (blocks > want) blocks = want;
  if (blocks < 1) blocks = 1;
  hipLaunchKernelGGL(stream_read, dim3((unsigned)blocks), dim3(kProbeThreads), 0, st,
                     static_cast<const u32x4*>(src), n16, sink);
  return hipGetLastError();
}

}  // namespace pa
