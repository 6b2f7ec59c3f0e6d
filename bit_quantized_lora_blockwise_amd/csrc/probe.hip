// Streaming read of a device byte range: the achievable-bandwidth ceiling that
// the decode kernel's packed-weight rate is compared against (a measurement
// helper, not a step of the method).
#include "kernels.h"

namespace {

constexpr int kProbeThreads = 256;
constexpr int kProbeLoads = 4;   // 16-byte loads in flight per thread

// Work group w reads 16 KB at 16 KB * w: load j of lane t is the 16 bytes at
// (j * 256 + t) * 16 of that span (each load instruction of a wave covers 1 KB
// contiguous).  The XOR of everything read is stored only when it equals a
// fixed word, so the loads cannot be dropped.
__global__ __launch_bounds__(kProbeThreads) void k_read_probe(const u32x4* __restrict__ p, int64_t n16,
                                                              uint32_t* __restrict__ sink) {
  const int64_t base = (int64_t)blockIdx.x * kProbeThreads * kProbeLoads + threadIdx.x;
  u32x4 v[kProbeLoads];
#pragma unroll
  for (int j = 0; j < kProbeLoads; ++j) {
    const int64_t i = base + (int64_t)j * kProbeThreads;
    v[j] = i < n16 ? __builtin_nontemporal_load(p + i) : u32x4{0, 0, 0, 0};
  }
  uint32_t x = 0;
#pragma unroll
  for (int j = 0; j < kProbeLoads; ++j) x ^= v[j][0] ^ v[j][1] ^ v[j][2] ^ v[j][3];
  if (x == 0x9E3779B9u) sink[0] = x;
}

}  // namespace

hipError_t launch_read_probe(const void* data, int64_t bytes, uint32_t* sink, hipStream_t s) {
  const int64_t n16 = bytes / 16;
  const int64_t per = (int64_t)kProbeThreads * kProbeLoads;
  const int64_t grid = (n16 + per - 1) / per;
  if (grid < 1 || grid > 0x7FFFFFFF) return hipErrorInvalidValue;
  hipLaunchKernelGGL(k_read_probe, dim3((unsigned)grid), dim3(kProbeThreads), 0, s, (const u32x4*)data, n16, sink);
  return hipGetLastError();
}
