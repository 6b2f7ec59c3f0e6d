// Measurement helpers of libqlprobe.so (include/qlprobe.h): a plain streaming
// read of a device byte range and an empty grid.  They are the yardsticks the
// benchmark puts next to the layer's kernels; none of them is a step of the
// method, and the layer library does not contain them.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/qlprobe.h"

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kProbeThreads = 256;

// Work group w reads kLoads * 4 KB starting at w * kLoads * 4 KB: load j of
// lane t is the 16 bytes at (j * 256 + t) * 16 of that span, so each load
// instruction of a wave covers 1 KB contiguous.  The XOR of everything read is
// stored only when it equals a fixed word, so the loads cannot be dropped.
template <int kLoads>
__global__ __launch_bounds__(kProbeThreads) void k_read_probe(const u32x4* __restrict__ p, int64_t n16,
                                                              uint32_t* __restrict__ sink) {
  const int64_t base = (int64_t)blockIdx.x * kProbeThreads * kLoads + threadIdx.x;
  u32x4 v[kLoads];
#pragma unroll
  for (int j = 0; j < kLoads; ++j) {
    const int64_t i = base + (int64_t)j * kProbeThreads;
    v[j] = i < n16 ? __builtin_nontemporal_load(p + i) : u32x4{0, 0, 0, 0};
  }
  uint32_t x = 0;
#pragma unroll
  for (int j = 0; j < kLoads; ++j) x ^= v[j][0] ^ v[j][1] ^ v[j][2] ^ v[j][3];
  if (x == 0x9E3779B9u) sink[0] = x;
}

__global__ void k_empty_probe() {}

template <int kLoads>
hipError_t launch_read(const void* data, int64_t n16, uint32_t* sink, hipStream_t s) {
  const int64_t per = (int64_t)kProbeThreads * kLoads;
  const int64_t grid = (n16 + per - 1) / per;
  if (grid < 1 || grid > 0x7FFFFFFF) return hipErrorInvalidValue;
  hipLaunchKernelGGL(k_read_probe<kLoads>, dim3((unsigned)grid), dim3(kProbeThreads), 0, s, (const u32x4*)data,
                     n16, sink);
  return hipGetLastError();
}

int status(hipError_t e) { return e == hipSuccess ? 0 : -6; }

}  // namespace

extern "C" {

int ql_read_probe(const void* data, int64_t bytes, int loads, uint32_t* sink, void* stream) {
  if (!data || !sink) return -1;
  if (bytes <= 0 || (bytes % 16) != 0 || bytes > (int64_t(1) << 40)) return -2;
  if (loads != 1 && loads != 2 && loads != 4 && loads != 8 && loads != 16) return -2;
  if ((reinterpret_cast<uintptr_t>(data) & 15u) != 0 || (reinterpret_cast<uintptr_t>(sink) & 3u) != 0) return -4;
  hipStream_t s = (hipStream_t)stream;
  const int64_t n16 = bytes / 16;
  switch (loads) {
    case 1: return status(launch_read<1>(data, n16, sink, s));
    case 2: return status(launch_read<2>(data, n16, sink, s));
    case 4: return status(launch_read<4>(data, n16, sink, s));
    case 8: return status(launch_read<8>(data, n16, sink, s));
    default: return status(launch_read<16>(data, n16, sink, s));
  }
}

int ql_empty_probe(int64_t groups, int threads, void* stream) {
  if (groups < 1 || groups > 0x7FFFFFFF || threads < 1 || threads > 1024) return -2;
  hipLaunchKernelGGL(k_empty_probe, dim3((unsigned)groups), dim3(threads), 0, (hipStream_t)stream);
  return status(hipGetLastError());
}

}  // extern "C"
