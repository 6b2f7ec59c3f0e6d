// qlora_linear_fwd for callers that cannot allocate device memory (code under
// HIP graph capture, tight serving loops, harnesses that forbid hipMalloc):
// the same kernels, with the forward's scratch -- T when the caller keeps no
// T_out, and the fp32 partial sums of T = X L1 -- in a file-scope device array
// instead of a caller-supplied workspace.  Every element of the scratch that a
// kernel reads is written earlier in the same call, so nothing needs clearing.
#include <mutex>

#include "../../include/qlora.h"
#include "kernels.h"

namespace {

static_assert(QL_NOALLOC_SCRATCH_BYTES % 256 == 0, "scratch size is a multiple of its alignment");

// One copy per GPU, held until the process ends.  In host code this name is a
// host-side stand-in, never a device address: kernels get the address that
// hipGetSymbolAddress returns for the current device.
static __device__ __align__(256) unsigned char scratch[QL_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void* g_ptr[kMaxDevices] = {};

// Device address of this GPU's scratch array, looked up once per device (the
// device is current here) and kept.
hipError_t scratch_ptr(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_mu);
  if (!g_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    g_ptr[dev] = p;
  }
  *out = g_ptr[dev];
  return hipSuccess;
}

}  // namespace

extern "C" int qlora_linear_fwd_noalloc(const uint16_t* X, int64_t M, int64_t K, int64_t N, const uint8_t* codes,
                                        const uint8_t* c2, const float* c1, const uint16_t* L1, const uint16_t* L2,
                                        int r, float lora_scale, uint16_t* Y, uint16_t* T_out, void* stream) {
  if (!X || !codes || !c2 || !c1 || !L1 || !L2 || !Y) return QL_ERR_NULL;
  const size_t need = qlora_linear_fwd_workspace(M, K, N, r);
  if (need == 0) return QL_ERR_SHAPE;
  if (need > QL_NOALLOC_SCRATCH_BYTES) return QL_ERR_WORKSPACE;
  for (const void* p : {(const void*)X, (const void*)codes, (const void*)c2, (const void*)c1, (const void*)L1,
                        (const void*)L2, (const void*)Y, (const void*)T_out})
    if ((reinterpret_cast<uintptr_t>(p) & 15u) != 0) return QL_ERR_ALIGN;
  void* ws = nullptr;
  const hipError_t e = scratch_ptr(&ws);
  if (e != hipSuccess) return ql_record_hip_error(e);
  return qlora_linear_fwd(X, M, K, N, codes, c2, c1, L1, L2, r, lora_scale, Y, T_out, ws, QL_NOALLOC_SCRATCH_BYTES,
                          stream);
}
