// Adapter-only optimizer step.  The 4-bit base is frozen, so the optimizer
// keeps momentum and variance for the adapters alone (inferensys glossary
// entry "QLoRA", frozen-base paragraph; nlp-lineage milestone page, "The
// idea": only L1 and L2 get weight gradients).  AdamW with decoupled weight
// decay over one flat array holding every adapter of a block (or a model), fp32
// master weights and moments, and the bf16 copy the layer multiplies with.
//
// Per element: theta = theta * decay; m = b1 m + (1 - b1) g; v = b2 v + (1 - b2) g^2;
// theta -= step_size * m / (sqrt(v) / bc2_sqrt + eps), with decay = 1 - lr wd,
// step_size = lr / (1 - b1^t) and bc2_sqrt = sqrt(1 - b2^t) from the host.
// Purely streaming: 16 bytes read and 12 (+2 for the bf16 copy) written per weight.
#include <cmath>

#include "kernels.h"

namespace {

constexpr int kThreads = 256;

struct AdamCoef {
  float b1, b2, eps, decay, step_size, bc2_sqrt;
};

__device__ __forceinline__ void adam1(float& th, float& m, float& v, float g, const AdamCoef& c) {
  th = th * c.decay;
  m = c.b1 * m + (1.0f - c.b1) * g;
  v = c.b2 * v + (1.0f - c.b2) * (g * g);
  const float denom = __builtin_sqrtf(v) / c.bc2_sqrt + c.eps;
  th = th - c.step_size * (m / denom);
}

__global__ __launch_bounds__(kThreads) void k_adamw(float* __restrict__ p, float* __restrict__ m,
                                                    float* __restrict__ v, const float* __restrict__ g,
                                                    uint16_t* __restrict__ pb, int64_t n, AdamCoef c) {
  const int64_t n4 = n / 4;
  const int64_t stride = (int64_t)gridDim.x * kThreads;
  for (int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x; i < n4; i += stride) {
    f32x4 th = ((const f32x4*)p)[i], mm = ((const f32x4*)m)[i], vv = ((const f32x4*)v)[i];
    const f32x4 gg = ((const f32x4*)g)[i];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      float a = th[j], b = mm[j], d = vv[j];
      adam1(a, b, d, gg[j], c);
      th[j] = a;
      mm[j] = b;
      vv[j] = d;
    }
    ((f32x4*)p)[i] = th;
    ((f32x4*)m)[i] = mm;
    ((f32x4*)v)[i] = vv;
    if (pb) ((u32x2*)pb)[i] = u32x2{qk::pack_bf16x2(th[0], th[1]), qk::pack_bf16x2(th[2], th[3])};
  }
  // tail (n % 4 elements)
  for (int64_t i = 4 * n4 + (int64_t)blockIdx.x * kThreads + threadIdx.x; i < n; i += stride) {
    float a = p[i], b = m[i], d = v[i];
    adam1(a, b, d, g[i], c);
    p[i] = a;
    m[i] = b;
    v[i] = d;
    if (pb) pb[i] = qk::f32_to_bf16(a);
  }
}

}  // namespace

hipError_t launch_adamw(float* param, float* exp_avg, float* exp_avg_sq, const float* grad, uint16_t* param_bf16,
                        int64_t n, float lr, float beta1, float beta2, float eps, float weight_decay, int64_t step,
                        hipStream_t s) {
  AdamCoef c;
  c.b1 = beta1;
  c.b2 = beta2;
  c.eps = eps;
  c.decay = (float)(1.0 - (double)lr * (double)weight_decay);
  c.step_size = (float)((double)lr / (1.0 - std::pow((double)beta1, (double)step)));
  c.bc2_sqrt = (float)std::sqrt(1.0 - std::pow((double)beta2, (double)step));
  int64_t blocks = (n / 4 + kThreads - 1) / kThreads;
  if (blocks > 4096) blocks = 4096;
  if (blocks < 1) blocks = 1;
  hipLaunchKernelGGL(k_adamw, dim3((unsigned)blocks), dim3(kThreads), 0, s, param, exp_avg, exp_avg_sq, grad,
                     param_bf16, n, c);
  return hipGetLastError();
}
