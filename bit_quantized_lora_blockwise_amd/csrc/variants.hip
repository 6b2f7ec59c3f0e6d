// The 4-bit formats and second-level scale codes that the pages rank NF4
// against (nlp-lineage milestone page on QLoRA, "What it showed": NF4 with
// double quantization against a standard 4-bit float and 4-bit integers;
// inferensys glossary entry "QLoRA", NF4 against standard 4-bit integers).
//
// The same blockwise-absmax encoder and table dequantizer as NF4, with the
// 16-entry level table as a parameter:
//   4-bit float   E2M1 values / 6 (absmax maps to the largest, 6),
//   4-bit integer k / 7 for k = -7..7,
// each held ascending with code 15 repeating +1 (never produced), and three
// ways to code the block scales: the fp32 absmax itself, the E4M3FN codes over
// the full range (c1 = group max / 448), and mean-centred codes (the signed
// differences from the group mean, full range, s' = mu + dec(c2) c1).
#include "kernels.h"

namespace {

constexpr int kThreads = 256;

// One thread encodes 8 consecutive weights; 8 lanes share a block's absmax.
// n = fl32(w / a) (correctly rounded), code = #{k : n >= thr[k]}.
template <bool kBf16>
__global__ __launch_bounds__(kThreads) void k_q4_encode(const void* __restrict__ W, int64_t n_oct,
                                                        uint32_t* __restrict__ codes,
                                                        float* __restrict__ absmax, Nf4Params p) {
  const int64_t stride = (int64_t)gridDim.x * kThreads;
  for (int64_t o = (int64_t)blockIdx.x * kThreads + threadIdx.x; o < n_oct; o += stride) {
    float w[8];
    if (kBf16) {
      const u32x4 v = ((const u32x4*)W)[o];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        w[2 * j] = __uint_as_float(v[j] << 16);
        w[2 * j + 1] = __uint_as_float(v[j] & 0xFFFF0000u);
      }
    } else {
      const u32x4 v0 = ((const u32x4*)W)[2 * o], v1 = ((const u32x4*)W)[2 * o + 1];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        w[j] = __uint_as_float(v0[j]);
        w[4 + j] = __uint_as_float(v1[j]);
      }
    }
    uint32_t m = 0;
#pragma unroll
    for (int j = 0; j < 8; ++j) m = max(m, __float_as_uint(w[j]) & 0x7FFFFFFFu);
    m = qk::dpp_max8(m);
    const float a = __uint_as_float(m);
    uint32_t packed = 0;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const float n = (m == 0) ? 0.0f : w[j] / a;
      uint32_t c = 0;
#pragma unroll
      for (int k = 0; k < 15; ++k) c += (n >= p.thr[k]) ? 1u : 0u;
      packed |= c << (4 * j);
    }
    codes[o] = packed;
    if ((threadIdx.x & 7) == 0) absmax[o >> 3] = a;
  }
}

// One wavefront per group of 256 scales; lane l owns scales 4l..4l+3.
// kMean = false: c1 = fl32(max / 448), c2 = E4M3FN(fl32(a / c1)).
// kMean = true:  mu = fl32(tree sum / count) (pairs i, i + h for h = 128 .. 1 over
// the zero-padded group), d = fl32(a - mu), c1 = fl32(max |d| / 448),
// c2 = sign | E4M3FN(|fl32(d / c1)|).
template <bool kMean>
__global__ __launch_bounds__(kThreads) void k_double_quant_full(const float* __restrict__ absmax, int64_t nb,
                                                                uint8_t* __restrict__ c2, float* __restrict__ c1,
                                                                float* __restrict__ mu, int64_t ngroups) {
  const int lane = threadIdx.x & 63;
  const int64_t wstride = (int64_t)gridDim.x * (kThreads / 64);
  for (int64_t g = (int64_t)blockIdx.x * (kThreads / 64) + (threadIdx.x >> 6); g < ngroups; g += wstride) {
    const int64_t base = g * qk::kGroup + 4 * lane;
    float v[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) v[j] = (base + j < nb) ? absmax[base + j] : 0.0f;
    float m0 = 0.0f;
    if (kMean) {
      // element 4 l + j pairs with 4 l + j + h: lane l ^ (h / 4) for h >= 4, then within the lane
      float x[4] = {v[0], v[1], v[2], v[3]};
#pragma unroll
      for (int o = 32; o >= 1; o >>= 1)
#pragma unroll
        for (int j = 0; j < 4; ++j) x[j] = __fadd_rn(x[j], __shfl_xor(x[j], o, 64));
      x[0] = __fadd_rn(x[0], x[2]);
      x[1] = __fadd_rn(x[1], x[3]);
      const float total = __fadd_rn(x[0], x[1]);
      const int64_t rest = nb - g * qk::kGroup;
      const float count = (float)(rest < qk::kGroup ? rest : qk::kGroup);
      m0 = total / count;
#pragma unroll
      for (int j = 0; j < 4; ++j) v[j] = (base + j < nb) ? __fsub_rn(v[j], m0) : 0.0f;
    }
    uint32_t m = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) m = max(m, __float_as_uint(v[j]) & 0x7FFFFFFFu);
    m = qk::wave_max_u32(m);
    const float cs = __uint_as_float(m) / 448.0f;
    if (lane == 0) {
      c1[g] = cs;
      if (kMean) mu[g] = m0;
    }
    uint32_t packed = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float t = (cs == 0.0f) ? 0.0f : v[j] / cs;
      const uint32_t mag = qk::e4m3fn_encode(__builtin_fabsf(t));
      packed |= (mag | ((t < 0.0f && mag != 0) ? 0x80u : 0u)) << (8 * j);
    }
    if (base + 4 <= nb) {
      *(uint32_t*)(c2 + base) = packed;
    } else {
      for (int j = 0; j < 4; ++j)
        if (base + j < nb) c2[base + j] = (uint8_t)(packed >> (8 * j));
    }
  }
}

// W'[e] = bf16(fl32(q[code_e] * s_b)) with the block scale of the mode:
// 0: fl32(dec(c2) c1); 1: absmax; 2: fl32(mu + fl32(dec(c2) c1)).
template <int kMode>
__global__ __launch_bounds__(kThreads) void k_q4_dequant(const uint32_t* __restrict__ codes,
                                                         const float* __restrict__ absmax,
                                                         const uint8_t* __restrict__ c2,
                                                         const float* __restrict__ c1, const float* __restrict__ mu,
                                                         int64_t n_oct, u32x4* __restrict__ out, Nf4Params p) {
  __shared__ float q[16];
  if (threadIdx.x < 16) q[threadIdx.x] = p.q[threadIdx.x];
  __syncthreads();
  const int64_t stride = (int64_t)gridDim.x * kThreads;
  for (int64_t o = (int64_t)blockIdx.x * kThreads + threadIdx.x; o < n_oct; o += stride) {
    const int64_t b = o >> 3;
    float s;
    if (kMode == 1) {
      s = absmax[b];
    } else {
      s = __fmul_rn(qk::e4m3fn_to_f32(c2[b]), c1[b >> 8]);
      if (kMode == 2) s = __fadd_rn(mu[b >> 8], s);
    }
    const uint32_t cw = codes[o];
    u32x4 r;
#pragma unroll
    for (int j = 0; j < 4; ++j)
      r[j] = qk::pack_bf16x2(__fmul_rn(q[(cw >> (8 * j)) & 15], s), __fmul_rn(q[(cw >> (8 * j + 4)) & 15], s));
    out[o] = r;
  }
}

int grid_for(int64_t items, int per_block) {
  int64_t g = (items + per_block - 1) / per_block;
  if (g > 8192) g = 8192;
  if (g < 1) g = 1;
  return (int)g;
}

}  // namespace

hipError_t launch_q4_encode(const void* W, bool bf16, int64_t elems, const Nf4Params& p, uint8_t* codes,
                            float* absmax, hipStream_t s) {
  const int64_t n_oct = elems / 8;
  const int grid = grid_for(n_oct, kThreads);
  if (bf16)
    hipLaunchKernelGGL(k_q4_encode<true>, dim3(grid), dim3(kThreads), 0, s, W, n_oct, (uint32_t*)codes, absmax, p);
  else
    hipLaunchKernelGGL(k_q4_encode<false>, dim3(grid), dim3(kThreads), 0, s, W, n_oct, (uint32_t*)codes, absmax, p);
  return hipGetLastError();
}

hipError_t launch_double_quant_full(const float* absmax, int64_t n_blocks, bool mean, uint8_t* c2, float* c1,
                                    float* mu, hipStream_t s) {
  const int64_t ngroups = (n_blocks + qk::kGroup - 1) / qk::kGroup;
  const int grid = grid_for(ngroups, kThreads / 64);
  if (mean)
    hipLaunchKernelGGL(k_double_quant_full<true>, dim3(grid), dim3(kThreads), 0, s, absmax, n_blocks, c2, c1, mu,
                       ngroups);
  else
    hipLaunchKernelGGL(k_double_quant_full<false>, dim3(grid), dim3(kThreads), 0, s, absmax, n_blocks, c2, c1, mu,
                       ngroups);
  return hipGetLastError();
}

hipError_t launch_q4_dequant(const uint8_t* codes, int mode, const float* absmax, const uint8_t* c2,
                             const float* c1, const float* mu, int64_t elems, const Nf4Params& p, uint16_t* out,
                             hipStream_t s) {
  const int64_t n_oct = elems / 8;
  const int grid = grid_for(n_oct, kThreads);
  const uint32_t* cw = (const uint32_t*)codes;
  if (mode == 0)
    hipLaunchKernelGGL(k_q4_dequant<0>, dim3(grid), dim3(kThreads), 0, s, cw, absmax, c2, c1, mu, n_oct,
                       (u32x4*)out, p);
  else if (mode == 1)
    hipLaunchKernelGGL(k_q4_dequant<1>, dim3(grid), dim3(kThreads), 0, s, cw, absmax, c2, c1, mu, n_oct,
                       (u32x4*)out, p);
  else
    hipLaunchKernelGGL(k_q4_dequant<2>, dim3(grid), dim3(kThreads), 0, s, cw, absmax, c2, c1, mu, n_oct,
                       (u32x4*)out, p);
  return hipGetLastError();
}
