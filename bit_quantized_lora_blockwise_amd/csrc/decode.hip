// Decode-sized forward (M <= 16): Y = bf16(X W'^T + s T L2) as one pass over
// the packed 4-bit weight stream.  At these sizes the layer is bound by HBM
// traffic of the codes and scales, so the kernel is organised around a
// coalesced stream of 16-byte code loads; the dequantised bf16 weights live
// only in registers and feed a 16x16x32 bf16 MFMA against X.
// Layer formula: nlp-lineage milestone page on QLoRA, "The idea", notation
// paragraph.
#include "kernels.h"

namespace {

constexpr int kThreads = 256;
constexpr int kRows = 16;  // output columns (weight rows) per work group

__device__ __forceinline__ f32x4 mfma16(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// Work group: 16 weight rows x all of K.  Lane l of each wave handles weight row
// n0 + l % 16 and, per 128-wide step of K, the 32 columns 32 * (l / 16) .. +32;
// the four waves interleave the steps.  MFMA operands use the same permuted
// order of k for X and W', so the sum is unchanged.
__global__ __launch_bounds__(kThreads) void k_qgemv_fwd(const uint16_t* __restrict__ X, int64_t M, int64_t K,
                                                        int64_t N, const uint8_t* __restrict__ codes,
                                                        const uint8_t* __restrict__ c2,
                                                        const float* __restrict__ c1,
                                                        const uint16_t* __restrict__ T,
                                                        const uint16_t* __restrict__ L2, int r, float scale,
                                                        uint16_t* __restrict__ Y, Nf4Params p) {
  __shared__ __attribute__((aligned(16))) float qs[16];
  __shared__ f32x4 red[4][64];
  const int t = threadIdx.x;
  const int w = t >> 6, l = t & 63;
  const int g = l >> 4, col = l & 15;
  if (t < 16) qs[t] = p.q[t];
  __syncthreads();
  const int64_t n0 = (int64_t)blockIdx.x * kRows;
  const int64_t nrow = n0 + col;
  const int64_t kblocks = K / qk::kBlock;
  const bool row_ok = nrow < N;
  const bool m_ok = col < M;  // A operand row of this lane is X[col]
  f32x4 acc = {0, 0, 0, 0};
  for (int64_t kb = 128 * w; kb < K; kb += 512) {
    const int64_t k = kb + 32 * g;
    u32x4 cw = {0, 0, 0, 0};
    float s = 0.0f;
    const bool k_ok = k < K;
    if (row_ok && k_ok) {
      cw = *(const u32x4*)(codes + nrow * (K / 2) + k / 2);
      const int64_t b = nrow * kblocks + (k >> 6);
      s = qk::e4m3fn_to_f32(c2[b]) * c1[b >> 8];
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      u32x4 bw;
#pragma unroll
      for (int h = 0; h < 4; ++h) {
        const float lo = qs[(cw[j] >> (8 * h)) & 15] * s;
        const float hi = qs[(cw[j] >> (8 * h + 4)) & 15] * s;
        bw[h] = qk::pack_bf16x2(lo, hi);
      }
      u32x4 aw = {0, 0, 0, 0};
      if (m_ok && k_ok) aw = *(const u32x4*)(X + col * K + k + 8 * j);
      acc = mfma16(__builtin_bit_cast(bf16x8, aw), __builtin_bit_cast(bf16x8, bw), acc);
    }
  }
  red[w][l] = acc;
  __syncthreads();
  if (w == 0) {
    f32x4 sum = red[0][l];
#pragma unroll
    for (int ww = 1; ww < 4; ++ww) sum += red[ww][l];
    // lane l holds C[m = 4g + i][n = col]; add s * T[m] . L2[:, n]
    float lora[4] = {0, 0, 0, 0};
    if (row_ok) {
      for (int c = 0; c < r; ++c) {
        const float lv = qk::bf16_to_f32(L2[(int64_t)c * N + nrow]);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int m = 4 * g + i;
          if (m < M) lora[i] += qk::bf16_to_f32(T[(int64_t)m * r + c]) * lv;
        }
      }
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int m = 4 * g + i;
      if (m < M && row_ok) Y[(int64_t)m * N + nrow] = qk::f32_to_bf16(sum[i] + scale * lora[i]);
    }
  }
}

}  // namespace

hipError_t launch_qgemv_fwd(const uint16_t* X, int64_t M, int64_t K, int64_t N, const uint8_t* codes,
                            const uint8_t* c2, const float* c1, const uint16_t* T, const uint16_t* L2, int r,
                            float scale, uint16_t* Y, hipStream_t s) {
  dim3 grid((unsigned)((N + kRows - 1) / kRows));
  hipLaunchKernelGGL(k_qgemv_fwd, grid, dim3(kThreads), 0, s, X, M, K, N, codes, c2, c1, T, L2, r, scale, Y,
                     nf4_params());
  return hipGetLastError();
}
