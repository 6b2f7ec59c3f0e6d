// Skinny products of the LoRA branch (rank r <= 64):
//   T = bf16(X L1)            (forward, and recomputation in the backward)
//   G = bf16(s dY L2^T)       (backward)
//   dL1 = fp32(X^T G)         (backward)
//   dL2 = fp32(s T^T dY)      (backward)
// Layer formula and gradient flow: nlp-lineage milestone page on QLoRA,
// section "The idea", notation paragraph (only L1 and L2 get gradients).
//
// All four are memory-bound passes over an [M, R] bf16 activation.  Each work
// group owns a 64-row tile of the long dimension and one slice of the
// reduction; slices write fp32 partials that a second kernel sums in a fixed
// order, so results are deterministic.
#include "kernels.h"

namespace {

constexpr int kThreads = 256;
constexpr int kTile = 64;
constexpr int kPitch = 72;  // 64 + 8 elements of padding per LDS row

// 8 consecutive bf16 of a row starting at column `col`, zero past `ncols`.
__device__ __forceinline__ u32x4 load_row8(const uint16_t* __restrict__ row, int64_t col, int64_t ncols) {
  const uint16_t* p = row + col;
  if (col + 8 <= ncols && ((uintptr_t)p & 15) == 0) return *(const u32x4*)p;
  u32x4 v = {0, 0, 0, 0};
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const uint32_t h = (col + j < ncols) ? p[j] : 0;
    v[j >> 1] |= h << (16 * (j & 1));
  }
  return v;
}

__device__ __forceinline__ void store8(LDS_AS uint16_t* dst, u32x4 v) { *(LDS_AS u32x4*)dst = v; }

// Stage a 64 x 64 tile of a row-major [rows, cols] matrix (rows from r0, cols
// from c0) into LDS [64][kPitch]; out-of-range entries are zero.
__device__ __forceinline__ void stage_tile(LDS_AS uint16_t* dst, const uint16_t* __restrict__ src, int64_t ld,
                                           int64_t rows, int64_t cols, int64_t r0, int64_t c0) {
  const int t = threadIdx.x;
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int row = (t >> 3) + 32 * i;
    const int cc = (t & 7) * 8;
    u32x4 v = {0, 0, 0, 0};
    if (r0 + row < rows) v = load_row8(src + (r0 + row) * ld, c0 + cc, cols);
    store8(dst + row * kPitch + cc, v);
  }
}

// C[M, r] partial over one reduction slice: A [M, R] row-major times B, where
// B(k, c) = Bm[k * r + c] (kBkr, L1 [R, r]) or Bm[c * R + k] (!kBkr, L2 [r, R]).
template <bool kBkr>
__global__ __launch_bounds__(kThreads) void k_lora_skinny(const uint16_t* __restrict__ A, int64_t M, int64_t R,
                                                          const uint16_t* __restrict__ Bm, int r, int64_t chunk,
                                                          float* __restrict__ part) {
  __shared__ __attribute__((aligned(16))) uint16_t As[kTile * kPitch];
  __shared__ __attribute__((aligned(16))) uint16_t Bs[kTile * kPitch];
  const int w = threadIdx.x >> 6;
  const int wm = w & 1, wc = w >> 1;
  const int64_t m0 = (int64_t)blockIdx.x * kTile;
  const int split = blockIdx.y;
  const int64_t k_beg = split * chunk;
  const int64_t k_end = min(R, k_beg + chunk);
  f32x16 acc = {};
  for (int64_t k0 = k_beg; k0 < k_end; k0 += kTile) {
    stage_tile((LDS_AS uint16_t*)As, A, R, M, k_end, m0, k0);
    if (kBkr) {
      // Bs[k][c] = L1[k0 + k][c]
      stage_tile((LDS_AS uint16_t*)Bs, Bm, r, k_end, r, k0, 0);
    } else {
      // Bs[c][k] = L2[c][k0 + k]
      stage_tile((LDS_AS uint16_t*)Bs, Bm, R, r, k_end, 0, k0);
    }
    __syncthreads();
    if (wc * 32 < r) {
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        bf16x8 a = qk::frag_rowmajor((const LDS_AS uint16_t*)As, kPitch, 32 * wm, 16 * s);
        bf16x8 b = kBkr ? qk::frag_kmajor((const LDS_AS uint16_t*)Bs, kPitch, 16 * s, 32 * wc)
                        : qk::frag_rowmajor((const LDS_AS uint16_t*)Bs, kPitch, 32 * wc, 16 * s);
        acc = qk::mfma32(a, b, acc);
      }
    }
    __syncthreads();
  }
  if (wc * 32 < r) {
    const int c = 32 * wc + qk::acc_col();
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const int64_t m = m0 + 32 * wm + qk::acc_row(j);
      if (m < M && c < r) part[((int64_t)split * M + m) * r + c] = acc[j];
    }
  }
}

__global__ __launch_bounds__(kThreads) void k_skinny_reduce(const float* __restrict__ part, int splits, int64_t n,
                                                            float scale, uint16_t* __restrict__ out) {
  const int64_t stride = (int64_t)gridDim.x * kThreads;
  for (int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x; i < n; i += stride) {
    float s = 0.0f;
    for (int k = 0; k < splits; ++k) s += part[k * n + i];
    out[i] = qk::f32_to_bf16(scale * s);
  }
}

// C[p, c] partial over one slice of m: sum_m A[m][p] * B[m][c], A [M, P], B [M, r].
__global__ __launch_bounds__(kThreads) void k_lora_tn(const uint16_t* __restrict__ A, const uint16_t* __restrict__ B,
                                                      int64_t M, int64_t P, int r, int64_t chunk,
                                                      float* __restrict__ part) {
  __shared__ __attribute__((aligned(16))) uint16_t As[kTile * kPitch];
  __shared__ __attribute__((aligned(16))) uint16_t Bs[kTile * kPitch];
  const int w = threadIdx.x >> 6;
  const int wp = w & 1, wc = w >> 1;
  const int64_t p0 = (int64_t)blockIdx.x * kTile;
  const int split = blockIdx.y;
  const int64_t m_beg = split * chunk;
  const int64_t m_end = min(M, m_beg + chunk);
  f32x16 acc = {};
  for (int64_t mm = m_beg; mm < m_end; mm += kTile) {
    stage_tile((LDS_AS uint16_t*)As, A, P, m_end, P, mm, p0);   // As[m][p]
    stage_tile((LDS_AS uint16_t*)Bs, B, r, m_end, r, mm, 0);    // Bs[m][c]
    __syncthreads();
    if (wc * 32 < r) {
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        bf16x8 a = qk::frag_kmajor((const LDS_AS uint16_t*)As, kPitch, 16 * s, 32 * wp);
        bf16x8 b = qk::frag_kmajor((const LDS_AS uint16_t*)Bs, kPitch, 16 * s, 32 * wc);
        acc = qk::mfma32(a, b, acc);
      }
    }
    __syncthreads();
  }
  if (wc * 32 < r) {
    const int c = 32 * wc + qk::acc_col();
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const int64_t p = p0 + 32 * wp + qk::acc_row(j);
      if (p < P && c < r) part[((int64_t)split * P + p) * r + c] = acc[j];
    }
  }
}

__global__ __launch_bounds__(kThreads) void k_tn_reduce(const float* __restrict__ part, int splits, int64_t P, int r,
                                                        float scale, bool transpose_out, float* __restrict__ out) {
  const int64_t n = P * r;
  const int64_t stride = (int64_t)gridDim.x * kThreads;
  for (int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x; i < n; i += stride) {
    float s = 0.0f;
    for (int k = 0; k < splits; ++k) s += part[k * n + i];
    s *= scale;
    if (transpose_out) {
      const int64_t p = i / r, c = i - p * r;
      out[c * P + p] = s;
    } else {
      out[i] = s;
    }
  }
}

int grid_for(int64_t items) {
  int64_t g = (items + kThreads - 1) / kThreads;
  return (int)(g < 1 ? 1 : (g > 4096 ? 4096 : g));
}

}  // namespace

SplitPlan plan_rowsplit(int64_t tiles, int64_t R) {
  const int64_t want = (1024 + tiles - 1) / tiles;
  const int64_t max_splits = (R + 255) / 256;
  int64_t splits = want < 1 ? 1 : want;
  if (splits > max_splits) splits = max_splits;
  if (splits < 1) splits = 1;
  int64_t chunk = (R + splits - 1) / splits;
  chunk = (chunk + kTile - 1) / kTile * kTile;
  splits = (R + chunk - 1) / chunk;
  return SplitPlan{(int)splits, chunk};
}

size_t lora_skinny_ws(int64_t M, int64_t R, int r) {
  const SplitPlan sp = plan_rowsplit((M + kTile - 1) / kTile, R);
  return (size_t)sp.splits * M * r * sizeof(float);
}

hipError_t launch_lora_skinny(const uint16_t* A, int64_t M, int64_t R, const uint16_t* B, bool b_is_kr, int r,
                              float scale, uint16_t* out, float* ws, hipStream_t s) {
  const int64_t tiles = (M + kTile - 1) / kTile;
  const SplitPlan sp = plan_rowsplit(tiles, R);
  dim3 grid((unsigned)tiles, (unsigned)sp.splits);
  if (b_is_kr)
    hipLaunchKernelGGL(k_lora_skinny<true>, grid, dim3(kThreads), 0, s, A, M, R, B, r, sp.chunk, ws);
  else
    hipLaunchKernelGGL(k_lora_skinny<false>, grid, dim3(kThreads), 0, s, A, M, R, B, r, sp.chunk, ws);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(k_skinny_reduce, dim3(grid_for(M * r)), dim3(kThreads), 0, s, ws, sp.splits, M * (int64_t)r,
                     scale, out);
  return hipGetLastError();
}

size_t lora_tn_ws(int64_t M, int64_t P, int r) {
  const SplitPlan sp = plan_rowsplit((P + kTile - 1) / kTile, M);
  return (size_t)sp.splits * P * r * sizeof(float);
}

hipError_t launch_lora_tn(const uint16_t* A, const uint16_t* B, int64_t M, int64_t P, int r, float scale,
                          bool transpose_out, float* out, float* ws, hipStream_t s) {
  const int64_t tiles = (P + kTile - 1) / kTile;
  const SplitPlan sp = plan_rowsplit(tiles, M);
  dim3 grid((unsigned)tiles, (unsigned)sp.splits);
  hipLaunchKernelGGL(k_lora_tn, grid, dim3(kThreads), 0, s, A, B, M, P, r, sp.chunk, ws);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(k_tn_reduce, dim3(grid_for(P * r)), dim3(kThreads), 0, s, ws, sp.splits, P, r, scale,
                     transpose_out, out);
  return hipGetLastError();
}
