// Backward GEMM of the layer for the shapes the large-tile kernel does not
// take (N % 8 != 0, whose dY rows are not 16-byte aligned, and M <= 16):
//   dX = bf16(dY W' + G L1^T)       (transposed-weight path)
// W' = doubleDequant(c1, c2, W_NF4) is rebuilt tile by tile from the packed
// 4-bit stream into bf16 in LDS and fed to bf16 MFMA; it never reaches HBM.
// Layer formula: nlp-lineage milestone page on QLoRA, "The idea", notation
// paragraph; dequantisation on the fly: examadda page "The Core Idea";
// inferensys glossary, paragraph on the dequantising kernel.
#include "kernels.h"

namespace {

constexpr int kThreads = 256;
constexpr int kBM = 128;         // rows of X / dY per tile
constexpr int kBN = 128;         // output columns per tile
constexpr int kBK = 64;          // reduction step (one quant block along K in the forward)
constexpr int kPA = kBK + 8;     // LDS pitch of [row][k] tiles
constexpr int kPB = kBN + 8;     // LDS pitch of [k][col] tiles

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

// Dequantise 32 consecutive weights of one row (one 16-byte slice of codes, all
// in one block with scale s) into LDS as bf16: W' = bf16(fl32(q[code] * s)).
__device__ __forceinline__ void dequant32_to_lds(LDS_AS uint16_t* dst, u32x4 cw, float s,
                                                 const LDS_AS float* q) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    u32x4 o;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float lo = q[(cw[i] >> (8 * j)) & 15] * s;
      const float hi = q[(cw[i] >> (8 * j + 4)) & 15] * s;
      o[j] = qk::pack_bf16x2(lo, hi);
    }
    *(LDS_AS u32x4*)(dst + 8 * i) = o;
  }
}

__device__ __forceinline__ float block_scale(const uint8_t* __restrict__ c2, const float* __restrict__ c1,
                                             int64_t b) {
  return qk::e4m3fn_to_f32(c2[b]) * c1[b >> 8];
}

// Stage rows [r0, r0 + 128) x cols [c0, c0 + 64) of a row-major bf16 matrix into
// LDS [128][kPA]; out-of-range entries are zero.
__device__ __forceinline__ void stage_rows128(LDS_AS uint16_t* dst, const uint16_t* __restrict__ src, int64_t ld,
                                              int64_t rows, int64_t cols, int64_t r0, int64_t c0) {
  const int t = threadIdx.x;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int row = (t >> 3) + 32 * i;
    const int cc = (t & 7) * 8;
    u32x4 v = {0, 0, 0, 0};
    if (r0 + row < rows) v = load_row8(src + (r0 + row) * ld, c0 + cc, cols);
    *(LDS_AS u32x4*)(dst + row * kPA + cc) = v;
  }
}

// ---------------------------------------------------------------------------
// Backward dX: tile of 128 rows (m) x 128 columns (k); the reduction runs over
// the N stored rows of W in steps of 64.  The W' tile is dequantised in its
// stored [n][k] orientation and read transposed (ds_read_b64_tr_b16) as the
// MFMA B operand.
__global__ __launch_bounds__(kThreads) void k_qgemm_dx(const uint16_t* __restrict__ dY, int64_t M, int64_t K,
                                                       int64_t N, const uint8_t* __restrict__ codes,
                                                       const uint8_t* __restrict__ c2,
                                                       const float* __restrict__ c1,
                                                       const uint16_t* __restrict__ G,
                                                       const uint16_t* __restrict__ L1, int r,
                                                       uint16_t* __restrict__ dX, Nf4Params p) {
  constexpr int kBsElems = (kBN * kPA > kBK * kPB) ? kBN * kPA : kBK * kPB;
  __shared__ __attribute__((aligned(16))) uint16_t As[kBM * kPA];
  __shared__ __attribute__((aligned(16))) uint16_t Bs[kBsElems];
  __shared__ __attribute__((aligned(16))) float qs[16];
  const int t = threadIdx.x;
  const int w = t >> 6;
  const int wm = w & 1, wk = w >> 1;
  const int64_t m0 = (int64_t)blockIdx.y * kBM;
  const int64_t k0 = (int64_t)blockIdx.x * kBN;
  if (t < 16) qs[t] = p.q[t];

  f32x16 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[i][j] = f32x16{};

  // LoRA term: acc = G L1^T; A = G [m][c], B(c, k) = L1[k][c] staged as Bs[k][c].
  {
    stage_rows128((LDS_AS uint16_t*)As, G, r, M, r, m0, 0);
    stage_rows128((LDS_AS uint16_t*)Bs, L1, r, K, r, k0, 0);
    __syncthreads();
    const int ksteps = (r + 15) / 16;
    for (int s = 0; s < ksteps; ++s) {
      bf16x8 a0 = qk::frag_rowmajor((const LDS_AS uint16_t*)As, kPA, 64 * wm, 16 * s);
      bf16x8 a1 = qk::frag_rowmajor((const LDS_AS uint16_t*)As, kPA, 64 * wm + 32, 16 * s);
      bf16x8 b0 = qk::frag_rowmajor((const LDS_AS uint16_t*)Bs, kPA, 64 * wk, 16 * s);
      bf16x8 b1 = qk::frag_rowmajor((const LDS_AS uint16_t*)Bs, kPA, 64 * wk + 32, 16 * s);
      acc[0][0] = qk::mfma32(a0, b0, acc[0][0]);
      acc[0][1] = qk::mfma32(a0, b1, acc[0][1]);
      acc[1][0] = qk::mfma32(a1, b0, acc[1][0]);
      acc[1][1] = qk::mfma32(a1, b1, acc[1][1]);
    }
    __syncthreads();
  }

  const int64_t kblocks = K / qk::kBlock;
  const int drow = t >> 2, dq = t & 3;   // dequant: row drow of the 64-row step, 32 columns dq*32
  const int64_t kcol = k0 + 32 * dq;
  const int64_t nsteps = (N + kBK - 1) / kBK;
  for (int64_t nt = 0; nt < nsteps; ++nt) {
    const int64_t nbase = nt * kBK;
    stage_rows128((LDS_AS uint16_t*)As, dY, N, M, N, m0, nbase);
    LDS_AS uint16_t* bdst = (LDS_AS uint16_t*)Bs + drow * kPB + 32 * dq;
    const int64_t n = nbase + drow;
    if (n < N && kcol < K) {
      const int64_t b = n * kblocks + (kcol >> 6);
      const u32x4 cw = *(const u32x4*)(codes + n * (K / 2) + kcol / 2);
      dequant32_to_lds(bdst, cw, block_scale(c2, c1, b), (const LDS_AS float*)qs);
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i) *(LDS_AS u32x4*)(bdst + 8 * i) = u32x4{0, 0, 0, 0};
    }
    __syncthreads();
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      bf16x8 a0 = qk::frag_rowmajor((const LDS_AS uint16_t*)As, kPA, 64 * wm, 16 * s);
      bf16x8 a1 = qk::frag_rowmajor((const LDS_AS uint16_t*)As, kPA, 64 * wm + 32, 16 * s);
      bf16x8 b0 = qk::frag_kmajor((const LDS_AS uint16_t*)Bs, kPB, 16 * s, 64 * wk);
      bf16x8 b1 = qk::frag_kmajor((const LDS_AS uint16_t*)Bs, kPB, 16 * s, 64 * wk + 32);
      acc[0][0] = qk::mfma32(a0, b0, acc[0][0]);
      acc[0][1] = qk::mfma32(a0, b1, acc[0][1]);
      acc[1][0] = qk::mfma32(a1, b0, acc[1][0]);
      acc[1][1] = qk::mfma32(a1, b1, acc[1][1]);
    }
    __syncthreads();
  }

#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int64_t k = k0 + 64 * wk + 32 * j + qk::acc_col();
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int64_t m = m0 + 64 * wm + 32 * i + qk::acc_row(e);
        if (m < M && k < K) dX[m * K + k] = qk::f32_to_bf16(acc[i][j][e]);
      }
    }
}

}  // namespace

hipError_t launch_qgemm_dx(const uint16_t* dY, int64_t M, int64_t K, int64_t N, const uint8_t* codes,
                           const uint8_t* c2, const float* c1, const uint16_t* G, const uint16_t* L1, int r,
                           uint16_t* dX, hipStream_t s) {
  dim3 grid((unsigned)((K + kBN - 1) / kBN), (unsigned)((M + kBM - 1) / kBM));
  hipLaunchKernelGGL(k_qgemm_dx, grid, dim3(kThreads), 0, s, dY, M, K, N, codes, c2, c1, G, L1, r, dX,
                     nf4_params());
  return hipGetLastError();
}
