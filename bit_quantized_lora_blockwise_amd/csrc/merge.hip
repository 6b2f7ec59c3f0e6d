// Adapter merge for export: W_m = bf16(W' + s (L1 L2)^T), W' the exact bf16
// dequantised base (the weight every layer entry point multiplies with).  The
// pages' practical notes on merging (examadda page, "Practical Notes") say
// the base is dequantised first and the low-rank product added in high
// precision; the single rounding to bf16 happens at the end.
//
// One pass over HBM: a work group owns a 64 (n) x 64 (k) tile of W_m -- one
// NF4 block per row -- reads its codes and scales once and writes the bf16
// tile once (0.5 + 2 bytes per weight).  The rank-r product is one MFMA
// 32 x 32 sub-tile per wave out of LDS (rank zero-padded to a multiple of
// 16); it is parked in LDS as fp32 so that every thread then finishes 8
// consecutive weights of a row with one 16-byte store.  The small tile keeps
// LDS at 18 KB per work group, so that 8 of them share a compute unit.
#include "kernels.h"

namespace {

constexpr int kThreads = 256;
constexpr int kTn = 64;          // rows of W (output features) per tile
constexpr int kTk = 64;          // columns of W (input features) per tile
constexpr int kPitch = 72;       // bf16 per LDS row of the adapter tiles (64 + 8)
constexpr int kPP = kTk + 8;     // fp32 per LDS row of the low-rank tile
constexpr int kOcts = kTk / 8;   // octets (8 weights) per tile row
constexpr int kOct = kTn * kOcts / kThreads;  // octets per thread in the epilogue
constexpr int kRowStep = kThreads / kOcts;    // rows between a thread's octets

struct Smem {
  float q[16];
  union {
    struct {
      uint16_t a[64 * kPitch];   // L2 tile, [c][n]
      uint16_t b[kTk * kPitch];  // L1 tile, [k][c]
    } ab;
    float p[kTn * kPP];          // (L1 L2)^T tile, [n][k]
  } u;
};

// 8 consecutive bf16 of row `row` (ld elements per row) from column `col`;
// zero past `ncols`.  `vec`: ld, col and the base are 16-byte aligned.
__device__ __forceinline__ u32x4 load8(const uint16_t* __restrict__ base, int64_t ld, int64_t row, int64_t col,
                                       int64_t ncols, bool vec) {
  const uint16_t* p = base + row * ld + col;
  if (vec && col + 8 <= ncols) return *(const u32x4*)p;
  u32x4 v = {0, 0, 0, 0};
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const uint32_t h = (col + j < ncols) ? p[j] : 0;
    v[j >> 1] |= h << (16 * (j & 1));
  }
  return v;
}

__global__ __launch_bounds__(kThreads) void k_merge(const uint32_t* __restrict__ codes,
                                                    const uint8_t* __restrict__ c2, const float* __restrict__ c1,
                                                    const uint16_t* __restrict__ L1,
                                                    const uint16_t* __restrict__ L2, int64_t N, int64_t K, int r,
                                                    float scale, uint16_t* __restrict__ W, Nf4Params prm,
                                                    int l2vec, int l1vec, int64_t ktiles) {
  __shared__ __attribute__((aligned(16))) Smem sm;
  const int t = threadIdx.x;
  const int w = t >> 6;
  // Work groups go round-robin to the 8 XCDs; renumber them so that each XCD
  // takes a contiguous run of tiles, k fastest: the tiles that share a
  // 128-byte line of codes then meet in one L2.
  const int64_t T = gridDim.x, L = blockIdx.x;
  const int64_t per = T / 8, rem = T % 8, xcd = L % 8, slot = L / 8;
  const int64_t tile = (xcd < rem ? xcd * (per + 1) : rem * (per + 1) + (xcd - rem) * per) + slot;
  const int64_t k0 = (tile % ktiles) * kTk;
  const int64_t n0 = (tile / ktiles) * kTn;
  const int64_t kb = K / qk::kBlock;  // blocks per row

  // Epilogue work of this thread: octet column oc of rows t / kOcts + kRowStep i.
  // Codes and scales are requested first so that their latency overlaps the
  // low-rank product.
  const int oc = t % kOcts;
  const int64_t kk = k0 + oc * 8;
  uint32_t cw[kOct];
  float sc[kOct];
#pragma unroll
  for (int i = 0; i < kOct; ++i) {
    const int64_t n = n0 + t / kOcts + kRowStep * i;
    cw[i] = 0;
    sc[i] = 0.f;
    if (n < N && kk < K) {
      cw[i] = codes[(n * K + kk) >> 3];
      const int64_t b = n * kb + (kk >> 6);
      sc[i] = qk::e4m3fn_to_f32(c2[b]) * c1[b >> 8];
    }
  }

  if (t < 16) sm.q[t] = prm.q[t];
  // Adapter tiles, zero outside [0, r) x [0, N) and [0, r) x [0, K).
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int c = (t >> 3) + 32 * i, col = (t & 7) * 8;
    const u32x4 v = (c < r) ? load8(L2 + n0, N, c, col, N - n0, l2vec) : u32x4{0, 0, 0, 0};
    *(LDS_AS u32x4*)((LDS_AS uint16_t*)sm.u.ab.a + c * kPitch + col) = v;
  }
#pragma unroll
  for (int i = 0; i < kTk / 32; ++i) {
    const int kr = (t >> 3) + 32 * i, col = (t & 7) * 8;
    const u32x4 v = (k0 + kr < K) ? load8(L1 + k0 * r, r, kr, col, r, l1vec) : u32x4{0, 0, 0, 0};
    *(LDS_AS u32x4*)((LDS_AS uint16_t*)sm.u.ab.b + kr * kPitch + col) = v;
  }
  __syncthreads();

  // Waves: kWk along k, 4 / kWk along n; wave w owns kM x kC sub-tiles of 32 x 32.
  constexpr int kWk = kTk / 32 < 4 ? kTk / 32 : 4, kWn = 4 / kWk;
  constexpr int kWc = kTk / kWk, kC = kWc / 32, kWr = kTn / kWn, kM = kWr / 32;
  const int wk = w % kWk, wn = w / kWk;
  f32x16 acc[kM][kC] = {};
  const int steps = (r + 15) >> 4;
  for (int s = 0; s < steps; ++s) {
    bf16x8 a[kM], b[kC];
#pragma unroll
    for (int m = 0; m < kM; ++m)
      a[m] = qk::frag_kmajor((const LDS_AS uint16_t*)sm.u.ab.a, kPitch, 16 * s, kWr * wn + 32 * m);
#pragma unroll
    for (int c = 0; c < kC; ++c)
      b[c] = qk::frag_rowmajor((const LDS_AS uint16_t*)sm.u.ab.b, kPitch, kWc * wk + 32 * c, 16 * s);
#pragma unroll
    for (int m = 0; m < kM; ++m)
#pragma unroll
      for (int c = 0; c < kC; ++c) acc[m][c] = qk::mfma32(a[m], b[c], acc[m][c]);
  }
  __syncthreads();  // the product tile reuses the adapter tiles' LDS
#pragma unroll
  for (int m = 0; m < kM; ++m)
#pragma unroll
    for (int c = 0; c < kC; ++c)
#pragma unroll
      for (int j = 0; j < 16; ++j)
        ((LDS_AS float*)sm.u.p)[(kWr * wn + 32 * m + qk::acc_row(j)) * kPP + kWc * wk + 32 * c + qk::acc_col()] =
            acc[m][c][j];
  __syncthreads();

#pragma unroll
  for (int i = 0; i < kOct; ++i) {
    const int nl = t / kOcts + kRowStep * i;
    const int64_t n = n0 + nl;
    if (n >= N || kk >= K) continue;
    const LDS_AS float* pr = (const LDS_AS float*)sm.u.p + nl * kPP + oc * 8;
    const f32x4 p0 = *(const LDS_AS f32x4*)pr, p1 = *(const LDS_AS f32x4*)(pr + 4);
    const float lo[8] = {p0[0], p0[1], p0[2], p0[3], p1[0], p1[1], p1[2], p1[3]};
    u32x4 o;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      // W' element (bf16, as the dequantiser writes it), then one rounding of W' + s P.
      const float w0 = (float)(__bf16)(sm.q[(cw[i] >> (8 * j)) & 15] * sc[i]);
      const float w1 = (float)(__bf16)(sm.q[(cw[i] >> (8 * j + 4)) & 15] * sc[i]);
      o[j] = qk::pack_bf16x2(w0 + scale * lo[2 * j], w1 + scale * lo[2 * j + 1]);
    }
    *(u32x4*)(W + n * K + kk) = o;
  }
}

}  // namespace

hipError_t launch_merge(const uint8_t* codes, const uint8_t* c2, const float* c1, int64_t N, int64_t K,
                        const uint16_t* L1, const uint16_t* L2, int r, float scale, uint16_t* W, hipStream_t s) {
  const int64_t ktiles = (K + kTk - 1) / kTk;
  const dim3 grid((unsigned)(ktiles * ((N + kTn - 1) / kTn)));
  const int l2vec = (N % 8) == 0 && (((uintptr_t)L2) & 15) == 0;
  const int l1vec = (r % 8) == 0 && (((uintptr_t)L1) & 15) == 0;
  hipLaunchKernelGGL(k_merge, grid, dim3(kThreads), 0, s, (const uint32_t*)codes, c2, c1, L1, L2, N, K, r, scale,
                     W, nf4_params(), l2vec, l1vec, ktiles);
  return hipGetLastError();
}
