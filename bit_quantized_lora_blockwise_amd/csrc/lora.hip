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
// order, so results are deterministic.  Within a slice the 64-wide steps are
// pipelined: the tiles of step st + 2 are loaded into registers while step st
// multiplies out of one LDS buffer and step st + 1's tiles go into the other.
#include <algorithm>

#include "kernels.h"

namespace {

constexpr int kThreads = 256;
constexpr int kTile = 64;
constexpr int kPitch = 72;  // 64 + 8 elements of padding per LDS row
constexpr uint32_t kOOB = 0x80000000u;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void* p, uint64_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc((void*)p, (short)0, (int)(bytes < 0x7FFFFFFFull ? bytes : 0x7FFFFFFFull),
                                           0x00020000);
}

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

// A 64 x 64 bf16 tile of a row-major matrix held in registers: thread t holds
// rows (t / 8) + 32 i, columns 8 (t % 8) .. +8.
struct Tile {
  u32x4 v[2];
};

// Tile at `base` (its element (0, 0)) of a matrix with `ld` elements per row;
// rows at or past `rows` and columns at or past `cols` read as zero.  With
// kVec (ld and cols multiples of 8, base 16-byte aligned) each thread issues
// two 16-byte buffer loads with no branch, so that the loads of later steps
// stay in flight; otherwise it reads element by element.  `bytes`: extent of
// the matrix from `base`.
template <bool kVec>
__device__ __forceinline__ Tile load_tile(const uint16_t* base, int64_t ld, int64_t rows, int64_t cols,
                                          uint64_t bytes) {
  constexpr bool vec = kVec;
  const int t = threadIdx.x;
  const int cc = (t & 7) * 8;
  Tile tl;
  if (vec) {
    const __amdgpu_buffer_rsrc_t rs = rsrc(base, bytes);
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int row = (t >> 3) + 32 * i;
      const bool ok = row < rows && cc < cols;
      tl.v[i] = __builtin_amdgcn_raw_buffer_load_b128(rs, ok ? (uint32_t)((row * ld + cc) * 2) : kOOB, 0, 0);
    }
  } else {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int row = (t >> 3) + 32 * i;
      tl.v[i] = (row < rows) ? load_row8(base + row * ld, cc, cols) : u32x4{0, 0, 0, 0};
    }
  }
  return tl;
}

__device__ __forceinline__ void store_tile(const Tile& tl, LDS_AS uint16_t* dst) {
  const int t = threadIdx.x;
#pragma unroll
  for (int i = 0; i < 2; ++i) *(LDS_AS u32x4*)(dst + ((t >> 3) + 32 * i) * kPitch + (t & 7) * 8) = tl.v[i];
}

// C[M, r] partial over one reduction slice: A [M, R] (row stride lda) times B, where
// B(k, c) = Bm[k * r + c] (kBkr, L1 [R, r]) or Bm[c * R + k] (!kBkr, L2 [r, R]).
template <bool kBkr, bool kVecA, bool kVecB>
__global__ __launch_bounds__(kThreads) void k_lora_skinny(const uint16_t* __restrict__ A, int64_t M, int64_t R,
                                                          int64_t lda, const uint16_t* __restrict__ Bm, int r,
                                                          int64_t chunk, float* __restrict__ part) {
  __shared__ __attribute__((aligned(16))) uint16_t As[2][kTile * kPitch];
  __shared__ __attribute__((aligned(16))) uint16_t Bs[2][kTile * kPitch];
  const int w = threadIdx.x >> 6;
  const int wm = w & 1, wc = w >> 1;
  const int64_t m0 = (int64_t)blockIdx.x * kTile;
  const int split = blockIdx.y;
  const int64_t k_beg = split * chunk;
  const int64_t k_end = min(R, k_beg + chunk);
  const int64_t nsteps = (k_end - k_beg + kTile - 1) / kTile;
  auto tiles = [&](int64_t st, Tile& ta, Tile& tb) {
    const int64_t k0 = k_beg + st * kTile;
    const int64_t kl = k_end - k0;                     // columns of the slice left (<= 0: zeros)
    const int64_t k0c = kl > 0 ? k0 : 0;
    ta = load_tile<kVecA>(A + m0 * lda + k0c, lda, M - m0, kl, (uint64_t)((M - m0) * lda - k0c) * 2);
    if (kBkr) tb = load_tile<kVecB>(Bm + k0c * r, r, kl, r, (uint64_t)((R - k0c) * r) * 2);
    else tb = load_tile<kVecB>(Bm + k0c, R, r, kl, (uint64_t)(r * R - k0c) * 2);
  };
  f32x16 acc = {};
  auto step = [&](int64_t st, const Tile& na, const Tile& nb, Tile& la, Tile& lb) {
    tiles(st + 2, la, lb);
    const LDS_AS uint16_t* as = (const LDS_AS uint16_t*)As[st & 1];
    const LDS_AS uint16_t* bs = (const LDS_AS uint16_t*)Bs[st & 1];
    if (wc * 32 < r) {
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        bf16x8 a = qk::frag_rowmajor(as, kPitch, 32 * wm, 16 * s);
        bf16x8 b = kBkr ? qk::frag_kmajor(bs, kPitch, 16 * s, 32 * wc) : qk::frag_rowmajor(bs, kPitch, 32 * wc, 16 * s);
        acc = qk::mfma32(a, b, acc);
      }
    }
    store_tile(na, (LDS_AS uint16_t*)As[(st + 1) & 1]);
    store_tile(nb, (LDS_AS uint16_t*)Bs[(st + 1) & 1]);
    __syncthreads();
  };
  Tile a0, b0, aA, bA, aB, bB;
  tiles(0, a0, b0);
  tiles(1, aA, bA);
  store_tile(a0, (LDS_AS uint16_t*)As[0]);
  store_tile(b0, (LDS_AS uint16_t*)Bs[0]);
  __syncthreads();
  for (int64_t st = 0; st < nsteps; st += 2) {   // an odd count runs one more step over zeros
    step(st, aA, bA, aB, bB);
    step(st + 1, aB, bB, aA, bA);
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

// Sum of `splits` fp32 partials, part[k * n + i], added in order k = 0, 1, ...
// starting from 0 (every path that adds these partials uses this order).
// Four outputs per thread: 16-byte loads, all splits' loads of a group of
// four issued before the additions.
__device__ __forceinline__ f32x4 sum_splits4(const f32x4* __restrict__ p4, int splits, int64_t n4, int64_t i4) {
  f32x4 s = {0.0f, 0.0f, 0.0f, 0.0f};
  int k = 0;
  for (; k + 4 <= splits; k += 4) {
    const f32x4 a = p4[(k + 0) * n4 + i4], b = p4[(k + 1) * n4 + i4];
    const f32x4 c = p4[(k + 2) * n4 + i4], d = p4[(k + 3) * n4 + i4];
    s += a;
    s += b;
    s += c;
    s += d;
  }
  for (; k < splits; ++k) s += p4[k * n4 + i4];
  return s;
}

__global__ __launch_bounds__(kThreads) void k_skinny_reduce(const float* __restrict__ part, int splits, int64_t n,
                                                            float scale, uint16_t* __restrict__ out) {
  const int64_t stride = (int64_t)gridDim.x * kThreads;
  const int64_t t0 = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  if ((n & 3) == 0) {
    const int64_t n4 = n >> 2;
    for (int64_t i4 = t0; i4 < n4; i4 += stride) {
      const f32x4 s = sum_splits4((const f32x4*)part, splits, n4, i4);
      *(u32x2*)(out + 4 * i4) = u32x2{qk::pack_bf16x2(scale * s[0], scale * s[1]),
                                      qk::pack_bf16x2(scale * s[2], scale * s[3])};
    }
    return;
  }
  for (int64_t i = t0; i < n; i += stride) {
    float s = 0.0f;
    for (int k = 0; k < splits; ++k) s += part[k * n + i];
    out[i] = qk::f32_to_bf16(scale * s);
  }
}

// C[p, c] partial over one slice of m: sum_m A[m][p] * B[m][c], A [M, P], B [M, r].
template <bool kVecA, bool kVecB>
__global__ __launch_bounds__(kThreads) void k_lora_tn(const uint16_t* __restrict__ A, int64_t lda,
                                                      const uint16_t* __restrict__ B, int64_t M, int64_t P, int r,
                                                      int64_t chunk, float* __restrict__ part) {
  __shared__ __attribute__((aligned(16))) uint16_t As[2][kTile * kPitch];
  __shared__ __attribute__((aligned(16))) uint16_t Bs[2][kTile * kPitch];
  const int w = threadIdx.x >> 6;
  const int wp = w & 1, wc = w >> 1;
  const int64_t p0 = (int64_t)blockIdx.x * kTile;
  const int split = blockIdx.y;
  const int64_t m_beg = split * chunk;
  const int64_t m_end = min(M, m_beg + chunk);
  const int64_t nsteps = (m_end - m_beg + kTile - 1) / kTile;
  auto tiles = [&](int64_t st, Tile& ta, Tile& tb) {
    const int64_t mm = m_beg + st * kTile;
    const int64_t ml = m_end - mm;                     // rows of the slice left (<= 0: zeros)
    const int64_t mmc = ml > 0 ? mm : 0;
    ta = load_tile<kVecA>(A + mmc * lda + p0, lda, ml, P - p0, (uint64_t)((M - mmc) * lda - p0) * 2);   // [m][p]
    tb = load_tile<kVecB>(B + mmc * r, r, ml, r, (uint64_t)((M - mmc) * r) * 2);                // [m][c]
  };
  f32x16 acc = {};
  auto step = [&](int64_t st, const Tile& na, const Tile& nb, Tile& la, Tile& lb) {
    tiles(st + 2, la, lb);
    const LDS_AS uint16_t* as = (const LDS_AS uint16_t*)As[st & 1];
    const LDS_AS uint16_t* bs = (const LDS_AS uint16_t*)Bs[st & 1];
    if (wc * 32 < r) {
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        bf16x8 a = qk::frag_kmajor(as, kPitch, 16 * s, 32 * wp);
        bf16x8 b = qk::frag_kmajor(bs, kPitch, 16 * s, 32 * wc);
        acc = qk::mfma32(a, b, acc);
      }
    }
    store_tile(na, (LDS_AS uint16_t*)As[(st + 1) & 1]);
    store_tile(nb, (LDS_AS uint16_t*)Bs[(st + 1) & 1]);
    __syncthreads();
  };
  Tile a0, b0, aA, bA, aB, bB;
  tiles(0, a0, b0);
  tiles(1, aA, bA);
  store_tile(a0, (LDS_AS uint16_t*)As[0]);
  store_tile(b0, (LDS_AS uint16_t*)Bs[0]);
  __syncthreads();
  for (int64_t st = 0; st < nsteps; st += 2) {
    step(st, aA, bA, aB, bB);
    step(st + 1, aB, bB, aA, bA);
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
                                                        float scale, float* __restrict__ out) {
  const int64_t n = P * r;
  const int64_t stride = (int64_t)gridDim.x * kThreads;
  const int64_t t0 = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  if ((n & 3) == 0) {
    const int64_t n4 = n >> 2;
    for (int64_t i4 = t0; i4 < n4; i4 += stride) ((f32x4*)out)[i4] = scale * sum_splits4((const f32x4*)part, splits, n4, i4);
    return;
  }
  for (int64_t i = t0; i < n; i += stride) {
    float s = 0.0f;
    for (int k = 0; k < splits; ++k) s += part[k * n + i];
    out[i] = scale * s;
  }
}

// Same sum written transposed, out[c * P + p] for the partial element p * r + c:
// a work group takes 16 consecutive p, adds its 16 x r partials (each thread
// four adjacent c of one p when r % 4 == 0, all loads of a group issued
// together) into LDS and writes r rows of 16 contiguous outputs.
constexpr int kTrP = 16;

__global__ __launch_bounds__(kThreads) void k_tn_reduce_t(const float* __restrict__ part, int splits, int64_t P, int r,
                                                          float scale, float* __restrict__ out) {
  __shared__ float tile[kTrP][65];
  const int64_t n = P * r;
  const int64_t p0 = (int64_t)blockIdx.x * kTrP;
  const int np = (int)min((int64_t)kTrP, P - p0);
  if ((r & 3) == 0) {
    const int r4 = r >> 2;
    for (int e = threadIdx.x; e < np * r4; e += kThreads) {
      const int pl = e / r4, c4 = e - pl * r4;
      const f32x4 v = scale * sum_splits4((const f32x4*)part, splits, n >> 2, ((p0 + pl) * r >> 2) + c4);
#pragma unroll
      for (int j = 0; j < 4; ++j) tile[pl][4 * c4 + j] = v[j];
    }
  } else {
    for (int e = threadIdx.x; e < np * r; e += kThreads) {
      const int pl = e / r, c = e - pl * r;
      const int64_t i = (p0 + pl) * r + c;
      float s = 0.0f;
      for (int k = 0; k < splits; ++k) s += part[k * n + i];
      tile[pl][c] = scale * s;
    }
  }
  __syncthreads();
  for (int e = threadIdx.x; e < r * kTrP; e += kThreads) {
    const int c = e / kTrP, pl = e - c * kTrP;
    if (pl < np) out[(int64_t)c * P + p0 + pl] = tile[pl][c];
  }
}

int grid_for(int64_t items) {
  int64_t g = (items + kThreads - 1) / kThreads;
  return (int)(g < 1 ? 1 : (g > 4096 ? 4096 : g));
}

// ---------------------------------------------------------------------------
// T = X L1 at decode-sized M (<= 16): fp32 partial sums over S slices of the
// reduction, part[s][m][c], each slice covering all r columns so that every
// 128-byte row of L1 is read by one work group.  Work group (b, s): columns
// 16 b .. 16 b + 15 of slice s; its 16 waves take 32-row steps in turn with one
// 16x16x32 MFMA each (lane (g, col): X row col, L1 column 16 b + col, rows
// 8 g .. 8 g + 7 of the step) and add their results in LDS in a fixed order.
// The slices are summed in order s = 0 .. S-1 by whoever needs T (the reduce
// kernel below, or the decode kernel's prologue), so every path gets the same T.
constexpr int kPartWaves = 16;
constexpr int kPartCh = 4;

__global__ __launch_bounds__(64 * kPartWaves) void k_lora_part(const uint16_t* __restrict__ X, int64_t M, int64_t K,
                                                               const uint16_t* __restrict__ L1, int r, int64_t rows,
                                                               float* __restrict__ part) {
  __shared__ f32x4 red[kPartWaves * 64];
  const int t = threadIdx.x;
  const int w = __builtin_amdgcn_readfirstlane(t >> 6), l = t & 63;
  const int g = l >> 4, col = l & 15;
  const int c = blockIdx.x * 16 + col;
  const bool c_ok = c < r;
  const bool m_ok = col < M;
  const int64_t k_beg = (int64_t)blockIdx.y * rows;
  const int64_t k_end = min(K, k_beg + rows);
  const int64_t nk = k_end > k_beg ? (k_end - k_beg) / 32 : 0;      // rows and K are multiples of 32
  const int64_t nst = nk > w ? (nk - w + kPartWaves - 1) / kPartWaves : 0;   // uniform
  const __amdgpu_buffer_rsrc_t ra = rsrc(X, (uint64_t)M * K * 2);
  const __amdgpu_buffer_rsrc_t rb = rsrc(L1, (uint64_t)K * r * 2);

  struct Op {
    u32x4 a, b;
  };
  auto load = [&](int64_t i, Op& o) {
    const int64_t k0 = k_beg + 32 * (w + i * kPartWaves) + 8 * g;
    const bool ok = k0 < k_end;
    o.a = __builtin_amdgcn_raw_buffer_load_b128(ra, (ok && m_ok) ? (uint32_t)((col * K + k0) * 2) : kOOB, 0, 0);
    // eight 2-byte loads down column c: one base offset per lane (out of range
    // for an idle lane, so every load returns 0), the row step as a uniform offset
    const uint32_t bo = (ok && c_ok) ? (uint32_t)((k0 * r + c) * 2) : kOOB;
    uint32_t v[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) v[j] = __builtin_amdgcn_raw_buffer_load_b16(rb, bo, 2 * r * j, 0);
#pragma unroll
    for (int j = 0; j < 4; ++j) o.b[j] = v[2 * j] | (v[2 * j + 1] << 16);
  };
  Op ca[kPartCh], cb[kPartCh];
#pragma unroll
  for (int j = 0; j < kPartCh; ++j) load(j, ca[j]);
  f32x4 acc = {0, 0, 0, 0};
  auto mul = [&](int64_t i0, const Op (&o)[kPartCh]) {
#pragma unroll
    for (int j = 0; j < kPartCh; ++j)
      if (i0 + j < nst)
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, o[j].a),
                                                       __builtin_bit_cast(bf16x8, o[j].b), acc, 0, 0, 0);
  };
  for (int64_t i0 = 0; i0 < nst; i0 += 2 * kPartCh) {
    if (i0 + kPartCh < nst) {
#pragma unroll
      for (int j = 0; j < kPartCh; ++j) load(i0 + kPartCh + j, cb[j]);
    }
    mul(i0, ca);
    if (i0 + kPartCh >= nst) break;
    if (i0 + 2 * kPartCh < nst) {
#pragma unroll
      for (int j = 0; j < kPartCh; ++j) load(i0 + 2 * kPartCh + j, ca[j]);
    }
    mul(i0 + kPartCh, cb);
  }
  red[w * 64 + l] = acc;
  __syncthreads();
  if (w == 0) {
    f32x4 sum = red[l];
#pragma unroll
    for (int ww = 1; ww < kPartWaves; ++ww) sum += red[ww * 64 + l];
    // lane l holds C[m = 4 g + i][c]
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int m = 4 * g + i;
      if (m < M && c_ok) part[((int64_t)blockIdx.y * M + m) * r + c] = sum[i];
    }
  }
}

}  // namespace

int decode_t_slices(int64_t K) {
  const int64_t s = K / 512;
  return (int)(s < 1 ? 1 : (s > kDecodeTSlices ? kDecodeTSlices : s));
}

bool decode_t_ok(int64_t M, int64_t K, const void* X, const void* L1) {
  return M >= 1 && M <= 16 && (K % 64) == 0 && ((uintptr_t)X & 15) == 0 && ((uintptr_t)L1 & 1) == 0;
}

hipError_t launch_lora_part(const uint16_t* X, int64_t M, int64_t K, const uint16_t* L1, int r, float* part,
                            hipStream_t s) {
  const int S = decode_t_slices(K);
  const int64_t rows = ((K + S - 1) / S + 31) / 32 * 32;
  dim3 grid((unsigned)((r + 15) / 16), (unsigned)S);
  hipLaunchKernelGGL(k_lora_part, grid, dim3(64 * kPartWaves), 0, s, X, M, K, L1, r, rows, part);
  return hipGetLastError();
}

// Split of a reduction of length R over `tiles` output tiles: about 768 work
// groups in all, but at most one slice per 512 of reduction, so that the fp32
// partials stay small next to the activation pass.
SplitPlan plan_rowsplit(int64_t tiles, int64_t R) {
  int64_t splits = (768 + tiles - 1) / tiles;
  const int64_t max_splits = R / 512;
  if (splits > max_splits) splits = max_splits;
  if (splits < 1) splits = 1;
  int64_t chunk = (R + splits - 1) / splits;
  chunk = (chunk + kTile - 1) / kTile * kTile;
  splits = (R + chunk - 1) / chunk;
  return SplitPlan{(int)splits, chunk};
}

size_t lora_skinny_ws(int64_t M, int64_t R, int r) {
  const SplitPlan sp = plan_rowsplit((M + kTile - 1) / kTile, R);
  const int64_t splits = M <= 16 ? std::max<int64_t>(sp.splits, decode_t_slices(R)) : sp.splits;
  return (size_t)splits * M * r * sizeof(float);
}

hipError_t launch_lora_skinny(const uint16_t* A, int64_t M, int64_t R, int64_t lda, const uint16_t* B, bool b_is_kr,
                              int r, float scale, uint16_t* out, float* ws, hipStream_t s) {
  if (b_is_kr && lda == R && decode_t_ok(M, R, A, B)) {
    // decode-sized T: the slices the decode kernel also sums, added here in the same order
    hipError_t e = launch_lora_part(A, M, R, B, r, ws, s);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(k_skinny_reduce, dim3(grid_for((M * r + 3) / 4)), dim3(kThreads), 0, s, ws, decode_t_slices(R),
                       M * (int64_t)r, scale, out);
    return hipGetLastError();
  }
  const int64_t tiles = (M + kTile - 1) / kTile;
  const SplitPlan sp = plan_rowsplit(tiles, R);
  dim3 grid((unsigned)tiles, (unsigned)sp.splits);
  const bool avec = (R % 8) == 0 && (lda % 8) == 0 && ((uintptr_t)A & 15) == 0;
  const bool bvec = (b_is_kr ? (r % 8) == 0 : (R % 8) == 0) && ((uintptr_t)B & 15) == 0;
#define QL_SKINNY(BKR, VA, VB)                                                                                \
  hipLaunchKernelGGL((k_lora_skinny<BKR, VA, VB>), grid, dim3(kThreads), 0, s, A, M, R, lda, B, r, sp.chunk, ws)
  if (b_is_kr) {
    if (avec && bvec) QL_SKINNY(true, true, true);
    else if (avec) QL_SKINNY(true, true, false);
    else if (bvec) QL_SKINNY(true, false, true);
    else QL_SKINNY(true, false, false);
  } else {
    if (avec && bvec) QL_SKINNY(false, true, true);
    else if (avec) QL_SKINNY(false, true, false);
    else if (bvec) QL_SKINNY(false, false, true);
    else QL_SKINNY(false, false, false);
  }
#undef QL_SKINNY
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(k_skinny_reduce, dim3(grid_for((M * r + 3) / 4)), dim3(kThreads), 0, s, ws, sp.splits, M * (int64_t)r,
                     scale, out);
  return hipGetLastError();
}

size_t lora_tn_ws(int64_t M, int64_t P, int r) {
  const SplitPlan sp = plan_rowsplit((P + kTile - 1) / kTile, M);
  return (size_t)sp.splits * P * r * sizeof(float);
}

hipError_t launch_lora_tn(const uint16_t* A, int64_t lda, const uint16_t* B, int64_t M, int64_t P, int r,
                          float scale, bool transpose_out, float* out, float* ws, hipStream_t s) {
  const int64_t tiles = (P + kTile - 1) / kTile;
  const SplitPlan sp = plan_rowsplit(tiles, M);
  dim3 grid((unsigned)tiles, (unsigned)sp.splits);
  const bool avec = (P % 8) == 0 && (lda % 8) == 0 && ((uintptr_t)A & 15) == 0;
  const bool bvec = (r % 8) == 0 && ((uintptr_t)B & 15) == 0;
#define QL_TN(VA, VB) \
  hipLaunchKernelGGL((k_lora_tn<VA, VB>), grid, dim3(kThreads), 0, s, A, lda, B, M, P, r, sp.chunk, ws)
  if (avec && bvec) QL_TN(true, true);
  else if (avec) QL_TN(true, false);
  else if (bvec) QL_TN(false, true);
  else QL_TN(false, false);
#undef QL_TN
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (transpose_out)
    hipLaunchKernelGGL(k_tn_reduce_t, dim3((unsigned)((P + kTrP - 1) / kTrP)), dim3(kThreads), 0, s, ws, sp.splits, P,
                       r, scale, out);
  else
    hipLaunchKernelGGL(k_tn_reduce, dim3(grid_for((P * r + 3) / 4)), dim3(kThreads), 0, s, ws, sp.splits, P, r, scale,
                       out);
  return hipGetLastError();
}
