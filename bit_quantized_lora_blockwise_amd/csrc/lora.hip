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
#include "tpart.h"

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

// The same partial product for the common case (R, lda, r multiples of 8,
// 8 <= r <= 64, 16-byte aligned operands), laid out for streaming with about one
// work group per CU.  A work group owns 64 rows of A and one slice of the
// reduction and runs 16 waves: wave (g, p) takes rows 16 g .. 16 g + 15 of the
// tile, all r columns (four 16x16x32 MFMA tiles), and the 64-column steps
// p, p + 4, p + 8, ... of the slice.  The rows of A go straight from memory into
// MFMA operand registers (lane l: row l % 16, eight columns at 8 (l / 16)),
// kSkDepth of the wave's steps ahead; the four B tiles of a group of steps
// (64 x 64 each, from L2) are held in registers as far ahead and pass through
// double-buffered LDS, one barrier per group.
// At the end the four phases' sums are added in LDS in the order p = 0 .. 3.
// Per CU this keeps well over 100 KB of A in flight with four waves per SIMD,
// while each slice of B is read once per 64 rows and the slices stay few.
constexpr int kSkGroups = 4;                       // row groups of 16
constexpr int kSkPhases = 4;                       // steps taken in turn
constexpr int kSkThreads = 64 * kSkGroups * kSkPhases;
constexpr int kSkDepth = 4;                        // groups of A and B in flight

template <bool kBkr>
__global__ __launch_bounds__(kSkThreads, 1) void k_lora_skinny_stream(const uint16_t* __restrict__ A, int64_t M,
                                                                     int64_t R, int64_t lda,
                                                                     const uint16_t* __restrict__ Bm, int r,
                                                                     int64_t chunk, float* __restrict__ part) {
  __shared__ __attribute__((aligned(16))) uint16_t Bs[2][kSkPhases][kTile * kPitch];
  const int t = threadIdx.x;
  const int w = __builtin_amdgcn_readfirstlane(t >> 6), l = t & 63;
  const int rg = w % kSkGroups, ph = w / kSkGroups;
  const int64_t m0 = (int64_t)blockIdx.x * kTile;
  const int split = blockIdx.y;
  const int64_t k_beg = split * chunk;
  const int64_t k_end = min(R, k_beg + chunk);
  const int nsteps = (int)((k_end - k_beg + kTile - 1) / kTile);
  const int ngroups = (nsteps + kSkPhases - 1) / kSkPhases;   // group gi: steps kSkPhases gi + p

  // A operand: lane l reads row m0 + 16 rg + l % 16, columns k + 8 (l / 16) .. +8
  const int64_t arow = m0 + 16 * rg + (l & 15);
  const __amdgpu_buffer_rsrc_t ra = rsrc(A, (uint64_t)M * lda * 2);
  const uint32_t abase = (uint32_t)(arow * lda * 2);
  const int64_t akq = 8 * (l >> 4);
  auto load_a = [&](int gi, u32x4 (&v)[2]) {
    const int64_t k0 = k_beg + (int64_t)(kSkPhases * gi + ph) * kTile;
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int64_t k = k0 + 32 * u + akq;
      const bool ok = arow < M && k < k_end;             // k_end is a multiple of 8
      v[u] = __builtin_amdgcn_raw_buffer_load_b128(ra, ok ? abase + (uint32_t)(k * 2) : kOOB, 0, 0);
    }
  };
  // B tiles of a group: threads 256 q .. 256 q + 255 move the tile of step
  // kSkPhases gi + q, thread tt row tt / 8 (+32), eight columns at 8 (tt % 8);
  // kBkr: tile [k][c] from L1 [R, r]; otherwise tile [c][k] from L2 [r, R]
  const __amdgpu_buffer_rsrc_t rb = rsrc(Bm, (uint64_t)R * r * 2);
  const int bq = t >> 8, tt = t & 255;
  auto load_b = [&](int gi, u32x4 (&v)[2]) {
    const int64_t k0 = k_beg + (int64_t)(kSkPhases * gi + bq) * kTile;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int rr = (tt >> 3) + 32 * i, q = 8 * (tt & 7);
      bool ok;
      int64_t off;
      if (kBkr) {
        ok = k0 + rr < k_end && q < r;
        off = (k0 + rr) * r + q;
      } else {
        ok = rr < r && k0 + q < k_end;
        off = (int64_t)rr * R + k0 + q;
      }
      v[i] = __builtin_amdgcn_raw_buffer_load_b128(rb, ok ? (uint32_t)(off * 2) : kOOB, 0, 0);
    }
  };
  auto store_b = [&](const u32x4 (&v)[2], int buf) {
    LDS_AS uint16_t* dst = (LDS_AS uint16_t*)Bs[buf][bq];
#pragma unroll
    for (int i = 0; i < 2; ++i) *(LDS_AS u32x4*)(dst + ((tt >> 3) + 32 * i) * kPitch + 8 * (tt & 7)) = v[i];
  };
  // B operand of the 16x16x32 MFMA: lane l holds B(k + 8 (l / 16) .. +8, c + l % 16)
  auto frag_b = [&](const LDS_AS uint16_t* bs, int k, int c) -> bf16x8 {
    const int G = l >> 4, i = l & 15;
    if (kBkr) {
      // [k][c] tile: transposed reads, each 16-lane group a 4 x 16 block
      const LDS_AS uint16_t* p = bs + (k + 8 * G + (i >> 2)) * kPitch + c + 4 * (i & 3);
      i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS_AS i16x4*)p);
      i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS_AS i16x4*)(p + 4 * kPitch));
      u32x2 a = __builtin_bit_cast(u32x2, lo), b = __builtin_bit_cast(u32x2, hi);
      return __builtin_bit_cast(bf16x8, u32x4{a[0], a[1], b[0], b[1]});
    }
    return *(const LDS_AS bf16x8*)(bs + (c + i) * kPitch + k + 8 * G);
  };

  // this wave's A rows and the work group's B tiles, kSkDepth groups ahead: group
  // gi's A in a[gi % kSkDepth], its B tiles in breg[gi % kSkDepth] until they are
  // stored to LDS during group gi - 1
  u32x4 a[kSkDepth][2], breg[kSkDepth][2];
  // Loads return in issue order, so the B tiles (small, soon needed) are
  // requested ahead of the A rows: a wait for a B tile then never waits for A.
  {
    u32x4 b0[2];
    load_b(0, b0);
#pragma unroll
    for (int j = 1; j <= kSkDepth; ++j) load_b(j, breg[j % kSkDepth]);
#pragma unroll
    for (int j = 0; j < kSkDepth; ++j) load_a(j, a[j]);
    store_b(b0, 0);
  }
  __syncthreads();
  f32x4 acc[4] = {};
  const int ntile = (r + 15) / 16;
  // group gi: MFMAs out of Bs[gi & 1], the tiles of gi + 1 into the other
  // buffer, then the tiles of gi + 1 + kSkDepth and this wave's A rows of
  // gi + kSkDepth are requested
  auto group = [&](int gi, u32x4 (&av)[2], u32x4 (&bn)[2]) {
    const LDS_AS uint16_t* bs = (const LDS_AS uint16_t*)Bs[gi & 1][ph];
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const bf16x8 x = __builtin_bit_cast(bf16x8, av[u]);
#pragma unroll
      for (int j = 0; j < 4; ++j)
        if (j < ntile) acc[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(x, frag_b(bs, 32 * u, 16 * j), acc[j], 0, 0, 0);
    }
    store_b(bn, (gi + 1) & 1);
    load_b(gi + 1 + kSkDepth, bn);
    load_a(gi + kSkDepth, av);
    __syncthreads();
  };
  for (int g0 = 0; g0 < ngroups; g0 += kSkDepth) {
#pragma unroll
    for (int j = 0; j < kSkDepth; ++j)
      if (g0 + j < ngroups) group(g0 + j, a[j], breg[(j + 1) % kSkDepth]);
  }
  // the phases' sums added in order p = 0 .. 3 (the LDS tiles are free: every
  // wave has passed the barrier after its last fragment reads)
  float* red = (float*)&Bs[0][0][0];
#pragma unroll
  for (int j = 0; j < 4; ++j)
#pragma unroll
    for (int v = 0; v < 4; ++v) red[(w * 16 + 4 * j + v) * 64 + l] = acc[j][v];
  __syncthreads();
  if (ph == 0) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int c = 16 * j + (l & 15);
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        float sum = red[(rg * 16 + 4 * j + v) * 64 + l];
#pragma unroll
        for (int p = 1; p < kSkPhases; ++p) sum += red[((p * kSkGroups + rg) * 16 + 4 * j + v) * 64 + l];
        // lane l holds C[4 (l / 16) + v][16 j + l % 16]
        const int64_t m = m0 + 16 * rg + 4 * (l >> 4) + v;
        if (j < ntile && m < M && c < r) part[((int64_t)split * M + m) * r + c] = sum;
      }
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

// C[p, c] partial over one slice of m: sum_m A[m][p] * B[m][c], A [M, P], B [M, r];
// this work group's tile of 64 p is `tile`, its slice of m is `split`.
template <bool kVecA, bool kVecB>
__device__ __forceinline__ void tn_tile(const uint16_t* __restrict__ A, int64_t lda, const uint16_t* __restrict__ B,
                                        int64_t M, int64_t P, int r, int64_t chunk, float* __restrict__ part,
                                        int tile, int split) {
  __shared__ __attribute__((aligned(16))) uint16_t As[2][kTile * kPitch];
  __shared__ __attribute__((aligned(16))) uint16_t Bs[2][kTile * kPitch];
  const int w = threadIdx.x >> 6;
  const int wp = w & 1, wc = w >> 1;
  const int64_t p0 = (int64_t)tile * kTile;
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

template <bool kVecA, bool kVecB>
__global__ __launch_bounds__(kThreads) void k_lora_tn(const uint16_t* __restrict__ A, int64_t lda,
                                                      const uint16_t* __restrict__ B, int64_t M, int64_t P, int r,
                                                      int64_t chunk, float* __restrict__ part) {
  tn_tile<kVecA, kVecB>(A, lda, B, M, P, r, chunk, part, blockIdx.x, blockIdx.y);
}

// Two independent products of this kind in one launch (the backward's dL1 and
// dL2): work groups 0 .. n0 - 1 take the first, the rest the second.
struct TnJob {
  const uint16_t* A;
  int64_t lda;
  const uint16_t* B;
  int64_t P, chunk;
  float* part;
  int tiles, splits;
};

template <bool kVecA, bool kVecB>
__global__ __launch_bounds__(kThreads) void k_lora_tn_pair(TnJob j0, TnJob j1, int64_t M, int r) {
  const int n0 = j0.tiles * j0.splits;
  const bool second = (int)blockIdx.x >= n0;         // uniform over the work group
  const TnJob j = second ? j1 : j0;
  const int b = second ? (int)blockIdx.x - n0 : (int)blockIdx.x;
  tn_tile<kVecA, kVecB>(j.A, j.lda, j.B, M, j.P, r, j.chunk, j.part, b % j.tiles, b / j.tiles);
}

// out[i] = scale * (sum of the slices), i over P * r, by work groups blk of nblk.
__device__ __forceinline__ void tn_reduce_span(const float* __restrict__ part, int splits, int64_t P, int r,
                                               float scale, float* __restrict__ out, int blk, int nblk) {
  const int64_t n = P * r;
  const int64_t stride = (int64_t)nblk * kThreads;
  const int64_t t0 = (int64_t)blk * kThreads + threadIdx.x;
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

__global__ __launch_bounds__(kThreads) void k_tn_reduce(const float* __restrict__ part, int splits, int64_t P, int r,
                                                        float scale, float* __restrict__ out) {
  tn_reduce_span(part, splits, P, r, scale, out, blockIdx.x, gridDim.x);
}

// Same sum written transposed, out[c * P + p] for the partial element p * r + c:
// a work group takes 16 consecutive p, adds its 16 x r partials (each thread
// four adjacent c of one p when r % 4 == 0, all loads of a group issued
// together) into LDS and writes r rows of 16 contiguous outputs.
constexpr int kTrP = 16;

__device__ __forceinline__ void tn_reduce_t_block(const float* __restrict__ part, int splits, int64_t P, int r,
                                                  float scale, float* __restrict__ out, int blk) {
  __shared__ float tile[kTrP][65];
  const int64_t n = P * r;
  const int64_t p0 = (int64_t)blk * kTrP;
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

__global__ __launch_bounds__(kThreads) void k_tn_reduce_t(const float* __restrict__ part, int splits, int64_t P, int r,
                                                          float scale, float* __restrict__ out) {
  tn_reduce_t_block(part, splits, P, r, scale, out, blockIdx.x);
}

// The two sums of a k_lora_tn_pair launch in one launch: work groups 0 .. nb0 - 1
// write the first product as out0[P0, r], the rest the second transposed as
// out1[r, P1].
__global__ __launch_bounds__(kThreads) void k_tn_reduce_pair(const float* __restrict__ part0, int splits0, int64_t P0,
                                                             float scale0, float* __restrict__ out0, int nb0,
                                                             const float* __restrict__ part1, int splits1, int64_t P1,
                                                             float scale1, float* __restrict__ out1, int r) {
  if ((int)blockIdx.x < nb0) tn_reduce_span(part0, splits0, P0, r, scale0, out0, blockIdx.x, nb0);
  else tn_reduce_t_block(part1, splits1, P1, r, scale1, out1, (int)blockIdx.x - nb0);
}

int grid_for(int64_t items) {
  int64_t g = (items + kThreads - 1) / kThreads;
  return (int)(g < 1 ? 1 : (g > 4096 ? 4096 : g));
}

// ---------------------------------------------------------------------------
// T = X L1 at decode-sized M (<= 16): fp32 partial sums over S slices of the
// reduction, part[s][m][c], each slice covering all r columns so that every
// 128-byte row of L1 is read by one work group.  Work group (b, s): columns
// 16 b .. 16 b + 15 of slice s, sixteen waves, one per virtual wave of
// tpart::slice_tile (32-row steps, one 16x16x32 MFMA each, the waves' results
// added in LDS in a fixed order).  The slices are summed in order s = 0 .. S-1
// by whoever needs T (the reduce kernel below, or the decode kernel), so every
// path gets the same T; the decode kernel can also form the slices itself with
// the same function.
// Stacked linears: G adapters L1_g [K, r] at L1 + g K r, all in one launch (the
// column tiles of segment g follow those of g - 1), slices of segment g at
// part + g S M r.
__global__ __launch_bounds__(64 * tpart::kVirt) void k_lora_part(const uint16_t* __restrict__ X, int64_t M, int64_t K,
                                                                const uint16_t* __restrict__ L1, int r, int64_t rows,
                                                                float* __restrict__ part) {
  __shared__ f32x4 red[tpart::kVirt * 64];
  const int ctiles = (r + 15) / 16;
  const int seg = blockIdx.x / ctiles;                    // stacked adapter of this work group
  tpart::slice_tile<tpart::kVirt>(X, M, K, L1 + (int64_t)seg * K * r, r, rows,
                                  part + (int64_t)seg * gridDim.y * M * r, (int)blockIdx.x - seg * ctiles,
                                  (int)blockIdx.y, red);
}

}  // namespace

int decode_t_slices(int64_t K) {
  const int64_t s = K / 512;
  return (int)(s < 1 ? 1 : (s > kDecodeTSlices ? kDecodeTSlices : s));
}

int64_t decode_t_rows(int64_t K) {
  const int S = decode_t_slices(K);
  return ((K + S - 1) / S + 31) / 32 * 32;
}

bool decode_t_ok(int64_t M, int64_t K, const void* X, const void* L1) {
  return M >= 1 && M <= 16 && (K % 64) == 0 && ((uintptr_t)X & 15) == 0 && ((uintptr_t)L1 & 1) == 0;
}

hipError_t launch_lora_part(const uint16_t* X, int64_t M, int64_t K, const uint16_t* L1, int r, float* part,
                            hipStream_t s, int G) {
  const int S = decode_t_slices(K);
  const int64_t rows = decode_t_rows(K);
  dim3 grid((unsigned)(G * ((r + 15) / 16)), (unsigned)S);
  hipLaunchKernelGGL(k_lora_part, grid, dim3(64 * tpart::kVirt), 0, s, X, M, K, L1, r, rows, part);
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

// Split for the streaming kernel: about one work group per CU (64-row tiles
// times slices), each slice at least four 64-column steps long.
static SplitPlan plan_stream(int64_t tiles, int64_t R) {
  static const int cus = [] {
    int dev = 0, n = 0;
    if (hipGetDevice(&dev) != hipSuccess || hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) !=
                                                hipSuccess || n < 1)
      n = 256;
    return n;
  }();
  int64_t splits = (cus + tiles / 2) / tiles;
  const int64_t max_splits = R / 256;
  if (splits > max_splits) splits = max_splits;
  if (splits < 1) splits = 1;
  int64_t chunk = (R + splits - 1) / splits;
  chunk = (chunk + kTile - 1) / kTile * kTile;
  splits = (R + chunk - 1) / chunk;
  return SplitPlan{(int)splits, chunk};
}

static bool skinny_stream_ok(const uint16_t* A, int64_t M, int64_t R, int64_t lda, const uint16_t* B, int r) {
  return (R % 8) == 0 && (lda % 8) == 0 && (r % 8) == 0 && r >= 8 && r <= 64 && ((uintptr_t)A & 15) == 0 &&
         ((uintptr_t)B & 15) == 0 && M * lda * 2 < (int64_t(1) << 31) && R * r * 2 < (int64_t(1) << 31);
}

size_t lora_skinny_ws(int64_t M, int64_t R, int r) {
  const int64_t tiles = (M + kTile - 1) / kTile;
  int64_t splits = std::max<int64_t>(plan_rowsplit(tiles, R).splits, plan_stream(tiles, R).splits);
  if (M <= 16) splits = std::max<int64_t>(splits, decode_t_slices(R));
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
  if (skinny_stream_ok(A, M, R, lda, B, r)) {
    const SplitPlan sp = plan_stream(tiles, R);
    dim3 grid((unsigned)tiles, (unsigned)sp.splits);
    if (b_is_kr)
      hipLaunchKernelGGL((k_lora_skinny_stream<true>), grid, dim3(kSkThreads), 0, s, A, M, R, lda, B, r, sp.chunk, ws);
    else
      hipLaunchKernelGGL((k_lora_skinny_stream<false>), grid, dim3(kSkThreads), 0, s, A, M, R, lda, B, r, sp.chunk, ws);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(k_skinny_reduce, dim3(grid_for((M * r + 3) / 4)), dim3(kThreads), 0, s, ws, sp.splits,
                       M * (int64_t)r, scale, out);
    return hipGetLastError();
  }
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

size_t lora_tn_pair_ws(int64_t M, int64_t P0, int64_t P1, int r) {
  return (lora_tn_ws(M, P0, r) + 255) / 256 * 256 + lora_tn_ws(M, P1, r);
}

hipError_t launch_lora_tn_pair(const uint16_t* A0, int64_t lda0, const uint16_t* B0, int64_t P0, float scale0,
                               float* out0, const uint16_t* A1, int64_t lda1, const uint16_t* B1, int64_t P1,
                               float scale1, float* out1_t, int64_t M, int r, float* ws, hipStream_t s) {
  const bool vec = (P0 % 8) == 0 && (lda0 % 8) == 0 && ((uintptr_t)A0 & 15) == 0 && (P1 % 8) == 0 &&
                   (lda1 % 8) == 0 && ((uintptr_t)A1 & 15) == 0 && (r % 8) == 0 && ((uintptr_t)B0 & 15) == 0 &&
                   ((uintptr_t)B1 & 15) == 0;
  float* part1 = ws + (lora_tn_ws(M, P0, r) + 255) / 256 * 256 / sizeof(float);
  if (!vec) {
    hipError_t e = launch_lora_tn(A0, lda0, B0, M, P0, r, scale0, false, out0, ws, s);
    if (e != hipSuccess) return e;
    return launch_lora_tn(A1, lda1, B1, M, P1, r, scale1, true, out1_t, part1, s);
  }
  const SplitPlan sp0 = plan_rowsplit((P0 + kTile - 1) / kTile, M);
  const SplitPlan sp1 = plan_rowsplit((P1 + kTile - 1) / kTile, M);
  const TnJob j0{A0, lda0, B0, P0, sp0.chunk, ws, (int)((P0 + kTile - 1) / kTile), sp0.splits};
  const TnJob j1{A1, lda1, B1, P1, sp1.chunk, part1, (int)((P1 + kTile - 1) / kTile), sp1.splits};
  const unsigned nwg = (unsigned)(j0.tiles * j0.splits + j1.tiles * j1.splits);
  hipLaunchKernelGGL((k_lora_tn_pair<true, true>), dim3(nwg), dim3(kThreads), 0, s, j0, j1, M, r);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int nb0 = grid_for((P0 * r + 3) / 4);
  const unsigned nb1 = (unsigned)((P1 + kTrP - 1) / kTrP);
  hipLaunchKernelGGL(k_tn_reduce_pair, dim3((unsigned)nb0 + nb1), dim3(kThreads), 0, s, ws, sp0.splits, P0, scale0,
                     out0, nb0, part1, sp1.splits, P1, scale1, out1_t, r);
  return hipGetLastError();
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
