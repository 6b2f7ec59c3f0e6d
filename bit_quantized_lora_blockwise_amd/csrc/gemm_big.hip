// Quantised GEMMs of the layer for training-sized M, large-tile version:
//   forward  Y  = bf16(X W'^T + s T L2)       (C = Y,  P = N, reduction R = K)
//   backward dX = bf16(dY W' + G L1^T)        (C = dX, P = K, reduction R = N)
// Layer formula: nlp-lineage milestone page on QLoRA, "The idea", notation
// paragraph; the frozen base is dequantised on the fly (examadda page, "The
// Core Idea"; inferensys glossary, paragraph on the dequantising kernel).
//
// Tile: 256 rows of the activation x 256 output columns, reduction steps of 64.
// Four waves; wave w owns activation rows 64 w .. 64 w + 63 and all 256 output
// columns, i.e. 2 x 8 MFMA 32x32x16 tiles (256 fp32 accumulators per lane).
//  * The activation (X or dY) goes straight from HBM into MFMA A fragments,
//    one step ahead; no wave shares them.
//  * The weight tile is rebuilt from the packed 4-bit stream once per work
//    group: each thread dequantises one first-level block (64 weights) per step
//    into a double-buffered LDS tile, and every wave reads its B fragments from
//    there (directly in the forward, through ds_read_b64_tr_b16 in the dX path,
//    where the reduction runs across the stored rows of W).
//  * Dequantisation keeps the block's 16 bf16 values W'(v) = bf16(fl32(q[v] s'))
//    in registers as two byte planes and looks each nibble up with v_perm_b32
//    (three byte selects per four nibbles and plane), so it needs no LDS reads.
#include "kernels.h"

namespace {

constexpr int kT = 256;           // threads per work group
constexpr int kBM = 256;          // activation rows per tile
constexpr int kBP = 256;          // output columns per tile
constexpr int kBR = 64;           // reduction per step
constexpr int kPF = kBR + 8;      // pitch of the forward B tile [p][r] (elements)
constexpr int kPD = kBP + 32;     // pitch of the dX B tile [r][p] (elements): 144 dwords, so the
                                  // 4 rows x 2 column halves of a 32-lane transposed read hit 64 banks
constexpr int kBufElems = (kBP * kPF > kBR * kPD) ? kBP * kPF : kBR * kPD;
constexpr int kPL = 64 + 8;       // pitch of the LoRA A tile [m][c]
constexpr uint32_t kOOB = 0x80000000u;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void* p, uint64_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc((void*)p, (short)0, (int)bytes, 0x00020000);
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

// ---------------------------------------------------------------------------
// Dequantisation of one block held in registers.
struct BlockLut {
  uint32_t lo[4], hi[4];   // byte planes: lo[j] byte i = low byte of W'(4 j + i), hi likewise
};

__device__ __forceinline__ BlockLut make_lut(float s, const Nf4Params& p) {
  uint32_t pk[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) pk[i] = qk::pack_bf16x2(p.q[2 * i] * s, p.q[2 * i + 1] * s);
  BlockLut L;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    L.lo[j] = __builtin_amdgcn_perm(pk[2 * j + 1], pk[2 * j], 0x06040200u);
    L.hi[j] = __builtin_amdgcn_perm(pk[2 * j + 1], pk[2 * j], 0x07050301u);
  }
  return L;
}

// 16-entry byte lookup of the four index bytes of x (values 0..15).
__device__ __forceinline__ uint32_t lut16(const uint32_t (&T)[4], uint32_t x, uint32_t x7, uint32_t selc) {
  const uint32_t a = __builtin_amdgcn_perm(T[1], T[0], x);    // entries 0..7 (bytes of x < 8 are right)
  const uint32_t b = __builtin_amdgcn_perm(T[3], T[2], x7);   // entries 8..15
  return __builtin_amdgcn_perm(b, a, selc);                   // byte i from b when x_i >= 8
}

// Eight nibbles (one 32-bit word, element j in bits 4j..4j+3) -> four packed
// bf16 pairs in element order.
__device__ __forceinline__ u32x4 dequant8(const BlockLut& L, uint32_t c) {
  const uint32_t xe = c & 0x0F0F0F0Fu;             // elements 0, 2, 4, 6
  const uint32_t xo = (c >> 4) & 0x0F0F0F0Fu;      // elements 1, 3, 5, 7
  const uint32_t se = ((xe >> 1) & 0x04040404u) | 0x03020100u;
  const uint32_t so = ((xo >> 1) & 0x04040404u) | 0x03020100u;
  const uint32_t xe7 = xe & 0x07070707u, xo7 = xo & 0x07070707u;
  const uint32_t le = lut16(L.lo, xe, xe7, se), he = lut16(L.hi, xe, xe7, se);
  const uint32_t lo_ = lut16(L.lo, xo, xo7, so), ho = lut16(L.hi, xo, xo7, so);
  const uint32_t e02 = __builtin_amdgcn_perm(he, le, 0x05010400u);   // [W'(e0), W'(e2)]
  const uint32_t e46 = __builtin_amdgcn_perm(he, le, 0x07030602u);   // [W'(e4), W'(e6)]
  const uint32_t o13 = __builtin_amdgcn_perm(ho, lo_, 0x05010400u);  // [W'(e1), W'(e3)]
  const uint32_t o57 = __builtin_amdgcn_perm(ho, lo_, 0x07030602u);  // [W'(e5), W'(e7)]
  u32x4 r;
  r[0] = __builtin_amdgcn_perm(o13, e02, 0x05040100u);   // e0, e1
  r[1] = __builtin_amdgcn_perm(o13, e02, 0x07060302u);   // e2, e3
  r[2] = __builtin_amdgcn_perm(o57, e46, 0x05040100u);   // e4, e5
  r[3] = __builtin_amdgcn_perm(o57, e46, 0x07060302u);   // e6, e7
  return r;
}

// A block's packed codes, scale byte and group scale, as loaded for one step.
struct BlockCodes {
  u32x4 c0, c1;
  uint32_t c2b;
  float c1v;
};

// ---------------------------------------------------------------------------
template <bool kDx>
__global__ __launch_bounds__(kT, 1) void k_qgemm_big(const uint16_t* __restrict__ A, int64_t M, int64_t K,
                                                     int64_t N, const uint8_t* __restrict__ codes,
                                                     const uint8_t* __restrict__ c2,
                                                     const float* __restrict__ c1,
                                                     const uint16_t* __restrict__ LA,   // T (fwd) / G (dX)
                                                     const uint16_t* __restrict__ LB,   // L2 (fwd) / L1 (dX)
                                                     int r, float scale, uint16_t* __restrict__ C,
                                                     Nf4Params p) {
  __shared__ __attribute__((aligned(16))) uint16_t lds[2 * kBufElems];
  const int t = threadIdx.x;
  const int w = t >> 6, l = t & 63;
  const int64_t P = kDx ? K : N;          // output columns
  const int64_t R = kDx ? N : K;          // reduction length
  const int64_t m0 = (int64_t)blockIdx.y * kBM;
  const int64_t p0 = (int64_t)blockIdx.x * kBP;
  const int64_t kblocks = K / qk::kBlock;

  f32x16 acc[2][8];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[i][j] = f32x16{};

  // ---- LoRA term first, one 32x32 tile at a time: fwd acc = s * (T L2); dX acc = G L1^T
  //      (rank zero-padded to 64); the base product then accumulates onto it.
  {
    LDS_AS uint16_t* la = (LDS_AS uint16_t*)lds;                 // [256][kPL]: T / G rows
    LDS_AS uint16_t* lb = (LDS_AS uint16_t*)lds + kBM * kPL;     // fwd: L2 [64][kPD]; dX: L1 [256][kPL]
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int row = (t >> 3) + 32 * i, cc = (t & 7) * 8;
      u32x4 v = {0, 0, 0, 0};
      if (m0 + row < M) v = load_row8(LA + (m0 + row) * r, cc, r);
      *(LDS_AS u32x4*)(la + row * kPL + cc) = v;
    }
    if (!kDx) {
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int c = (t >> 5) + 8 * i, pp = (t & 31) * 8;
        u32x4 v = {0, 0, 0, 0};
        if (c < r) v = load_row8(LB + (int64_t)c * N, p0 + pp, N);
        *(LDS_AS u32x4*)(lb + c * kPD + pp) = v;
      }
    } else {
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int row = (t >> 3) + 32 * i, cc = (t & 7) * 8;
        u32x4 v = {0, 0, 0, 0};
        if (p0 + row < K) v = load_row8(LB + (p0 + row) * r, cc, r);
        *(LDS_AS u32x4*)(lb + row * kPL + cc) = v;
      }
    }
    __syncthreads();
    const int ksteps = (r + 15) / 16;
    const float ls = kDx ? 1.0f : scale;
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        f32x16 z = {};
        for (int s = 0; s < ksteps; ++s) {
          const bf16x8 a = qk::frag_rowmajor(la, kPL, 64 * w + 32 * i, 16 * s);
          const bf16x8 b = kDx ? qk::frag_rowmajor(lb, kPL, 32 * j, 16 * s) : qk::frag_kmajor(lb, kPD, 16 * s, 32 * j);
          z = qk::mfma32(a, b, z);
        }
        acc[i][j] = ls * z;
      }
    __syncthreads();
  }

  // ---- per-thread roles
  // A fragments: rows m0 + 64 w + 32 i + l % 32, reduction columns 16 s + 8 (l / 32).
  const __amdgpu_buffer_rsrc_t ra = rsrc(A, (uint64_t)M * R * 2);
  const int64_t arow0 = m0 + 64 * w + (l & 31);
  const uint32_t aoff0 = (uint32_t)(arow0 * R * 2) + 16u * (uint32_t)(l >> 5);
  const uint32_t aoff1 = aoff0 + (uint32_t)(32 * R * 2);
  const bool arow0_ok = arow0 < M, arow1_ok = arow0 + 32 < M;
  auto load_a = [&](int64_t rs, u32x4 (&a)[2][4]) {   // rs: first reduction index of the step
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const int64_t col = rs + 16 * s + 8 * (l >> 5);
      const bool cok = col < R;
      const uint32_t d = (uint32_t)(rs * 2 + 32 * s);
      a[0][s] = __builtin_amdgcn_raw_buffer_load_b128(ra, (arow0_ok && cok) ? aoff0 + d : kOOB, 0, 0);
      a[1][s] = __builtin_amdgcn_raw_buffer_load_b128(ra, (arow1_ok && cok) ? aoff1 + d : kOOB, 0, 0);
    }
  };
  // Dequantisation role: one block per thread per step.
  //  fwd: weight row p0 + t, block = step;            tile position [t][0..64)
  //  dX : weight row rs + t / 4, block (p0 / 64) + t % 4; tile position [t / 4][64 (t % 4) ..)
  const __amdgpu_buffer_rsrc_t rc = rsrc(codes, (uint64_t)N * (K / 2));
  const __amdgpu_buffer_rsrc_t r2 = rsrc(c2, (uint64_t)N * kblocks);
  const __amdgpu_buffer_rsrc_t r1 = rsrc(c1, 4 * (((uint64_t)N * kblocks + 255) / 256));
  auto load_codes = [&](int64_t step) {
    int64_t wrow, kb;
    if (!kDx) { wrow = p0 + t; kb = step; }
    else { wrow = step * kBR + (t >> 2); kb = p0 / 64 + (t & 3); }
    const bool ok = wrow < N && kb < kblocks;
    const uint32_t co = ok ? (uint32_t)(wrow * (K / 2) + kb * 32) : kOOB;
    const uint32_t b = (uint32_t)(wrow * kblocks + kb);
    BlockCodes bc;
    bc.c0 = __builtin_amdgcn_raw_buffer_load_b128(rc, co, 0, 0);
    bc.c1 = __builtin_amdgcn_raw_buffer_load_b128(rc, co + 16, 0, 0);
    bc.c2b = __builtin_amdgcn_raw_buffer_load_b8(r2, ok ? b : kOOB, 0, 0);
    bc.c1v = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(r1, ok ? 4 * (b >> 8) : kOOB, 0, 0));
    return bc;
  };
  auto dequant_store = [&](const BlockCodes& bc, LDS_AS uint16_t* buf) {
    const BlockLut L = make_lut(qk::e4m3fn_to_f32(bc.c2b) * bc.c1v, p);
    LDS_AS uint16_t* dst = kDx ? buf + (t >> 2) * kPD + 64 * (t & 3) : buf + t * kPF;
#pragma unroll
    for (int j = 0; j < 4; ++j) *(LDS_AS u32x4*)(dst + 8 * j) = dequant8(L, bc.c0[j]);
#pragma unroll
    for (int j = 0; j < 4; ++j) *(LDS_AS u32x4*)(dst + 32 + 8 * j) = dequant8(L, bc.c1[j]);
  };
  // ---- main loop.  Step st multiplies A(st) (registers) by the B tile in LDS
  // buffer st % 2 while it dequantises block codes(st + 1) into the other
  // buffer; the codes are loaded two steps ahead and the A fragments one step
  // ahead.  The body has no branches (out-of-range steps load zeros), so the
  // MFMAs, the dequantisation VALU work and the LDS traffic interleave.
  LDS_AS uint16_t* buf0 = (LDS_AS uint16_t*)lds;
  LDS_AS uint16_t* buf1 = (LDS_AS uint16_t*)lds + kBufElems;
  const int64_t nsteps = (R + kBR - 1) / kBR;
  auto step = [&](int64_t st, const u32x4 (&acur)[2][4], u32x4 (&anext)[2][4], const LDS_AS uint16_t* bcur,
                  LDS_AS uint16_t* bnext, const BlockCodes& bc_now, BlockCodes& bc_later) {
    bc_later = load_codes(st + 2);
    load_a((st + 1) * kBR, anext);
    const BlockLut L = make_lut(qk::e4m3fn_to_f32(bc_now.c2b) * bc_now.c1v, p);
    LDS_AS uint16_t* dst = kDx ? bnext + (t >> 2) * kPD + 64 * (t & 3) : bnext + t * kPF;
    // B fragments of sub-step s + 1 are read from LDS while sub-step s runs
    auto bfrag = [&](int s, int j) {
      return kDx ? qk::frag_kmajor(bcur, kPD, 16 * s, 32 * j) : qk::frag_rowmajor(bcur, kPF, 32 * j, 16 * s);
    };
    bf16x8 bq[2][8];
#pragma unroll
    for (int j = 0; j < 8; ++j) bq[0][j] = bfrag(0, j);
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      if (s < 3) {
#pragma unroll
        for (int j = 0; j < 8; ++j) bq[(s + 1) & 1][j] = bfrag(s + 1, j);
      }
      const bf16x8 a0 = __builtin_bit_cast(bf16x8, acur[0][s]);
      const bf16x8 a1 = __builtin_bit_cast(bf16x8, acur[1][s]);
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        acc[0][j] = qk::mfma32(a0, bq[s & 1][j], acc[0][j]);
        acc[1][j] = qk::mfma32(a1, bq[s & 1][j], acc[1][j]);
      }
      // two of the eight 8-weight groups of the next tile per sub-step
      const u32x4 cw = (s < 2) ? bc_now.c0 : bc_now.c1;
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int q = 2 * (s & 1) + h;          // code word within cw
        *(LDS_AS u32x4*)(dst + 32 * (s >> 1) + 8 * q) = dequant8(L, cw[q]);
      }
      // schedule: the next sub-step's fragment reads first, then MFMA pairs
      // interleaved with the dequantisation VALU work, then the LDS stores
      if (s < 3) __builtin_amdgcn_sched_group_barrier(0x100, kDx ? 16 : 8, 0);   // DS read
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);                        // MFMA
        __builtin_amdgcn_sched_group_barrier(0x002, kDx ? 14 : 11, 0);            // VALU
      }
      __builtin_amdgcn_sched_group_barrier(0x200, 2, 0);                          // DS write
    }
    __syncthreads();
  };
  u32x4 aA[2][4], aB[2][4];
  BlockCodes bcA, bcB;
  {
    const BlockCodes bc0 = load_codes(0);
    bcA = load_codes(1);
    load_a(0, aA);
    dequant_store(bc0, buf0);
    __syncthreads();
  }
  // bcA holds codes(st + 1) at the top of each even step
  for (int64_t st = 0; st < nsteps; st += 2) {
    step(st, aA, aB, buf0, buf1, bcA, bcB);
    if (st + 1 >= nsteps) break;
    step(st + 1, aB, aA, buf1, buf0, bcB, bcA);
  }

  // ---- store C (bf16), lane layout of the 32x32 accumulators
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int64_t pc = p0 + 32 * j + qk::acc_col();
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int64_t m = m0 + 64 * w + 32 * i + qk::acc_row(e);
        if (m < M && pc < P) C[m * P + pc] = qk::f32_to_bf16(acc[i][j][e]);
      }
    }
}

}  // namespace

bool qgemm_big_ok(bool dx, int64_t M, int64_t K, int64_t N) {
  // 32-bit buffer offsets; 16-byte aligned activation rows (R % 8 == 0)
  const int64_t R = dx ? N : K;
  return (R % 8) == 0 && M * R * 2 < (int64_t(1) << 31) && N * (K / 2) < (int64_t(1) << 31) && M > 16;
}

hipError_t launch_qgemm_big(bool dx, const uint16_t* A, int64_t M, int64_t K, int64_t N, const uint8_t* codes,
                            const uint8_t* c2, const float* c1, const uint16_t* LA, const uint16_t* LB, int r,
                            float scale, uint16_t* C, hipStream_t s) {
  const int64_t P = dx ? K : N;
  dim3 grid((unsigned)((P + kBP - 1) / kBP), (unsigned)((M + kBM - 1) / kBM));
  if (dx)
    hipLaunchKernelGGL(k_qgemm_big<true>, grid, dim3(kT), 0, s, A, M, K, N, codes, c2, c1, LA, LB, r, scale, C,
                       nf4_params());
  else
    hipLaunchKernelGGL(k_qgemm_big<false>, grid, dim3(kT), 0, s, A, M, K, N, codes, c2, c1, LA, LB, r, scale, C,
                       nf4_params());
  return hipGetLastError();
}
