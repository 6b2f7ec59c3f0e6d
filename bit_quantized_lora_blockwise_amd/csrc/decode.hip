// Decode-sized forward (M <= 16): Y = bf16(X W'^T + s T L2) as one pass over
// the packed 4-bit weight stream.  At these sizes the layer is bound by HBM
// traffic of the codes and scales and by the VALU work of the dequantisation;
// the bf16 weights live only in registers and feed a 16x16x32 bf16 MFMA
// against X.
// Layer formula: nlp-lineage milestone page on QLoRA, "The idea", notation
// paragraph; dequantisation on the fly: examadda page, "The Core Idea".
//
// Work group: 16 weight rows x all of K, four waves taking 256-column steps in
// turn; in a step, lane (g = l / 16, row = l % 16) holds one block (64 weights,
// 32 bytes of codes): it builds the block's 16-entry bf16 table in registers
// (two byte planes) and looks each nibble up with v_perm_b32.
// When X is small (M * K <= 16384) it is staged once in LDS, with each group of
// eight columns stored in the order (0, 2, 4, 6, 1, 3, 5, 7): that is the order
// in which the lookups produce the weights (low nibbles, then high nibbles), so
// the MFMA needs no re-interleaving of the looked-up values.  The staging is
// finished before the code stream is requested, so the first steps do not wait
// for X behind the stream.  Larger X is read per step from global memory.
#include "kernels.h"

namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / 64;
constexpr int kRows = 16;                 // weight rows (output columns) per work group
constexpr int kChunk = 4;                 // steps of a lane whose loads are issued together
constexpr int kXBytes = 32768;            // LDS budget for X: M * K <= 16384
constexpr int kZeroBytes = 128;           // zeros read in place of X by idle lanes
constexpr int kRedBytes = kWaves * 64 * 16;
constexpr uint32_t kOOB = 0x80000000u;    // buffer offset past every range: the load returns 0

__device__ __forceinline__ f32x4 mfma16(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void* p, uint64_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc((void*)p, (short)0, (int)bytes, 0x00020000);
}

// ---------------------------------------------------------------------------
// One block's dequantisation table held in registers.
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


// Same lookup, weights in the order (0, 2, 4, 6, 1, 3, 5, 7) of the word.
__device__ __forceinline__ u32x4 dequant8_eo(const BlockLut& L, uint32_t c) {
  const uint32_t xe = c & 0x0F0F0F0Fu;
  const uint32_t xo = (c >> 4) & 0x0F0F0F0Fu;
  const uint32_t se = ((xe >> 1) & 0x04040404u) | 0x03020100u;
  const uint32_t so = ((xo >> 1) & 0x04040404u) | 0x03020100u;
  const uint32_t xe7 = xe & 0x07070707u, xo7 = xo & 0x07070707u;
  const uint32_t le = lut16(L.lo, xe, xe7, se), he = lut16(L.hi, xe, xe7, se);
  const uint32_t lo_ = lut16(L.lo, xo, xo7, so), ho = lut16(L.hi, xo, xo7, so);
  u32x4 r;
  r[0] = __builtin_amdgcn_perm(he, le, 0x05010400u);    // W'(e0), W'(e2)
  r[1] = __builtin_amdgcn_perm(he, le, 0x07030602u);    // W'(e4), W'(e6)
  r[2] = __builtin_amdgcn_perm(ho, lo_, 0x05010400u);   // W'(e1), W'(e3)
  r[3] = __builtin_amdgcn_perm(ho, lo_, 0x07030602u);   // W'(e5), W'(e7)
  return r;
}

// Codes and scales of kChunk steps of one lane.
struct Chunk {
  u32x4 cw[kChunk][2];
  uint32_t c2b[kChunk];
  float c1v[kChunk];
};

template <bool kXLds>
__global__ __launch_bounds__(kThreads) void k_qgemv_fwd(const uint16_t* __restrict__ X, int64_t M, int64_t K,
                                                        int64_t N, int64_t ld, const uint8_t* __restrict__ codes,
                                                        const uint8_t* __restrict__ c2,
                                                        const float* __restrict__ c1,
                                                        const uint16_t* __restrict__ T,
                                                        const uint16_t* __restrict__ L2, int r, float scale,
                                                        uint16_t* __restrict__ Y, Nf4Params p) {
  __shared__ __attribute__((aligned(16))) uint8_t lds[(kXLds ? kXBytes + kZeroBytes : 0) + kRedBytes];
  const int t = threadIdx.x;
  const int w = __builtin_amdgcn_readfirstlane(t >> 6), l = t & 63;
  const int g = l >> 4, col = l & 15;
  const int64_t n0 = (int64_t)blockIdx.x * kRows;
  const int64_t nrow = n0 + col;
  const bool row_ok = nrow < N;
  const bool m_ok = col < M;                       // A-operand row of this lane is X[col]
  const uint32_t kblocks = (uint32_t)(K / qk::kBlock);

  // K is walked in steps of four blocks (256 columns); the waves take the steps
  // in turn, and in step s lane group g takes block 4 s + g, so the four lanes
  // of a row read 128 contiguous bytes of codes.  Step i of wave w is s = w + 4 i.
  const uint32_t nsteps = (kblocks + 3) / 4;
  const uint32_t nst = nsteps > (uint32_t)w ? (nsteps - (uint32_t)w + kWaves - 1) / kWaves : 0u;   // uniform
  const uint32_t kb0 = 4u * (uint32_t)w + (uint32_t)g;
  const uint32_t kbstep = 4u * kWaves;
  const uint32_t kb_lim = row_ok ? kblocks : 0u;   // blocks valid for the lane's weight row

  const __amdgpu_buffer_rsrc_t rc = rsrc(codes, (uint64_t)N * (K / 2));
  const __amdgpu_buffer_rsrc_t r2 = rsrc(c2, (uint64_t)N * kblocks);
  const __amdgpu_buffer_rsrc_t r1 = rsrc(c1, 4 * (((uint64_t)N * kblocks + 255) / 256));
  const __amdgpu_buffer_rsrc_t rx = rsrc(X, (uint64_t)M * K * 2);

  // ---- small X: its loads are issued first, then the first chunk of the code
  // stream, then X is written to LDS (waiting for the X loads only).  Every
  // 16-byte group of eight columns is stored as (0, 2, 4, 6, 1, 3, 5, 7).
  LDS_AS uint8_t* xl = (LDS_AS uint8_t*)lds;
  constexpr int kXPer = kXBytes / (16 * kThreads);       // 16-byte X loads per thread
  u32x4 xr[kXLds ? kXPer : 1];
  const uint32_t xbytes = kXLds ? (uint32_t)(M * K * 2) : 0u;
  if (kXLds) {
#pragma unroll
    for (int j = 0; j < kXPer; ++j) {
      const uint32_t o = 16u * (uint32_t)(t + j * kThreads);
      xr[j] = __builtin_amdgcn_raw_buffer_load_b128(rx, o < xbytes ? o : kOOB, 0, 0);
    }
  }
  __builtin_amdgcn_sched_barrier(0);
  // ---- code stream: chunk c covers steps 4c .. 4c + 3 of the lane
  const uint32_t code_row = (uint32_t)(nrow * (K / 2));
  const uint32_t blk_row = (uint32_t)(nrow * kblocks);
  auto load_chunk = [&](uint32_t i0, Chunk& ch) {
#pragma unroll
    for (int i = 0; i < kChunk; ++i) {
      const uint32_t kb = kb0 + (i0 + i) * kbstep;
      const bool ok = kb < kb_lim;
      const uint32_t co = ok ? code_row + 32u * kb : kOOB;
      const uint32_t b = blk_row + kb;
      ch.cw[i][0] = __builtin_amdgcn_raw_buffer_load_b128(rc, co, 0, 0);
      ch.cw[i][1] = __builtin_amdgcn_raw_buffer_load_b128(rc, co + 16, 0, 0);
      ch.c2b[i] = __builtin_amdgcn_raw_buffer_load_b8(r2, ok ? b : kOOB, 0, 0);
      ch.c1v[i] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(r1, ok ? 4 * (b >> 8) : kOOB, 0, 0));
    }
  };
  Chunk ca, cb;
  load_chunk(0, ca);
  __builtin_amdgcn_sched_barrier(0);

  // ---- LoRA term operands, one 16x16x32 MFMA per wave: wave w covers ranks
  // 16 w .. 16 w + 15 (lane groups 0 and 1; groups 2 and 3 contribute zeros).
  u32x4 lt, ll;
  {
    const __amdgpu_buffer_rsrc_t rl = rsrc(L2, 2 * ((uint64_t)(r - 1) * ld + N));
    const __amdgpu_buffer_rsrc_t rt = rsrc(T, 2 * (uint64_t)M * r);
    const int rb = 16 * w + 8 * g;        // first rank of this lane's eight
    uint32_t vl[8], vt[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const bool rk = g < 2 && rb + j < r;
      const uint32_t ol = (rk && row_ok) ? (uint32_t)(2 * ((int64_t)(rb + j) * ld + nrow)) : kOOB;
      const uint32_t ot = (rk && m_ok) ? (uint32_t)(2 * (col * r + rb + j)) : kOOB;
      vl[j] = __builtin_amdgcn_raw_buffer_load_b16(rl, ol, 0, 0);
      vt[j] = __builtin_amdgcn_raw_buffer_load_b16(rt, ot, 0, 0);
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      ll[j] = vl[2 * j] | (vl[2 * j + 1] << 16);
      lt[j] = vt[2 * j] | (vt[2 * j + 1] << 16);
    }
  }

  if (kXLds) {
#pragma unroll
    for (int j = 0; j < kXPer; ++j) {
      const uint32_t o = 16u * (uint32_t)(t + j * kThreads);
      const u32x4 v = xr[j];
      u32x4 e;
      e[0] = __builtin_amdgcn_perm(v[1], v[0], 0x05040100u);
      e[1] = __builtin_amdgcn_perm(v[3], v[2], 0x05040100u);
      e[2] = __builtin_amdgcn_perm(v[1], v[0], 0x07060302u);
      e[3] = __builtin_amdgcn_perm(v[3], v[2], 0x07060302u);
      if (o < xbytes) *(LDS_AS u32x4*)(xl + o) = e;
    }
    if (t < kZeroBytes / 16) *(LDS_AS u32x4*)(xl + kXBytes + 16 * t) = u32x4{0, 0, 0, 0};
    __syncthreads();
  }

  f32x4 acc = {0, 0, 0, 0};
  auto compute_chunk = [&](uint32_t i0, const Chunk& ch) {
#pragma unroll
    for (int i = 0; i < kChunk; ++i) {
      if (i0 + i >= nst) break;                  // uniform
      const uint32_t kb = kb0 + (i0 + i) * kbstep;
      const bool xok = m_ok && kb < kblocks;      // the lane's row of X (independent of its weight row)
      const BlockLut L = make_lut(qk::e4m3fn_to_f32(ch.c2b[i]) * ch.c1v[i], p);
      if (kXLds) {
        // X'[col][64 kb .. +64] (eight 16-byte groups), zeros for idle lanes
        const LDS_AS u32x4* xs =
            (const LDS_AS u32x4*)(xl + (xok ? ((uint32_t)col * (uint32_t)K + 64u * kb) * 2u : (uint32_t)kXBytes));
#pragma unroll
        for (int d = 0; d < 8; ++d) {
          const u32x4 bv = dequant8_eo(L, ch.cw[i][d >> 2][d & 3]);
          acc = mfma16(__builtin_bit_cast(bf16x8, xs[d]), __builtin_bit_cast(bf16x8, bv), acc);
        }
      } else {
        const uint32_t xo = xok ? (uint32_t)((col * K) * 2) + 128u * kb : kOOB;
        u32x4 a[8];
#pragma unroll
        for (int d = 0; d < 8; ++d) a[d] = __builtin_amdgcn_raw_buffer_load_b128(rx, xo + 16 * d, 0, 0);
#pragma unroll
        for (int d = 0; d < 8; ++d) {
          const u32x4 bv = dequant8(L, ch.cw[i][d >> 2][d & 3]);
          acc = mfma16(__builtin_bit_cast(bf16x8, a[d]), __builtin_bit_cast(bf16x8, bv), acc);
        }
      }
    }
  };
  // chunks in pairs: the loads of the next chunk are issued before the current
  // one is converted
  for (uint32_t i0 = 0; i0 < nst; i0 += 2 * kChunk) {
    if (i0 + kChunk < nst) load_chunk(i0 + kChunk, cb);
    compute_chunk(i0, ca);
    if (i0 + kChunk >= nst) break;
    if (i0 + 2 * kChunk < nst) load_chunk(i0 + 2 * kChunk, ca);
    compute_chunk(i0 + kChunk, cb);
  }

  {
    f32x4 zl = {0, 0, 0, 0};
    zl = mfma16(__builtin_bit_cast(bf16x8, lt), __builtin_bit_cast(bf16x8, ll), zl);
    acc += scale * zl;
  }
  f32x4* red = (f32x4*)(lds + (kXLds ? kXBytes + kZeroBytes : 0));
  red[w * 64 + l] = acc;
  __syncthreads();
  if (w == 0) {
    f32x4 sum = red[l];
#pragma unroll
    for (int ww = 1; ww < kWaves; ++ww) sum += red[ww * 64 + l];
    // lane l holds C[m = 4g + i][n = col]
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int m = 4 * g + i;
      if (m < M && row_ok) Y[(int64_t)m * ld + nrow] = qk::f32_to_bf16(sum[i]);
    }
  }
}

}  // namespace

hipError_t launch_qgemv_fwd(const uint16_t* X, int64_t M, int64_t K, int64_t N, const uint8_t* codes,
                            const uint8_t* c2, const float* c1, const uint16_t* T, const uint16_t* L2, int r,
                            float scale, uint16_t* Y, hipStream_t s) {
  // Buffer offsets are 32-bit: split the rows into chunks whose packed codes stay
  // below 2^31 bytes; chunks start on multiples of 256 rows, so every chunk's
  // blocks start a new double-quantisation group.
  const int64_t kblocks = K / qk::kBlock;
  if (M * K * 2 >= (int64_t(1) << 31)) return hipErrorInvalidValue;
  int64_t chunk = ((int64_t(1) << 31) - (int64_t(1) << 20)) / (K / 2);
  chunk = chunk / 256 * 256;
  if (chunk < 256) return hipErrorInvalidValue;
  const bool xlds = M * K * 2 <= kXBytes;
  for (int64_t r0 = 0; r0 < N; r0 += chunk) {
    const int64_t rows = N - r0 < chunk ? N - r0 : chunk;
    dim3 grid((unsigned)((rows + kRows - 1) / kRows));
    if (xlds)
      hipLaunchKernelGGL(k_qgemv_fwd<true>, grid, dim3(kThreads), 0, s, X, M, K, rows, N, codes + r0 * (K / 2),
                         c2 + r0 * kblocks, c1 + r0 * kblocks / 256, T, L2 + r0, r, scale, Y + r0, nf4_params());
    else
      hipLaunchKernelGGL(k_qgemv_fwd<false>, grid, dim3(kThreads), 0, s, X, M, K, rows, N, codes + r0 * (K / 2),
                         c2 + r0 * kblocks, c1 + r0 * kblocks / 256, T, L2 + r0, r, scale, Y + r0, nf4_params());
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}
