// Decode-sized forward (M <= 16): Y = bf16(X W'^T + s T L2) as one pass over
// the packed 4-bit weight stream.  At these sizes the layer is bound by HBM
// traffic of the codes and scales, so the kernel is organised around a
// coalesced stream of 16-byte code loads, issued several steps ahead, and a
// dequantiser cheap enough in VALU to keep up with it; the bf16 weights live
// only in registers and feed a 16x16x32 bf16 MFMA against X.
// Layer formula: nlp-lineage milestone page on QLoRA, "The idea", notation
// paragraph; dequantisation on the fly: examadda page, "The Core Idea".
//
// Dequantisation: every lane owns one first-level block (64 weights) per step.
// It writes the block's 16 possible bf16 values, bf16(fl32(q[v] * s')), into a
// private LDS column (entry v at byte 256 v + 4 lane of its wave's region, so
// the 64 lanes of a lookup hit 64 distinct banks) and then replaces each
// nibble by one 16-bit LDS read.  The read address is assembled with one
// v_perm_b32 from the nibble and the lane's column offset, and a second
// v_perm_b32 packs two looked-up values into one register, so a weight costs
// about 2.5 VALU instructions and one LDS read.
#include "kernels.h"

namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / 64;
constexpr int kRows = 16;                 // weight rows (output columns) per work group
constexpr int kLutDwords = 16 * 64;       // one wave's table region: 16 entries x 64 lanes
constexpr int kStepK = 256;               // K covered by one wave step (4 lane groups x 64)
constexpr int kChunk = 4;                 // steps of a wave whose loads are issued together
constexpr int kRedDwords = kWaves * 64 * 4;
constexpr int kXDwords = 4096;            // LDS budget for X (16 KB): M * K <= 8192
constexpr int kLdsDwords = kWaves * kLutDwords + kRedDwords + kXDwords;
constexpr uint32_t kOOB = 0x80000000u;    // buffer offset past every range: the load returns 0
static_assert(kWaves * kLutDwords * 4 <= 65536, "table addresses must fit in 16 bits");

__device__ __forceinline__ f32x4 mfma16(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void* p, uint64_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc((void*)p, (short)0, (int)bytes, 0x00020000);
}

// 8 packed bf16 pairs from 16 LDS addresses: out[p] = lut[lo[p]] | lut[hi[p]] << 16.
__device__ __forceinline__ void lookup8(const uint32_t (&lo)[8], const uint32_t (&hi)[8], uint32_t (&out)[8]) {
#pragma unroll
  for (int p = 0; p < 8; ++p) {
    const uint32_t a = *(const LDS_AS uint16_t*)(uintptr_t)lo[p];
    const uint32_t b = *(const LDS_AS uint16_t*)(uintptr_t)hi[p];
    out[p] = __builtin_amdgcn_perm(b, a, 0x05040100u);
  }
}

// Work group: 16 weight rows x all of K.  Lane l of each wave handles weight row
// n0 + l % 16 and, per 256-wide step of K, the block 4 * step + l / 16; the four
// waves take the steps in turn, four at a time with all their loads in flight.
// Within a block the MFMA reduction order is the natural one: MFMA t consumes
// the lane's weights 8t .. 8t + 7 and the matching eight columns of X.  Global
// reads are buffer loads whose out-of-range lanes (rows past N, blocks past K)
// read zero, so the loop has no divergent branches.  When M * K <= 8192, X is
// staged in LDS once per work group; otherwise its fragments are loaded per step.
__global__ __launch_bounds__(kThreads) void k_qgemv_fwd(const uint16_t* __restrict__ X, int64_t M, int64_t K,
                                                        int64_t N, int64_t ld, const uint8_t* __restrict__ codes,
                                                        const uint8_t* __restrict__ c2,
                                                        const float* __restrict__ c1,
                                                        const uint16_t* __restrict__ T,
                                                        const uint16_t* __restrict__ L2, int r, float scale,
                                                        uint16_t* __restrict__ Y, Nf4Params p) {
  // One LDS object so the tables start at LDS address 0 (the lookup addresses
  // are assembled bytewise); the reduction area and the X copy follow them.
  __shared__ __attribute__((aligned(16))) uint32_t lds[kLdsDwords];
  const int t = threadIdx.x;
  const int w = t >> 6, l = t & 63;
  const int g = l >> 4, col = l & 15;
  const int64_t n0 = (int64_t)blockIdx.x * kRows;
  const int64_t nrow = n0 + col;
  const uint32_t kblocks = (uint32_t)(K / qk::kBlock);
  const uint32_t nsteps = (uint32_t)((K + kStepK - 1) / kStepK);
  const bool row_ok = nrow < N;
  const bool m_ok = col < M;                       // A-operand row of this lane is X[col]
  const bool x_in_lds = M * K <= 2 * kXDwords;
  const uint32_t lanebase = 4u * (uint32_t)l;      // byte 0 of every table address
  const uint32_t wsel = 0x01010101u * (16u * (uint32_t)w);   // byte 1 gets 16 w + nibble
  LDS_AS uint16_t* lut16 = (LDS_AS uint16_t*)((LDS_AS uint32_t*)lds + w * kLutDwords + l);
  LDS_AS uint16_t* xl = (LDS_AS uint16_t*)((LDS_AS uint32_t*)lds + kWaves * kLutDwords + kRedDwords);

  const __amdgpu_buffer_rsrc_t rc = rsrc(codes, (uint64_t)N * (K / 2));
  const __amdgpu_buffer_rsrc_t r2 = rsrc(c2, (uint64_t)N * kblocks);
  const __amdgpu_buffer_rsrc_t r1 = rsrc(c1, 4 * (((uint64_t)N * kblocks + 255) / 256));
  const __amdgpu_buffer_rsrc_t rx = rsrc(X, (uint64_t)M * K * 2);

  // 32-bit offsets (the launcher keeps every chunk below 2^31 bytes); step i of
  // this wave covers block kb0 + i * kbstep.
  const uint32_t kb0 = 4u * (uint32_t)w + (uint32_t)g;
  const uint32_t kbstep = 4u * kWaves;
  const uint32_t kb_lim = row_ok ? kblocks : 0u;   // blocks valid for this lane: kb < kb_lim
  const uint32_t code0 = (uint32_t)(nrow * (K / 2)) + 32u * kb0;
  const uint32_t blk0 = (uint32_t)(nrow * kblocks) + kb0;
  const uint32_t nst = (nsteps > (uint32_t)w) ? (nsteps - (uint32_t)w + kWaves - 1) / kWaves : 0u;

  f32x4 acc = {0, 0, 0, 0};
  u32x4 cw[kChunk][2];
  uint32_t c2b[kChunk];
  float c1v[kChunk];
  auto load_chunk = [&](uint32_t i0) {
#pragma unroll
    for (int i = 0; i < kChunk; ++i) {
      const uint32_t ii = i0 + i;
      const bool ok = (kb0 + ii * kbstep) < kb_lim;
      const uint32_t co = ok ? code0 + 32u * kbstep * ii : kOOB;
      const uint32_t b = blk0 + kbstep * ii;
      cw[i][0] = __builtin_amdgcn_raw_buffer_load_b128(rc, co, 0, 0);
      cw[i][1] = __builtin_amdgcn_raw_buffer_load_b128(rc, co + 16, 0, 0);
      c2b[i] = __builtin_amdgcn_raw_buffer_load_b8(r2, ok ? b : kOOB, 0, 0);
      c1v[i] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(r1, ok ? 4 * (b >> 8) : kOOB, 0, 0));
    }
  };
  load_chunk(0);
  // the first chunk's code loads stay the first memory operations of the wave
  __builtin_amdgcn_sched_barrier(0);

  // LoRA term, one 16x16x32 MFMA per wave: wave w covers ranks 16 w .. 16 w + 15
  // (lane groups 0 and 1; groups 2 and 3 contribute zeros).  Its operands are
  // loaded first so their latency overlaps the main loop.
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
  // X in LDS when it fits: its loads are issued before the first code loads
  // (so waiting for them never waits for the code stream) and written to LDS
  // after the code loads are in flight.
  constexpr int kXPer = kXDwords * 4 / (16 * kThreads);      // 16-byte X loads per thread
  u32x4 xr[kXPer];
  const uint32_t xbytes = x_in_lds ? (uint32_t)(M * K * 2) : 0u;
#pragma unroll
  for (int j = 0; j < kXPer; ++j) {
    const uint32_t o = 16u * (uint32_t)(t + j * kThreads);
    xr[j] = __builtin_amdgcn_raw_buffer_load_b128(rx, o < xbytes ? o : kOOB, 0, 0);
  }


  __builtin_amdgcn_sched_barrier(0);
  if (x_in_lds) {
#pragma unroll
    for (int j = 0; j < kXPer; ++j)
      *(LDS_AS u32x4*)((LDS_AS uint8_t*)xl + 16u * (uint32_t)(t + j * kThreads)) = xr[j];
    __syncthreads();
  }
  for (uint32_t i0 = 0; i0 < nst; i0 += kChunk) {
    if (i0 > 0) load_chunk(i0);
#pragma unroll
    for (int i = 0; i < kChunk; ++i) {
      const uint32_t ii = i0 + i;
      if (ii >= nst) break;
      const uint32_t kb = kb0 + ii * kbstep;
      const bool xok = m_ok && kb < kblocks;
      // X columns 64 kb .. 64 kb + 63 of row `col`
      u32x4 a[8];
      if (x_in_lds) {
        const LDS_AS u32x4* xs = (const LDS_AS u32x4*)(xl + (xok ? (uint32_t)col * (uint32_t)K + 64u * kb : 0u));
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          a[j] = xs[j];
          if (!xok) a[j] = u32x4{0, 0, 0, 0};
        }
      } else {
        const uint32_t xo = xok ? (uint32_t)((col * K) * 2) + 128u * kb : kOOB;
#pragma unroll
        for (int j = 0; j < 8; ++j) a[j] = __builtin_amdgcn_raw_buffer_load_b128(rx, xo + 16 * j, 0, 0);
      }
      const float sc = qk::e4m3fn_to_f32(c2b[i]) * c1v[i];
      // the block's 16 dequantised values into this lane's table column
#pragma unroll
      for (int v = 0; v < 16; v += 2) {
        const uint32_t pk = qk::pack_bf16x2(p.q[v] * sc, p.q[v + 1] * sc);
        lut16[(v * 64) * 2] = (uint16_t)pk;
        lut16[((v + 1) * 64) * 2] = (uint16_t)(pk >> 16);
      }
      // dequantise by lookup and multiply
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const u32x4 c4 = cw[i][h];
#pragma unroll
        for (int d = 0; d < 2; ++d) {
          uint32_t lo[8], hi[8], bw[8];
#pragma unroll
          for (int e = 0; e < 2; ++e) {
            const uint32_t c = c4[2 * d + e];
            const uint32_t xe = (c & 0x0F0F0F0Fu) | wsel;           // nibbles 0, 2, 4, 6
            const uint32_t xo = ((c >> 4) & 0x0F0F0F0Fu) | wsel;    // nibbles 1, 3, 5, 7
#pragma unroll
            for (int q4 = 0; q4 < 4; ++q4) {
              const uint32_t sel = 0x0C0C0400u | ((uint32_t)q4 << 8);
              lo[4 * e + q4] = __builtin_amdgcn_perm(xe, lanebase, sel);
              hi[4 * e + q4] = __builtin_amdgcn_perm(xo, lanebase, sel);
            }
          }
          lookup8(lo, hi, bw);
#pragma unroll
          for (int e = 0; e < 2; ++e) {
            const int j = 4 * h + 2 * d + e;   // MFMA index = code dword index within the block
            u32x4 bv = {bw[4 * e + 0], bw[4 * e + 1], bw[4 * e + 2], bw[4 * e + 3]};
            acc = mfma16(__builtin_bit_cast(bf16x8, a[j]), __builtin_bit_cast(bf16x8, bv), acc);
          }
        }
      }
    }
  }

  {
    f32x4 zl = {0, 0, 0, 0};
    zl = mfma16(__builtin_bit_cast(bf16x8, lt), __builtin_bit_cast(bf16x8, ll), zl);
    acc += scale * zl;
  }
  f32x4* red = (f32x4*)(lds + kWaves * kLutDwords);
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
  for (int64_t r0 = 0; r0 < N; r0 += chunk) {
    const int64_t rows = N - r0 < chunk ? N - r0 : chunk;
    dim3 grid((unsigned)((rows + kRows - 1) / kRows));
    hipLaunchKernelGGL(k_qgemv_fwd, grid, dim3(kThreads), 0, s, X, M, K, rows, N, codes + r0 * (K / 2),
                       c2 + r0 * kblocks, c1 + r0 * kblocks / 256, T, L2 + r0, r, scale, Y + r0, nf4_params());
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}
