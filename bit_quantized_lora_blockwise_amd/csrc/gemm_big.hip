// Quantised GEMMs of the layer for training-sized M:
//   forward  Y  = bf16(X W'^T + s T L2)       (C = Y,  P = N, reduction R = K)
//   backward dX = bf16(dY W' + G L1^T)        (C = dX, P = K, reduction R = N)
// Layer formula: nlp-lineage milestone page on QLoRA, "The idea", notation
// paragraph; the frozen base is dequantised on the fly (examadda page, "The
// Core Idea"; inferensys glossary, paragraph on the dequantising kernel).
//
// Tile: 256 activation rows x 256 output columns, reduction steps of 64, in
// double-buffered LDS tiles.  768 threads = twelve waves in two roles:
//  * eight consumer waves (two per SIMD) only read fragments from LDS and
//    issue MFMA 32x32x16 bf16: wave c owns rows 64 (c % 4) .. +64 and columns
//    128 (c / 4) .. +128 of the tile, 2 x 4 MFMA tiles, 128 fp32 accumulators
//    per lane;
//  * four producer waves (one per SIMD) fill the other buffers for the next
//    step: the activation tile (256 x 64 bf16) goes from global memory straight
//    into LDS (buffer loads to LDS, XOR-swizzled through the lanes' global
//    offsets so that fragment reads are free of bank conflicts), and each
//    producer lane rebuilds one first-level block (64 weights) of the weight
//    tile from the packed 4-bit stream, loaded two steps ahead.
// The roles are split because a wave's own VALU work barely overlaps its own
// MFMAs on gfx950, while MFMA and VALU instructions of different waves on one
// SIMD co-issue: separating them measured 6-13% faster than eight waves that
// each did both.  One barrier per step hands the new buffers over.
//  * Dequantisation keeps the block's 16 bf16 values W'(v) = bf16(fl32(q[v] s'))
//    in registers as two byte planes and looks each nibble up with v_perm_b32
//    (three byte selects per four nibbles and plane), so it needs no LDS reads.
//    The forward's weight tile is [column][k] bf16 (plain fragment reads); the
//    dX path (where the reduction runs across the stored rows of W) keeps it as
//    byte planes read with ds_read_b64_tr_b8, which interleaves the planes.
//  * Work groups are dispatched round-robin over the 8 XCDs; the tile order is
//    remapped so that each XCD (with its own L2) gets a contiguous run of tiles.
//  * When the tiles outnumber the CUs, the grid is persistent (one work group
//    per CU, tiles v, v + grid, ...).  Each tile starts with its LoRA term:
//    the producers stage the LoRA operands in LDS, the consumers multiply them.
//    The consumers issue no global loads and wait only for their LDS reads,
//    and their output stores go through a buffer descriptor, so a tile's
//    stores drain while the next tile's LoRA term and first steps run (the
//    memory counter a wait would block on counts stores too).
#include <type_traits>

#include "dequant.h"
#include "kernels.h"

namespace {

using namespace nf4;

constexpr int kT = 768;           // threads per work group: 8 consumer + 4 producer waves
constexpr int kTC = 512;          // consumer threads
constexpr int kBM = 256;          // activation rows per tile
constexpr int kBP = 256;          // output columns per tile
constexpr int kBR = 64;           // reduction per step
constexpr int kPF = kBR + 8;      // pitch of the forward B tile [p][r] (elements)
constexpr int kPD = kBP + 32;     // pitch of the dX B tile [r][p] (elements): 144 dwords, so the
                                  // 4 rows x 2 column halves of a 32-lane transposed read hit 64 banks
constexpr int kPlane = kBP + 32;  // dX B tile: bytes per byte-plane row (72 dwords: the 8 rows x 32 columns
                                  // of a 32-lane transposed byte read hit 64 banks)
constexpr int kBufElems = (kBP * kPF > kBR * kPD) ? kBP * kPF : kBR * kPD;
static_assert(2 * kBR * kPlane <= 2 * kBufElems, "dX byte-plane tile fits the B buffer");
constexpr int kPL = 64 + 8;       // pitch of the LoRA operand tiles [row][c]

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

// Column held in slot `s` of a dX weight tile: within each group of eight the
// slots hold columns (0, 2, 4, 6, 1, 3, 5, 7).
__device__ __forceinline__ int dx_slot_col(int s) {
  const int u = s & 7;
  return (s & ~7) + (u < 4 ? 2 * u : 2 * u - 7);
}

// dX B fragment from the byte-plane tile (plane row 2 k + {0: low, 1: high}
// bytes, kPlane bytes per row): two ds_read_b64_tr_b8, each returning for the
// lane's column the low and high bytes of four consecutive k, i.e. four bf16.
__device__ __forceinline__ bf16x8 frag_planes(const LDS_AS uint8_t* base, int k0, int col0) {
  const int l = threadIdx.x & 63;
  const int g = l >> 4, i = l & 15;
  const int row = 2 * (k0 + 8 * (g >> 1)) + (i >> 1);
  // 8-byte chunk c of each 32-byte column group G of weight row k is stored at
  // chunk c ^ (k % 4) of group G ^ ((k / 4) % 2): with 64 four-byte banks and
  // 32 lanes of 8-byte accesses served together, neither the dequantisation's
  // writes nor these reads then put two addresses on one bank.  Here
  // k % 4 = (i / 4) % 4; the first read covers rows with (k / 4) % 2 = 0 (k0 is
  // a multiple of 16), the second, eight plane rows on, those with 1: it takes
  // the other 32-byte group of the pair (col0 is a multiple of 32).
  const int chunk = (2 * (g & 1) + (i & 1)) ^ ((i >> 2) & 3);
  const LDS_AS uint8_t* p = base + row * kPlane + 8 * chunk;
  typedef int v2i __attribute__((ext_vector_type(2)));
  const v2i a = __builtin_amdgcn_ds_read_tr8_b64_v2i32((LDS_AS v2i*)(p + col0));
  const v2i b = __builtin_amdgcn_ds_read_tr8_b64_v2i32((LDS_AS v2i*)(p + 8 * kPlane + (col0 ^ 32)));
  const u32x4 v = {(uint32_t)a[0], (uint32_t)a[1], (uint32_t)b[0], (uint32_t)b[1]};
  return __builtin_bit_cast(bf16x8, v);
}

// What a producer lane loads for one step of the packed weight: a block's 32
// bytes of codes with its scale byte and group scale (the bf16 weight goes
// straight to LDS and needs none).
struct BlockCodes {
  u32x4 v[2];
  uint32_t c2b;
  float c1v;
};
struct NoCodes {};

// bf16 dX weight tile [64 rows of W][256 columns], rows of 512 bytes: 16-byte
// chunk c of row k is kept in slot c ^ (4 (k % 4)), so that the 4 rows x 64
// bytes that 32 lanes of a transposed read touch fall on distinct banks.
__device__ __forceinline__ bf16x8 frag_kmajor_sw(const LDS_AS uint16_t* base, int k0, int col0) {
  const int l = threadIdx.x & 63;
  const int G = l >> 4, i = l & 15;
  const int row = k0 + ((G >> 1) << 3) + (i >> 2);
  const int col = col0 + ((G & 1) << 4) + ((i & 3) << 2);
  const int off = row * 512 + 16 * ((col >> 3) ^ (4 * (row & 3))) + 2 * (col & 7);
  const LDS_AS char* pb = (const LDS_AS char*)base + off;
  i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS_AS i16x4*)pb);
  i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS_AS i16x4*)(pb + 4 * 512));
  u32x2 a = __builtin_bit_cast(u32x2, lo), b = __builtin_bit_cast(u32x2, hi);
  u32x4 v = {a[0], a[1], b[0], b[1]};
  return __builtin_bit_cast(bf16x8, v);
}

// kTail: dX with N not a multiple of 64 (the last step masks activation
// columns past N).
// kB16: the same kernel with a bf16 weight W [N, K] in place of the packed 4-bit
// one (LoRA over a bf16 base, and the dequantise-then-GEMM strategy that gives
// it the dequantised W'): the producers send the forward's weight tile from
// global memory straight into LDS like the activation tile (same layout and
// swizzle), or stage the dX weight tile [64 rows of W][256 columns] through
// registers into a padded LDS tile that the consumers read with the transposing
// LDS read.  No dequantisation.
template <bool kDx, bool kTail, bool kB16 = false>
__global__ __launch_bounds__(kT, 1) void k_qgemm_big(const uint16_t* __restrict__ A, int64_t M, int64_t K,
                                                     int64_t N, const uint8_t* __restrict__ codes,
                                                     const uint8_t* __restrict__ c2,
                                                     const float* __restrict__ c1,
                                                     const uint16_t* __restrict__ LA,   // T (fwd) / G (dX)
                                                     const uint16_t* __restrict__ LB,   // L2 (fwd) / L1 (dX)
                                                     int r, float scale, uint16_t* __restrict__ C,
                                                     Nf4Params p, int nseg, int64_t seg,
                                                     const uint16_t* __restrict__ Wb) {
  __shared__ __attribute__((aligned(16))) uint16_t lds_b[2 * kBufElems];   // weight tiles; LoRA operands first
  __shared__ __attribute__((aligned(16))) uint16_t lds_a0[kBM * kBR];      // activation tiles (two buffers,
  __shared__ __attribute__((aligned(16))) uint16_t lds_a1[kBM * kBR];      //  filled by buffer-to-LDS loads)
  const int t = threadIdx.x;
  const int w = __builtin_amdgcn_readfirstlane(t >> 6), l = t & 63;
  const bool producer = w >= 8;           // uniform per wave
  const int rg = w & 3, ch = (w >> 2) & 1;  // consumers: row group (64 rows), column half (128 columns)
  const int64_t P = kDx ? K : N;          // output columns
  const int64_t R = kDx ? N : K;          // reduction length
  const int64_t kblocks = K / qk::kBlock;
  constexpr bool kPerm = kDx && !kB16;    // dX columns in the lookup order (0, 2, 4, 6, 1, 3, 5, 7)

  // ---- tiles: virtual work group v of the ntiles (one per tile) sits on XCD
  // v % 8, and XCD x takes a contiguous run of tiles in row-major tile order.
  // The launch has ntiles work groups (one tile each) or a multiple of 8 that
  // take tiles v, v + G, ... in turn (persistent).
  const int tiles_x = (int)((P + kBP - 1) / kBP);
  const int ntiles = tiles_x * (int)((M + kBM - 1) / kBM);
  const int vfirst = blockIdx.x + gridDim.x * blockIdx.y;
  const int vstride = gridDim.x * gridDim.y;
  int m0 = 0, p0 = 0;   // wave-uniform
  auto set_tile = [&](int v) {
    const int per = ntiles / 8, extra = ntiles % 8, xcd = v % 8, q = v / 8;
    const int tile = xcd < extra ? xcd * (per + 1) + q : extra * (per + 1) + (xcd - extra) * per + q;
    m0 = __builtin_amdgcn_readfirstlane((tile / tiles_x) * kBM);
    p0 = __builtin_amdgcn_readfirstlane((tile % tiles_x) * kBP);
  };
  const int ng = kDx ? nseg : 1;
  LDS_AS uint16_t* la = (LDS_AS uint16_t*)lds_b;                 // [256][kPL]: T / G rows
  LDS_AS uint16_t* lb = (LDS_AS uint16_t*)lds_b + kBM * kPL;     // fwd: L2 [64][kPD]; dX: L1 [256][kPL]

  LDS_AS uint16_t* b0 = (LDS_AS uint16_t*)lds_b;
  LDS_AS uint16_t* b1 = (LDS_AS uint16_t*)lds_b + kBufElems;
  LDS_AS uint16_t* a0 = (LDS_AS uint16_t*)lds_a0;
  LDS_AS uint16_t* a1 = (LDS_AS uint16_t*)lds_a1;
  const int64_t nsteps = (R + kBR - 1) / kBR;

  if (producer) {
    // ================================ producers ================================
    // At the top of step st the consumers multiply tiles st; the producers send
    // activation tile st + 1 (and, bf16 forward, weight tile st + 1) into the
    // other buffers, issue the loads for step st + 2, rebuild weight tile st + 1
    // from the codes loaded during the step before, and wait for all of it
    // before the barrier that ends the step.
    const int pw = w - 8;                 // producer wave 0..3
    const int tp = t - kTC;               // producer thread 0..255
    const SplitConst kc = split_const();

    // Activation (and bf16 forward weight) tiles: producer wave pw sends rows
    // 64 pw .. +64, eight rows of 128 bytes per 16-byte-per-lane load (lane l:
    // row + l / 8, written at LDS base + 16 l).  In LDS, row rho keeps its
    // 16-byte chunk c in slot c ^ ((rho >> 1) & 7): the lane loads chunk
    // (l % 8) ^ (that swizzle).
    uint32_t achunk[2], arow_off[8];
    achunk[0] = (uint32_t)((l & 7) ^ (l >> 4));     // rows with (rho >> 1) & 7 = l / 16
    achunk[1] = achunk[0] ^ 4u;                     // rows with (rho >> 1) & 7 = 4 + l / 16
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int row = 64 * pw + 8 * j + (l >> 3);
      arow_off[j] = (uint32_t)((int64_t)row * R * 2) + 16u * achunk[j & 1];
    }
    // Step st of a matrix with `rows` rows from row r0 goes through a descriptor
    // based at column 64 st of row r0 whose size ends at the end of the matrix:
    // rows past the end read as zeros, and a step past the reduction has size 0.
    // The loads are issued from inline assembly, which writes no register: the
    // compiler's own wait counting only over-waits around it, and it does not
    // make LDS reads wait for these loads (the builtin does, as it cannot tell
    // the buffers apart); the wait before each barrier covers them.
    auto dma_tile = [&](const uint16_t* src, int64_t rows, int64_t r0, int64_t st, LDS_AS uint16_t* buf) {
      const int64_t left = R - st * kBR;
      const int rem = __builtin_amdgcn_readfirstlane((int)(left < kBR ? left : kBR));   // columns in this step
      const uint64_t nrec = rem > 0 ? (uint64_t)(rows - r0) * R * 2 - (uint64_t)st * kBR * 2 : 0;
      const uint64_t base = (uint64_t)(uintptr_t)(src + r0 * R + (rem > 0 ? st * kBR : 0));
      const uint16_t* pa = (const uint16_t*)(((uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((int)(base >> 32)) << 32) |
                                             (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)base));
      const __amdgpu_buffer_rsrc_t ra = rsrc(pa, (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)nrec));
      const bool ok0 = !kTail || 8 * (int)achunk[0] < rem;    // chunks past the reduction read as zeros
      const bool ok1 = !kTail || 8 * (int)achunk[1] < rem;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const uint32_t dst = (uint32_t)(uintptr_t)(buf + (64 * pw + 8 * j) * kBR);
        const uint32_t vo = ((j & 1) ? ok1 : ok0) ? arow_off[j] : kOOB;
        // M0 (the LDS address, read when the load issues) is saved and restored
        // here, since the compiler does not track it across inline assembly
        uint32_t m0_saved;
        asm volatile(
            "s_mov_b32 %0, m0\n\ts_mov_b32 m0, %1\n\tbuffer_load_dwordx4 %2, %3, 0 offen lds\n\ts_mov_b32 m0, %0"
            : "=&s"(m0_saved)
            : "s"(__builtin_amdgcn_readfirstlane(dst)), "v"(vo), "s"(ra)
            : "memory");
      }
    };

    // Weight tiles.  Producer thread tp rebuilds one block per step:
    //  fwd: weight row p0 + tp, block st;                   tile [tp][k]
    //  dX : weight row 64 st + tp / 4, block p0 / 64 + tp % 4; byte-plane rows 2 (tp / 4) (+1)
    using Stage = typename std::conditional<kB16, NoCodes, BlockCodes>::type;
    const __amdgpu_buffer_rsrc_t rc = rsrc(codes, kB16 ? 0 : (uint64_t)N * (K / 2));
    const __amdgpu_buffer_rsrc_t r2 = rsrc(c2, kB16 ? 0 : (uint64_t)N * kblocks);
    const __amdgpu_buffer_rsrc_t r1 = rsrc(c1, kB16 ? 0 : 4 * (((uint64_t)N * kblocks + 255) / 256));
    auto load_stage = [&](int64_t step) {
      Stage h;
      if constexpr (!kB16) {
        int64_t wrow, kb;
        if (!kDx) { wrow = p0 + tp; kb = step; }
        else { wrow = step * kBR + (tp >> 2); kb = p0 / 64 + (tp & 3); }
        // out-of-range blocks get bit 31 set in their offsets: past every buffer end
        const uint32_t oob = (wrow < N && kb < kblocks) ? 0u : kOOB;
        const uint32_t b = (uint32_t)(wrow * kblocks + kb);
        const uint32_t co = (uint32_t)(wrow * (K / 2) + kb * 32) | oob;
        h.v[0] = __builtin_amdgcn_raw_buffer_load_b128(rc, co, 0, 0);
        h.v[1] = __builtin_amdgcn_raw_buffer_load_b128(rc, co + 16, 0, 0);
        h.c2b = __builtin_amdgcn_raw_buffer_load_b8(r2, b | oob, 0, 0);
        h.c1v = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(r1, (4 * (b >> 8)) | oob, 0, 0));
      }
      return h;
    };
    auto store_stage = [&](const Stage& h, LDS_AS uint16_t* buf) {
      if constexpr (!kB16) {
        const BlockLut L = make_lut(qk::e4m3fn_to_f32(h.c2b) * h.c1v, p);
#pragma unroll
        for (int q8 = 0; q8 < 8; ++q8) {
          const uint32_t c = h.v[q8 >> 2][q8 & 3];
          if (kDx) {
            u32x2 lo8, hi8;
            dequant8_planes(L, c, kc, lo8, hi8);
            // 8-byte chunk c of 32-byte column group G of weight row k at chunk
            // c ^ (k % 4) of group G ^ ((k / 4) % 2): rows k and k + 4 of a wave's
            // writes then fall on different banks
            const int k = tp >> 2, j = tp & 3;
            LDS_AS uint8_t* d = (LDS_AS uint8_t*)buf + 2 * k * kPlane + 32 * ((2 * j + (q8 >> 2)) ^ ((k >> 2) & 1)) +
                                8 * ((q8 & 3) ^ (k & 3));
            *(LDS_AS u32x2*)d = lo8;
            *(LDS_AS u32x2*)(d + kPlane) = hi8;
          } else {
            *(LDS_AS u32x4*)(buf + tp * kPF + 8 * q8) = dequant8(L, c, kc);
          }
        }
      }
    };
    // bf16 dX: weight rows 64 st .. +64, columns p0 .. p0 + 255, sent straight
    // to LDS: producer wave pw's load j fills rows 16 pw + 2 j (+1), lane l row
    // (l / 32), slot l % 32, fetching chunk (l % 32) ^ (4 (row % 4)); chunks past
    // column K and rows past N read as zeros.
    auto dma_wdx = [&](int64_t st, LDS_AS uint16_t* buf) {
      const int64_t r0 = st * kBR;
      const uint64_t nrec = r0 < N ? (uint64_t)(N - r0) * K * 2 - (uint64_t)p0 * 2 : 0;
      const uint64_t base = (uint64_t)(uintptr_t)(Wb + (r0 < N ? r0 * K + p0 : 0));
      const uint16_t* pa = (const uint16_t*)(((uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((int)(base >> 32)) << 32) |
                                             (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)base));
      const __amdgpu_buffer_rsrc_t ra = rsrc(pa, (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)nrec));
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int row = 16 * pw + 2 * j + (l >> 5);
        const int chunk = (l & 31) ^ (4 * (row & 3));
        const bool ok = p0 + 8 * chunk < K;
        const uint32_t vo = ok ? (uint32_t)(row * K * 2 + 16 * chunk) : kOOB;
        const uint32_t dst = (uint32_t)(uintptr_t)(buf + (16 * pw + 2 * j) * 256);
        uint32_t m0_saved;
        asm volatile(
            "s_mov_b32 %0, m0\n\ts_mov_b32 m0, %1\n\tbuffer_load_dwordx4 %2, %3, 0 offen lds\n\ts_mov_b32 m0, %0"
            : "=&s"(m0_saved)
            : "s"(__builtin_amdgcn_readfirstlane(dst)), "v"(vo), "s"(ra)
            : "memory");
      }
    };
    auto send = [&](int64_t st, LDS_AS uint16_t* abuf, LDS_AS uint16_t* bbuf) {
      dma_tile(A, M, m0, st, abuf);
      if constexpr (kB16 && !kDx) dma_tile(Wb, N, p0, st, bbuf);
      if constexpr (kB16 && kDx) dma_wdx(st, bbuf);
    };
    // LoRA operands of the tile into the B buffers (free: the consumers passed
    // the barrier after their last fragment reads of the previous tile), one
    // segment at a time; the consumers multiply them between the two barriers
    // that follow.  With 16-byte-aligned rows (r % 8 == 0, and in the forward
    // seg % 8 == 0) each thread moves its sixteen 16-byte chunks by buffer
    // loads, chunks past the matrices reading as zeros, all issued before the
    // first is written to LDS.
    const bool lora_vec = (r % 8) == 0 && (kDx || (seg % 8) == 0) && M * r * 2 < (int64_t(1) << 31) &&
                          (kDx ? K * r * 2 : r * seg * 2) < (int64_t(1) << 31);
    for (int v = vfirst; v < ntiles; v += vstride) {
    set_tile(v);
    Stage hA, hB, h0;
    for (int g = 0; g < ng; ++g) {
      const int64_t gs = kDx ? g : p0 / seg;
      const uint16_t* la_src = LA + gs * M * r;
      if (lora_vec) {
        u32x4 va[8], vb[8];
        const __amdgpu_buffer_rsrc_t rla = rsrc(la_src, (uint64_t)M * r * 2);
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const int idx = tp + 256 * i, row = idx >> 3, cc = (idx & 7) * 8;
          const bool ok = m0 + row < M && cc < r;
          va[i] = __builtin_amdgcn_raw_buffer_load_b128(rla, ok ? (uint32_t)(((m0 + row) * r + cc) * 2) : kOOB, 0, 0);
        }
        if constexpr (!kDx) {
          const uint16_t* lb_src = LB + gs * r * seg;
          const int pc = p0 - (int)(gs * seg);
          const __amdgpu_buffer_rsrc_t rlb = rsrc(lb_src, (uint64_t)r * seg * 2);
#pragma unroll
          for (int i = 0; i < 8; ++i) {
            const int idx = tp + 256 * i, c = idx >> 5, pp = (idx & 31) * 8;
            const bool ok = c < r && pc + pp < seg;
            vb[i] = __builtin_amdgcn_raw_buffer_load_b128(rlb, ok ? (uint32_t)(((int64_t)c * seg + pc + pp) * 2) : kOOB,
                                                          0, 0);
          }
#pragma unroll
          for (int i = 0; i < 8; ++i) {
            const int idx = tp + 256 * i;
            *(LDS_AS u32x4*)(la + (idx >> 3) * kPL + (idx & 7) * 8) = va[i];
            *(LDS_AS u32x4*)(lb + (idx >> 5) * kPD + (idx & 31) * 8) = vb[i];
          }
        } else {
          const uint16_t* lb_src = LB + gs * K * r;
          const __amdgpu_buffer_rsrc_t rlb = rsrc(lb_src, (uint64_t)K * r * 2);
#pragma unroll
          for (int i = 0; i < 8; ++i) {
            const int idx = tp + 256 * i, row = idx >> 3, cc = (idx & 7) * 8;
            const bool ok = p0 + row < K && cc < r;
            vb[i] = __builtin_amdgcn_raw_buffer_load_b128(rlb, ok ? (uint32_t)(((int64_t)(p0 + row) * r + cc) * 2) : kOOB,
                                                          0, 0);
          }
#pragma unroll
          for (int i = 0; i < 8; ++i) {
            const int idx = tp + 256 * i;
            *(LDS_AS u32x4*)(la + (idx >> 3) * kPL + (idx & 7) * 8) = va[i];
            *(LDS_AS u32x4*)(lb + (idx >> 3) * kPL + (idx & 7) * 8) = vb[i];
          }
        }
      } else {
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int idx = tp + 256 * i, row = idx >> 3, cc = (idx & 7) * 8;
        u32x4 v8 = {0, 0, 0, 0};
        if (m0 + row < M) v8 = load_row8(la_src + (m0 + row) * r, cc, r);
        *(LDS_AS u32x4*)(la + row * kPL + cc) = v8;
      }
      if constexpr (!kDx) {
        const uint16_t* lb_src = LB + gs * r * seg;
        const int64_t pc = p0 - gs * seg;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const int idx = tp + 256 * i, c = idx >> 5, pp = (idx & 31) * 8;
          u32x4 v8 = {0, 0, 0, 0};
          if (c < r) v8 = load_row8(lb_src + (int64_t)c * seg, pc + pp, seg);
          *(LDS_AS u32x4*)(lb + c * kPD + pp) = v8;
        }
      } else {
        const uint16_t* lb_src = LB + gs * K * r;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const int idx = tp + 256 * i, row = idx >> 3, cc = (idx & 7) * 8;
          u32x4 v8 = {0, 0, 0, 0};
          if (p0 + row < K) v8 = load_row8(lb_src + (p0 + row) * r, cc, r);
          *(LDS_AS u32x4*)(lb + row * kPL + cc) = v8;
        }
      }
      }
      __builtin_amdgcn_s_waitcnt(0x0070);   // vmcnt(0) lgkmcnt(0): this wave's loads and LDS writes
      __builtin_amdgcn_s_barrier();
      __builtin_amdgcn_s_barrier();         // the consumers have read them
    }
    {
      send(0, a0, b0);
      h0 = load_stage(0);
      hA = load_stage(1);
      store_stage(h0, b0);
      __builtin_amdgcn_s_waitcnt(0x0070);   // vmcnt(0) lgkmcnt(0), seen by the compiler's wait tracking
      __builtin_amdgcn_s_barrier();
    }
    // Steps in pairs with no exit between them, so that the loop body is one
    // basic block and the early loads stay where they are issued; an odd step
    // count runs one more step over zeros (codes and activations past the end).
    // The wait at the top of a step finds everything issued in the step before
    // arrived (the barrier waited for it) and tells the compiler's wait
    // tracking so, so that it places no wait after the loads to LDS it cannot
    // count.
    for (int64_t st = 0; st < nsteps; st += 2) {
      __builtin_amdgcn_s_waitcnt(0x0070);
      send(st + 1, a1, b1);
      hB = load_stage(st + 2);
      __builtin_amdgcn_sched_barrier(0);
      store_stage(hA, b1);
      __builtin_amdgcn_sched_barrier(0);
      __builtin_amdgcn_s_waitcnt(0x0070);
      __builtin_amdgcn_s_barrier();
      __builtin_amdgcn_s_waitcnt(0x0070);
      send(st + 2, a0, b0);
      hA = load_stage(st + 3);
      __builtin_amdgcn_sched_barrier(0);
      store_stage(hB, b0);
      __builtin_amdgcn_sched_barrier(0);
      __builtin_amdgcn_s_waitcnt(0x0070);
      __builtin_amdgcn_s_barrier();
    }
    }   // tiles
    return;
  }

  // ================================ consumers ================================
  // They issue no loads: between barriers they only read LDS and store their
  // outputs, and they wait only for their LDS reads, so one tile's output
  // stores drain while the next tile's LoRA term and first steps run.
  f32x16 acc[2][4];
  // A fragment of sub-step s, tile i: row 64 (c % 4) + 32 i + l % 32, chunk 2 s + l / 32.
  uint32_t afrag_off[4];
#pragma unroll
  for (int s = 0; s < 4; ++s)
    afrag_off[s] = (uint32_t)((64 * rg + (l & 31)) * kBR * 2 + 16 * ((2 * s + (l >> 5)) ^ ((l >> 1) & 7)));
  auto afrag = [&](const LDS_AS uint16_t* abuf, int s, int i) {
    return *(const LDS_AS bf16x8*)((const LDS_AS char*)abuf + afrag_off[s] + 32 * kBR * 2 * i);
  };
  // B fragment of sub-step s, column tile j (columns 128 (c / 4) + 32 j ..)
  auto bfrag = [&](const LDS_AS uint16_t* bcur, int s, int j) {
    if constexpr (kB16) {
      if constexpr (kDx) return frag_kmajor_sw(bcur, 16 * s, 128 * ch + 32 * j);
      else   // the [p][k] tile sent like the activations, addressed like the A fragments
        return *(const LDS_AS bf16x8*)((const LDS_AS char*)bcur + afrag_off[s] - (64 * rg) * kBR * 2 +
                                       (128 * ch + 32 * j) * kBR * 2);
    } else {
      return kDx ? frag_planes((const LDS_AS uint8_t*)bcur, 16 * s, 128 * ch + 32 * j)
                 : qk::frag_rowmajor(bcur, kPF, 128 * ch + 32 * j, 16 * s);
    }
  };
  // Fragments of sub-step s + 1 are read from LDS while sub-step s multiplies.
  auto compute = [&](const LDS_AS uint16_t* acur, const LDS_AS uint16_t* bcur) {
    bf16x8 bq[2][4], aq[2][2];
#pragma unroll
    for (int j = 0; j < 4; ++j) bq[0][j] = bfrag(bcur, 0, j);
    aq[0][0] = afrag(acur, 0, 0);
    aq[0][1] = afrag(acur, 0, 1);
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      if (s < 3) {
#pragma unroll
        for (int j = 0; j < 4; ++j) bq[(s + 1) & 1][j] = bfrag(bcur, s + 1, j);
        aq[(s + 1) & 1][0] = afrag(acur, s + 1, 0);
        aq[(s + 1) & 1][1] = afrag(acur, s + 1, 1);
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        acc[0][j] = qk::mfma32(aq[s & 1][0], bq[s & 1][j], acc[0][j]);
        acc[1][j] = qk::mfma32(aq[s & 1][1], bq[s & 1][j], acc[1][j]);
      }
    }
  };
  for (int v = vfirst; v < ntiles; v += vstride) {
  set_tile(v);
  // ---- LoRA term first: fwd acc = s * (T L2); dX acc = G L1^T (rank
  //      zero-padded to 64); the base product then accumulates onto it.  With
  //      nseg > 1 segments (stacked linears) the forward tile uses its own
  //      segment's pair (tiles never straddle segments), the dX tile sums the
  //      products of all segments.
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x16{};
  for (int g = 0; g < ng; ++g) {
    __builtin_amdgcn_s_barrier();          // the producers' LoRA operands are in LDS
    const int ksteps = (r + 15) / 16;
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      if (s < ksteps) {
        const bf16x8 a0f = qk::frag_rowmajor(la, kPL, 64 * rg, 16 * s);
        const bf16x8 a1f = qk::frag_rowmajor(la, kPL, 64 * rg + 32, 16 * s);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          // dX: the column of accumulator slot (l % 32) is dx_slot_col(l % 32)
          const bf16x8 b =
              kDx ? *(const LDS_AS bf16x8*)(lb + (128 * ch + 32 * j + (kPerm ? dx_slot_col(l & 31) : (l & 31))) *
                                                     kPL + 16 * s + 8 * (l >> 5))
                  : qk::frag_kmajor(lb, kPD, 16 * s, 128 * ch + 32 * j);
          acc[0][j] = qk::mfma32(a0f, b, acc[0][j]);
          acc[1][j] = qk::mfma32(a1f, b, acc[1][j]);
        }
      }
    }
    __builtin_amdgcn_s_waitcnt(0xC07F);    // lgkmcnt(0): this wave's reads of the LoRA operands are done
    __builtin_amdgcn_s_barrier();
  }
  if constexpr (!kDx) {
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[i][j] = scale * acc[i][j];
  }
  __builtin_amdgcn_s_barrier();            // first tiles in LDS
  for (int64_t st = 0; st < nsteps; st += 2) {
    compute(a0, b0);
    __builtin_amdgcn_s_waitcnt(0xC07F);    // lgkmcnt(0): this wave's fragment reads are done
    __builtin_amdgcn_s_barrier();
    compute(a1, b1);
    __builtin_amdgcn_s_waitcnt(0xC07F);
    __builtin_amdgcn_s_barrier();
  }

  // ---- store C (bf16), lane layout of the 32x32 accumulators, through a
  // buffer descriptor based at this wave's first output element whose size
  // ends with the last row of C (rows past M are dropped by the hardware);
  // lane offsets are 32-bit (M P < 2^30), the (i, j) part a scalar offset.
  {
    const int Pi = (int)P;
    const int rows_left = (int)M - (m0 + 64 * rg);
    const int cbase = p0 + 128 * ch;
    const uint32_t nbytes = rows_left > 0 ? (uint32_t)(rows_left * Pi - cbase) * 2u : 0u;
    const __amdgpu_buffer_rsrc_t rc_out = rsrc(C + (int64_t)(m0 + 64 * rg) * P + cbase, nbytes);
    const int col = kPerm ? dx_slot_col(l & 31) : (l & 31);
    const int prem = Pi - (cbase + col);           // columns of this lane still inside C
    const uint32_t lane_b = (uint32_t)((4 * (l >> 5)) * Pi + col) * 2u;   // acc_row(e) = 8 (e / 4) + 4 (l / 32) + e % 4
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        if (32 * j < prem) {
#pragma unroll
          for (int e = 0; e < 16; ++e) {
            const int so = ((32 * i + 8 * (e >> 2) + (e & 3)) * Pi + 32 * j) * 2;
            __builtin_amdgcn_raw_buffer_store_b16(qk::f32_to_bf16(acc[i][j][e]), rc_out, lane_b, so, 0);
          }
        }
      }
  }
  }   // tiles
}

}  // namespace

bool qgemm_big_ok(bool dx, int64_t M, int64_t K, int64_t N) {
  // 32-bit buffer offsets; 16-byte aligned activation rows (R % 8 == 0)
  const int64_t R = dx ? N : K;
  return (R % 8) == 0 && M * R * 2 < (int64_t(1) << 31) && N * (K / 2) < (int64_t(1) << 31) && M > 16;
}

// Launch grid: one work group per tile, or, when the tiles outnumber the CUs,
// a persistent grid of the CU count rounded down to a multiple of 8 (each
// work group then takes tiles v, v + grid, ... on one XCD), so that a work
// group's output stores drain while its next tile starts.
static dim3 tile_grid(int64_t M, int64_t P) {
  static const int cus = [] {
    int dev = 0, n = 0;
    if (hipGetDevice(&dev) != hipSuccess || hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) !=
                                                hipSuccess || n < 8)
      n = 256;
    return n;
  }();
  const int64_t tx = (P + kBP - 1) / kBP, ty = (M + kBM - 1) / kBM;
  const int64_t pers = cus / 8 * 8;
  if (tx * ty > pers) return dim3((unsigned)pers, 1);
  return dim3((unsigned)tx, (unsigned)ty);
}

hipError_t launch_qgemm_big(bool dx, const uint16_t* A, int64_t M, int64_t K, int64_t N, const uint8_t* codes,
                            const uint8_t* c2, const float* c1, const uint16_t* LA, const uint16_t* LB, int r,
                            float scale, uint16_t* C, hipStream_t s, int nseg) {
  const int64_t P = dx ? K : N;
  const int64_t seg = N / nseg;   // columns of W per segment (a multiple of 256 when nseg > 1)
  const dim3 grid = tile_grid(M, P);
  const uint16_t* nw = nullptr;
  if (!dx)
    hipLaunchKernelGGL((k_qgemm_big<false, false>), grid, dim3(kT), 0, s, A, M, K, N, codes, c2, c1, LA, LB, r,
                       scale, C, nf4_params(), nseg, seg, nw);
  else if (N % kBR == 0)
    hipLaunchKernelGGL((k_qgemm_big<true, false>), grid, dim3(kT), 0, s, A, M, K, N, codes, c2, c1, LA, LB, r,
                       scale, C, nf4_params(), nseg, seg, nw);
  else
    hipLaunchKernelGGL((k_qgemm_big<true, true>), grid, dim3(kT), 0, s, A, M, K, N, codes, c2, c1, LA, LB, r,
                       scale, C, nf4_params(), nseg, seg, nw);
  return hipGetLastError();
}

bool bgemm_ok(bool dx, int64_t M, int64_t K, int64_t N) {
  // 32-bit buffer offsets into the activations and the bf16 weight; 16-byte
  // aligned rows of the activations and of W (K % 8 == 0, N % 8 == 0)
  (void)dx;
  return (K % 8) == 0 && (N % 8) == 0 && M * K * 2 < (int64_t(1) << 31) && M * N * 2 < (int64_t(1) << 31) &&
         N * K * 2 < (int64_t(1) << 31);
}

hipError_t launch_bgemm_big(bool dx, const uint16_t* A, int64_t M, int64_t K, int64_t N, const uint16_t* W,
                            const uint16_t* LA, const uint16_t* LB, int r, float scale, uint16_t* C, hipStream_t s) {
  const int64_t P = dx ? K : N;
  const dim3 grid = tile_grid(M, P);
  const uint8_t* nc = nullptr;
  const float* nf = nullptr;
  if (!dx)
    hipLaunchKernelGGL((k_qgemm_big<false, false, true>), grid, dim3(kT), 0, s, A, M, K, N, nc, nc, nf, LA, LB, r,
                       scale, C, nf4_params(), 1, N, W);
  else if (N % kBR == 0)
    hipLaunchKernelGGL((k_qgemm_big<true, false, true>), grid, dim3(kT), 0, s, A, M, K, N, nc, nc, nf, LA, LB, r,
                       scale, C, nf4_params(), 1, N, W);
  else
    hipLaunchKernelGGL((k_qgemm_big<true, true, true>), grid, dim3(kT), 0, s, A, M, K, N, nc, nc, nf, LA, LB, r,
                       scale, C, nf4_params(), 1, N, W);
  return hipGetLastError();
}
