// Quantised GEMMs of the layer for training-sized M:
//   forward  Y  = bf16(X W'^T + s T L2)       (C = Y,  P = N, reduction R = K)
//   backward dX = bf16(dY W' + G L1^T)        (C = dX, P = K, reduction R = N)
// Layer formula: nlp-lineage milestone page on QLoRA, "The idea", notation
// paragraph; the frozen base is dequantised on the fly (examadda page, "The
// Core Idea"; inferensys glossary, paragraph on the dequantising kernel).
//
// Tile: 256 activation rows x 256 output columns, reduction steps of 64.
// 512 threads = eight waves, two per SIMD, so that the dequantisation VALU
// work of one wave fills the gaps between the MFMAs of the other (a single
// wave barely overlaps its own VALU work with its MFMAs on gfx950).  Wave w
// owns rows 64 (w % 4) .. +64 and columns 128 (w / 4) .. +128 of the tile:
// 2 x 4 MFMA 32x32x16 tiles, 128 fp32 accumulators per lane.
//  * Activation tile of a step (256 x 64 bf16): at the start of the step
//    before, each wave sends 32 of its rows (eight rows of 128 bytes per
//    16-byte-per-lane load) from global memory straight into the other buffer
//    of a double-buffered LDS tile (buffer loads to LDS: no registers, no LDS
//    store instructions), XOR-swizzled through the lanes' global offsets so that
//    fragment reads are free of bank conflicts.  The two waves of a row group
//    both read from it.
//  * Weight tile (256 x 64): rebuilt from the packed 4-bit stream once per work
//    group; each pair of threads owns one first-level block (64 weights) and
//    each thread converts half of it per step into a double-buffered LDS tile.
//    The forward reads B fragments directly, the dX path (where the reduction
//    runs across the stored rows of W) through ds_read_b64_tr_b16.
//  * Dequantisation keeps the block's 16 bf16 values W'(v) = bf16(fl32(q[v] s'))
//    in registers as two byte planes and looks each nibble up with v_perm_b32
//    (three byte selects per four nibbles and plane), so it needs no LDS reads.
//  * Work groups are dispatched round-robin over the 8 XCDs; the tile order is
//    remapped so that each XCD (with its own L2) gets a contiguous run of tiles.
#include <type_traits>

#include "kernels.h"

namespace {

constexpr int kT = 512;           // threads per work group
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

// (a & m) | o in one instruction; m and o are kept in VGPRs (a VOP3 encoding
// takes no literal and at most one SGPR).
__device__ __forceinline__ uint32_t and_or(uint32_t a, uint32_t m, uint32_t o) {
  uint32_t r;
  asm("v_and_or_b32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(m), "v"(o));
  return r;
}

// Constants of the nibble split, held in VGPRs for v_and_or_b32.
struct SplitConst {
  uint32_t m4, b0;   // 0x04040404, 0x03020100
};

// 16-entry byte lookup of four 4-bit indices: x7 holds their low three bits,
// sel = 0x03020100 + 4 * (bit 3 of each index) picks the entry 8..15 candidate.
__device__ __forceinline__ uint32_t lut16(const uint32_t (&T)[4], uint32_t x7, uint32_t sel) {
  const uint32_t a = __builtin_amdgcn_perm(T[1], T[0], x7);   // entries 0..7
  const uint32_t b = __builtin_amdgcn_perm(T[3], T[2], x7);   // entries 8..15
  return __builtin_amdgcn_perm(b, a, sel);
}

// Eight nibbles of one 32-bit word (element j in bits 4j..4j+3): index bytes of
// the even elements (xe, se) and the odd elements (xo, so).
struct Split {
  uint32_t xe, se, xo, so;
};

__device__ __forceinline__ Split split8(uint32_t c, const SplitConst& k) {
  Split sp;
  sp.xe = c & 0x07070707u;               // elements 0, 2, 4, 6: low 3 bits
  sp.se = and_or(c >> 1, k.m4, k.b0);    //   and their bit 3 as a selector
  sp.xo = (c >> 4) & 0x07070707u;        // elements 1, 3, 5, 7
  sp.so = and_or(c >> 5, k.m4, k.b0);
  return sp;
}

// Eight nibbles -> four packed bf16 pairs in element order.
__device__ __forceinline__ u32x4 dequant8(const BlockLut& L, uint32_t c, const SplitConst& k) {
  const Split sp = split8(c, k);
  const uint32_t le = lut16(L.lo, sp.xe, sp.se), he = lut16(L.hi, sp.xe, sp.se);
  const uint32_t lo_ = lut16(L.lo, sp.xo, sp.so), ho = lut16(L.hi, sp.xo, sp.so);
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

// Eight nibbles -> the low and high bytes of their bf16 values, each as eight
// bytes in the element order (0, 2, 4, 6, 1, 3, 5, 7).
__device__ __forceinline__ void dequant8_planes(const BlockLut& L, uint32_t c, const SplitConst& k, u32x2& lo8,
                                                u32x2& hi8) {
  const Split sp = split8(c, k);
  lo8 = u32x2{lut16(L.lo, sp.xe, sp.se), lut16(L.lo, sp.xo, sp.so)};
  hi8 = u32x2{lut16(L.hi, sp.xe, sp.se), lut16(L.hi, sp.xo, sp.so)};
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
  // 8-byte chunk c of each 32-byte column group of weight row k is stored at
  // chunk c ^ (k % 4) (k % 4 = (i / 4) % 4 here), which keeps the writes of the
  // dequantisation free of bank conflicts
  const int chunk = (2 * (g & 1) + (i & 1)) ^ ((i >> 2) & 3);
  const LDS_AS uint8_t* p = base + row * kPlane + col0 + 8 * chunk;
  typedef int v2i __attribute__((ext_vector_type(2)));
  const v2i a = __builtin_amdgcn_ds_read_tr8_b64_v2i32((LDS_AS v2i*)p);
  const v2i b = __builtin_amdgcn_ds_read_tr8_b64_v2i32((LDS_AS v2i*)(p + 8 * kPlane));
  const u32x4 v = {(uint32_t)a[0], (uint32_t)a[1], (uint32_t)b[0], (uint32_t)b[1]};
  return __builtin_bit_cast(bf16x8, v);
}

// Half a block's packed codes (32 weights), its scale byte and group scale.
struct HalfCodes {
  u32x4 c;
  uint32_t c2b;
  float c1v;
};

// bf16-weight variant, dX: a thread's 64 bytes (32 columns) of one weight row.
struct RowBytes {
  u32x4 v[4];
};
struct NoStage {};

template <bool kDx, bool kB16>
using StageT = typename std::conditional<kB16, typename std::conditional<kDx, RowBytes, NoStage>::type,
                                         HalfCodes>::type;

// ---------------------------------------------------------------------------
// kTail: dX with N not a multiple of 64 (the last step masks activation
// columns past N).
// kB16: the same kernel with a bf16 weight W [N, K] in place of the packed 4-bit
// one (LoRA over a bf16 base, and the dequantise-then-GEMM strategy that gives
// it the dequantised W'): the forward's weight tile is sent from global memory
// straight into LDS like the activation tile (same layout and swizzle); the dX
// weight tile [64 rows of W][256 columns] is staged through registers into a
// padded LDS tile and read with the transposing LDS read.  No dequantisation.
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
  SplitConst kc;
  asm volatile("v_mov_b32 %0, 0x04040404" : "=v"(kc.m4));
  asm volatile("v_mov_b32 %0, 0x03020100" : "=v"(kc.b0));
  const int rg = w & 3, ch = w >> 2;      // row group (64 rows), column half (128 columns)
  const int64_t P = kDx ? K : N;          // output columns
  const int64_t R = kDx ? N : K;          // reduction length
  const int64_t kblocks = K / qk::kBlock;
  constexpr bool kPerm = kDx && !kB16;    // dX columns in the lookup order (0, 2, 4, 6, 1, 3, 5, 7)

  // ---- tile of this work group: XCD x = (linear id) % 8 takes a contiguous
  // run of tiles in row-major tile order.
  int64_t m0, p0;
  {
    const int nwg = gridDim.x * gridDim.y;
    const int b = blockIdx.x + gridDim.x * blockIdx.y;
    const int per = nwg / 8, extra = nwg % 8, xcd = b % 8, q = b / 8;
    const int tile = xcd < extra ? xcd * (per + 1) + q : extra * (per + 1) + (xcd - extra) * per + q;
    m0 = (int64_t)(tile / gridDim.x) * kBM;
    p0 = (int64_t)(tile % gridDim.x) * kBP;
  }

  f32x16 acc[2][4];

  // ---- LoRA term first: fwd acc = s * (T L2); dX acc = G L1^T (rank zero-padded
  //      to 64); the base product then accumulates onto it.  With nseg > 1
  //      segments of seg output columns (fwd) or reduction columns (dX), each
  //      segment g has its own T_g / G_g [M, r] (at LA + g M r) and L2_g [r, seg]
  //      (at LB + g r seg) / L1_g [K, r] (at LB + g K r): the forward tile uses
  //      its own segment's pair (tiles never straddle segments), the dX tile
  //      sums the products of all segments.
  {
    LDS_AS uint16_t* la = (LDS_AS uint16_t*)lds_b;                 // [256][kPL]: T / G rows
    LDS_AS uint16_t* lb = (LDS_AS uint16_t*)lds_b + kBM * kPL;     // fwd: L2 [64][kPD]; dX: L1 [256][kPL]
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[i][j] = f32x16{};
    const int ng = kDx ? nseg : 1;
    for (int g = 0; g < ng; ++g) {
      const int64_t gs = kDx ? g : p0 / seg;
      const uint16_t* la_src = LA + gs * M * r;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int row = (t >> 3) + 64 * i, cc = (t & 7) * 8;
        u32x4 v = {0, 0, 0, 0};
        if (m0 + row < M) v = load_row8(la_src + (m0 + row) * r, cc, r);
        *(LDS_AS u32x4*)(la + row * kPL + cc) = v;
      }
      if (!kDx) {
        const uint16_t* lb_src = LB + gs * r * seg;
        const int64_t pc = p0 - gs * seg;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int c = (t >> 5) + 16 * i, pp = (t & 31) * 8;
          u32x4 v = {0, 0, 0, 0};
          if (c < r) v = load_row8(lb_src + (int64_t)c * seg, pc + pp, seg);
          *(LDS_AS u32x4*)(lb + c * kPD + pp) = v;
        }
      } else {
        const uint16_t* lb_src = LB + gs * K * r;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int row = (t >> 3) + 64 * i, cc = (t & 7) * 8;
          u32x4 v = {0, 0, 0, 0};
          if (p0 + row < K) v = load_row8(lb_src + (p0 + row) * r, cc, r);
          *(LDS_AS u32x4*)(lb + row * kPL + cc) = v;
        }
      }
      __syncthreads();
      const int ksteps = (r + 15) / 16;
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          f32x16 z = acc[i][j];
          for (int s = 0; s < ksteps; ++s) {
            const bf16x8 a = qk::frag_rowmajor(la, kPL, 64 * rg + 32 * i, 16 * s);
            // dX: the column of accumulator slot (l % 32) is dx_slot_col(l % 32)
            const bf16x8 b =
                kDx ? *(const LDS_AS bf16x8*)(lb + (128 * ch + 32 * j + (kPerm ? dx_slot_col(l & 31) : (l & 31))) *
                                                       kPL + 16 * s + 8 * (l >> 5))
                    : qk::frag_kmajor(lb, kPD, 16 * s, 128 * ch + 32 * j);
            z = qk::mfma32(a, b, z);
          }
          acc[i][j] = z;
        }
      __syncthreads();
    }
    if (!kDx) {
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = scale * acc[i][j];
    }
  }

  // ---- activation tiles.  Wave w loads rows 64 (w % 4) + 32 (w / 4) .. +32 of
  // the tile, eight rows per 16-byte load (lane l: row + l / 8, slot l % 8).
  // In LDS, row rho keeps its 16-byte chunk c in slot c ^ ((rho >> 1) & 7): the
  // lane loads chunk (l % 8) ^ (that swizzle) and stores linearly.
  uint32_t achunk[2], arow_off[4];
  achunk[0] = (uint32_t)((l & 7) ^ (l >> 4));     // rows with (rho >> 1) & 7 = l / 16
  achunk[1] = achunk[0] ^ 4u;                     // rows with (rho >> 1) & 7 = 4 + l / 16
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int row = 64 * rg + 32 * ch + 8 * j + (l >> 3);
    arow_off[j] = (uint32_t)((int64_t)row * R * 2) + 16u * achunk[j & 1];
  }
  // Step st reads through a descriptor based at column 64 st of the tile's first
  // row whose size ends at the end of A: rows past M read as zeros, and a step
  // past the reduction has size 0.
  // Tile st goes straight from global memory into the LDS buffer: each wave's
  // load j fills rows 64 (w % 4) + 32 (w / 4) + 8 j .. +8 in lane order (lane l:
  // 16 bytes at 16 l), the lane's global offset carrying the chunk swizzle.
  // The bf16-weight forward sends its weight tile (rows p0 .. p0 + 255 of W,
  // the same row length R = K) the same way.
  auto dma_tile = [&](const uint16_t* src, int64_t rows, int64_t r0, int64_t st, LDS_AS uint16_t* abuf) {
    const int64_t left = R - st * kBR;
    const int rem = __builtin_amdgcn_readfirstlane((int)(left < kBR ? left : kBR));   // columns in this step
    const uint64_t nrec = rem > 0 ? (uint64_t)(rows - r0) * R * 2 - (uint64_t)st * kBR * 2 : 0;
    const uint64_t base = (uint64_t)(uintptr_t)(src + r0 * R + (rem > 0 ? st * kBR : 0));
    const uint16_t* pa = (const uint16_t*)(((uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((int)(base >> 32)) << 32) |
                                           (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)base));
    const __amdgpu_buffer_rsrc_t ra = rsrc(pa, (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)nrec));
    const bool ok0 = !kTail || 8 * (int)achunk[0] < rem;    // chunks past the reduction read as zeros
    const bool ok1 = !kTail || 8 * (int)achunk[1] < rem;
    // Issued from inline assembly, which writes no register: the compiler's
    // own wait counting only over-waits around it, and it does not make every
    // LDS read of the step wait for these loads (the builtin does, as it cannot
    // tell the buffers apart); the barrier at the end of the step waits for them.
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const uint32_t dst = (uint32_t)(uintptr_t)(abuf + (64 * rg + 32 * ch + 8 * j) * kBR);
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
  auto dma_a = [&](int64_t st, LDS_AS uint16_t* abuf) { dma_tile(A, M, m0, st, abuf); };
  auto dma_w = [&](int64_t st, LDS_AS uint16_t* bbuf) { dma_tile(Wb, N, p0, st, bbuf); };
  // A fragment of sub-step s, tile i: row 64 (w % 4) + 32 i + l % 32, chunk 2 s + l / 32.
  uint32_t afrag_off[4];
#pragma unroll
  for (int s = 0; s < 4; ++s)
    afrag_off[s] = (uint32_t)((64 * rg + (l & 31)) * kBR * 2 + 16 * ((2 * s + (l >> 5)) ^ ((l >> 1) & 7)));
  auto afrag = [&](const LDS_AS uint16_t* abuf, int s, int i) {
    return *(const LDS_AS bf16x8*)((const LDS_AS char*)abuf + afrag_off[s] + 32 * kBR * 2 * i);
  };

  // ---- bf16 weight tiles (kB16).  Forward: B fragment of column p from the
  // DMA'd [p][k] tile, addressed like the A fragments.  dX: thread t loads 64
  // bytes of row 64 step + t / 8 of W (columns p0 + 32 (t % 8) .. +32) two steps
  // ahead and stores them into the [n][p] tile of pitch kPD.
  const __amdgpu_buffer_rsrc_t rw = rsrc(Wb, kB16 ? (uint64_t)N * K * 2 : 0);
  auto wfrag = [&](const LDS_AS uint16_t* bbuf, int s, int j) {
    return *(const LDS_AS bf16x8*)((const LDS_AS char*)bbuf + afrag_off[s] - (64 * rg) * kBR * 2 +
                                   (128 * ch + 32 * j) * kBR * 2);
  };
  auto load_wrow = [&](int64_t step) {
    RowBytes rb_;
    const int64_t wrow = step * kBR + (t >> 3);
    const int64_t col = p0 + 32 * (t & 7);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const bool ok = wrow < N && col + 8 * q < K;
      rb_.v[q] = __builtin_amdgcn_raw_buffer_load_b128(rw, ok ? (uint32_t)((wrow * K + col + 8 * q) * 2) : kOOB, 0, 0);
    }
    return rb_;
  };
  auto store_wrow = [&](const RowBytes& rb_, LDS_AS uint16_t* buf, int q) {
    *(LDS_AS u32x4*)(buf + (t >> 3) * kPD + 32 * (t & 7) + 8 * q) = rb_.v[q];
  };

  // ---- weight tiles.  The thread pair (2 u, 2 u + 1) owns one block per step,
  // thread 2 u + h converts its half h (32 weights):
  //  fwd: weight row p0 + t / 2, block = step;                  tile [t / 2][32 h ..)
  //  dX : weight row 64 step + t / 8, block p0 / 64 + (t / 2) % 4; tile [t / 8][64 ((t / 2) % 4) + 32 h ..)
  const __amdgpu_buffer_rsrc_t rc = rsrc(codes, (uint64_t)N * (K / 2));
  const __amdgpu_buffer_rsrc_t r2 = rsrc(c2, (uint64_t)N * kblocks);
  const __amdgpu_buffer_rsrc_t r1 = rsrc(c1, 4 * (((uint64_t)N * kblocks + 255) / 256));
  const int half = t & 1;
  auto load_codes = [&](int64_t step) {
    int64_t wrow, kb;
    if (!kDx) { wrow = p0 + (t >> 1); kb = step; }
    else { wrow = step * kBR + (t >> 3); kb = p0 / 64 + ((t >> 1) & 3); }
    // out-of-range blocks get bit 31 set in their offsets: past every buffer end
    const uint32_t oob = (wrow < N && kb < kblocks) ? 0u : kOOB;
    const uint32_t b = (uint32_t)(wrow * kblocks + kb);
    HalfCodes hc;
    hc.c = __builtin_amdgcn_raw_buffer_load_b128(rc, (uint32_t)(wrow * (K / 2) + kb * 32 + 16 * half) | oob, 0, 0);
    hc.c2b = __builtin_amdgcn_raw_buffer_load_b8(r2, b | oob, 0, 0);
    hc.c1v = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(r1, (4 * (b >> 8)) | oob, 0, 0));
    return hc;
  };
  // fwd: element offset of the thread's 32 weights; dX: byte offset of their
  // low-byte plane row (the high bytes follow one plane row later)
  const int dq_off = kDx ? 2 * (t >> 3) * kPlane + 64 * ((t >> 1) & 3) + 32 * half : (t >> 1) * kPF + 32 * half;
  auto store8 = [&](const BlockLut& L, uint32_t c, LDS_AS uint16_t* buf, int q) {
    if (kDx) {
      u32x2 lo8, hi8;
      dequant8_planes(L, c, kc, lo8, hi8);
      LDS_AS uint8_t* d = (LDS_AS uint8_t*)buf + dq_off + 8 * (q ^ ((t >> 3) & 3));   // chunk swizzle, see frag_planes
      *(LDS_AS u32x2*)d = lo8;
      *(LDS_AS u32x2*)(d + kPlane) = hi8;
    } else {
      *(LDS_AS u32x4*)(buf + dq_off + 8 * q) = dequant8(L, c, kc);
    }
  };
  auto dequant_store = [&](const HalfCodes& hc, LDS_AS uint16_t* buf) {
    const BlockLut L = make_lut(qk::e4m3fn_to_f32(hc.c2b) * hc.c1v, p);
#pragma unroll
    for (int q = 0; q < 4; ++q) store8(L, hc.c[q], buf, q);
  };

  // ---- main loop.  At the top of step st: LDS holds activation tile st and
  // weight tile st; registers hold codes(st + 1).  Step st sends activation tile
  // st + 1 into the other activation buffer (free: its last reads ended before
  // the previous barrier), loads codes(st + 2), multiplies, and converts
  // codes(st + 1) into the other weight buffer; the barrier at its end waits for
  // both new tiles.
  LDS_AS uint16_t* b0 = (LDS_AS uint16_t*)lds_b;
  LDS_AS uint16_t* b1 = (LDS_AS uint16_t*)lds_b + kBufElems;
  LDS_AS uint16_t* a0 = (LDS_AS uint16_t*)lds_a0;
  LDS_AS uint16_t* a1 = (LDS_AS uint16_t*)lds_a1;
  const int64_t nsteps = (R + kBR - 1) / kBR;
  using Stage = StageT<kDx, kB16>;
  auto step = [&](int64_t st, const LDS_AS uint16_t* acur, LDS_AS uint16_t* anext, const LDS_AS uint16_t* bcur,
                  LDS_AS uint16_t* bnext, const Stage& hc_now, Stage& hc_later) {
    // Nothing is in flight here but, on the first step, the loads issued before
    // the loop: waiting for them explicitly tells the compiler's wait tracking
    // that the codes of this step have arrived, so that it places no wait after
    // the loads to LDS below (which it cannot count, and would wait for).
    __builtin_amdgcn_s_waitcnt(0x0070);   // vmcnt(0) lgkmcnt(0)
    dma_a(st + 1, anext);
    if constexpr (kB16 && !kDx) dma_w(st + 1, bnext);
    else if constexpr (kB16) hc_later = load_wrow(st + 2);
    else hc_later = load_codes(st + 2);
    __builtin_amdgcn_sched_barrier(0);
    BlockLut L;
    if constexpr (!kB16) L = make_lut(qk::e4m3fn_to_f32(hc_now.c2b) * hc_now.c1v, p);
    // fragments of sub-step s + 1 are read from LDS while sub-step s runs
    auto bfrag = [&](int s, int j) {
      if constexpr (kB16) return kDx ? qk::frag_kmajor(bcur, kPD, 16 * s, 128 * ch + 32 * j) : wfrag(bcur, s, j);
      else
        return kDx ? frag_planes((const LDS_AS uint8_t*)bcur, 16 * s, 128 * ch + 32 * j)
                   : qk::frag_rowmajor(bcur, kPF, 128 * ch + 32 * j, 16 * s);
    };
    bf16x8 bq[2][4], aq[2][2];
#pragma unroll
    for (int j = 0; j < 4; ++j) bq[0][j] = bfrag(0, j);
    aq[0][0] = afrag(acur, 0, 0);
    aq[0][1] = afrag(acur, 0, 1);
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      if (s < 3) {
#pragma unroll
        for (int j = 0; j < 4; ++j) bq[(s + 1) & 1][j] = bfrag(s + 1, j);
        aq[(s + 1) & 1][0] = afrag(acur, s + 1, 0);
        aq[(s + 1) & 1][1] = afrag(acur, s + 1, 1);
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        acc[0][j] = qk::mfma32(aq[s & 1][0], bq[s & 1][j], acc[0][j]);
        acc[1][j] = qk::mfma32(aq[s & 1][1], bq[s & 1][j], acc[1][j]);
      }
      if constexpr (kB16) {
        // the bf16 weight: a quarter of the thread's row bytes per sub-step (dX);
        // the forward's tile is already on its way to LDS
        if constexpr (kDx) store_wrow(hc_now, bnext, s);
        if (s < 3) __builtin_amdgcn_sched_group_barrier(0x100, kDx ? 10 : 6, 0);   // DS read
        __builtin_amdgcn_sched_group_barrier(0x008, 8, 0);                         // MFMA
        if constexpr (kDx) __builtin_amdgcn_sched_group_barrier(0x200, 1, 0);      // DS write
      } else {
        // one 8-weight group of the next weight tile per sub-step
        store8(L, hc_now.c[s], bnext, s);
        // schedule: the next sub-step's fragment reads first, then one MFMA at a
        // time interleaved with the dequantisation VALU work, then the LDS store
        if (s < 3) __builtin_amdgcn_sched_group_barrier(0x100, kDx ? 10 : 6, 0);   // DS read
#pragma unroll
        for (int k = 0; k < 8; ++k) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);                         // MFMA
          __builtin_amdgcn_sched_group_barrier(0x002, 5, 0);                         // VALU
        }
        __builtin_amdgcn_sched_group_barrier(0x200, kDx ? 2 : 1, 0);                 // DS write
      }
    }
    __builtin_amdgcn_sched_barrier(0);
    // activation tile st + 1 has landed and this wave's LDS stores are done; the
    // barrier hands both new tiles to all waves
    __builtin_amdgcn_s_waitcnt(0x0070);   // vmcnt(0) lgkmcnt(0), seen by the compiler's wait tracking
    __builtin_amdgcn_s_barrier();
  };
  Stage hA, hB;
  {
    dma_a(0, a0);
    if constexpr (kB16 && !kDx) {
      dma_w(0, b0);
    } else if constexpr (kB16) {
      const RowBytes h0 = load_wrow(0);
      hA = load_wrow(1);
#pragma unroll
      for (int q = 0; q < 4; ++q) store_wrow(h0, b0, q);
    } else {
      const HalfCodes h0 = load_codes(0);
      hA = load_codes(1);
      dequant_store(h0, b0);
    }
    __builtin_amdgcn_s_waitcnt(0x0070);   // vmcnt(0) lgkmcnt(0), seen by the compiler's wait tracking
    __builtin_amdgcn_s_barrier();
  }
  // Steps in pairs with no exit between them, so that the loop body is one
  // basic block and the early loads stay where they are issued; an odd step
  // count runs one more step over zeros (codes and activations past the end).
  for (int64_t st = 0; st < nsteps; st += 2) {
    step(st, a0, a1, b0, b1, hA, hB);
    step(st + 1, a1, a0, b1, b0, hB, hA);
  }

  // ---- store C (bf16), lane layout of the 32x32 accumulators
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int64_t pc = p0 + 128 * ch + 32 * j + (kPerm ? dx_slot_col(qk::acc_col()) : qk::acc_col());
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int64_t m = m0 + 64 * rg + 32 * i + qk::acc_row(e);
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
                            float scale, uint16_t* C, hipStream_t s, int nseg) {
  const int64_t P = dx ? K : N;
  const int64_t seg = N / nseg;   // columns of W per segment (a multiple of 256 when nseg > 1)
  dim3 grid((unsigned)((P + kBP - 1) / kBP), (unsigned)((M + kBM - 1) / kBM));
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
  dim3 grid((unsigned)((P + kBP - 1) / kBP), (unsigned)((M + kBM - 1) / kBM));
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
