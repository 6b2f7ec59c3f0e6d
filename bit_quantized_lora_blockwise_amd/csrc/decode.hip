// Decode-sized forward (M <= 16): Y = bf16(X W'^T + s T L2) as one pass over
// the packed 4-bit weight stream.  At these sizes the layer is bound by HBM
// traffic of the codes and scales and by the VALU work of the dequantisation;
// the bf16 weights live only in registers and feed a 16x16x32 bf16 MFMA
// against X.
// Layer formula: nlp-lineage milestone page on QLoRA, "The idea", notation
// paragraph; dequantisation on the fly: examadda page, "The Core Idea".
//
// Work group: 16 weight rows x all of K, split over 8 waves (16 or 4 when X is
// read from global memory) that take 256-column steps in turn; in a step, lane
// (g = l / 16, row = l % 16) holds one block (64 weights, 32 bytes of codes): it
// builds the block's 16-entry bf16 table in registers (two byte planes) and
// looks each nibble up with v_perm_b32.  Each wave keeps one step in flight
// ahead of the one it converts: with many short waves per SIMD the memory
// system returns data in the order it is consumed and the VALU work of one wave
// overlaps the waits of the others (measured better than deeper prefetch in
// fewer waves).  The partial sums of the waves are added in LDS.
// When X is small (M * K <= 16384) it is staged once in LDS, with each group of
// eight columns stored in the order (0, 2, 4, 6, 1, 3, 5, 7): that is the order
// in which the lookups produce the weights (low nibbles, then high nibbles), so
// the MFMA needs no re-interleaving of the looked-up values.  The staging is
// finished before the code stream is requested, so the first steps do not wait
// for X behind the stream.  X of 32 to 128 KB goes to a persistent kernel that
// stages it in LDS once per CU and walks 16-row tiles in turn; larger X is staged
// slice by slice when there is at most one tile per CU, and otherwise read from
// global memory together with the step's codes.
#include "dequant.h"
#include "kernels.h"
#include "tpart.h"

namespace {

using namespace nf4;

constexpr int kRows = 16;                 // weight rows (output columns) per work group
constexpr int kXBytes = 32768;            // LDS budget for X: M * K <= 16384
constexpr int kZeroBytes = 128;           // zeros read in place of X by idle lanes
constexpr uint32_t kOOB = 0x80000000u;    // buffer offset past every range: the load returns 0

typedef short s16x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ f32x4 mfma16(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void* p, uint64_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc((void*)p, (short)0, (int)bytes, 0x00020000);
}

// Operands of one step of a lane: its block's codes and scales, and (when X is
// not staged in LDS) the 64 matching columns of its row of X.
template <bool kXLds>
struct Step {
  u32x4 cw[2];
  uint8_t c2b;                                     // kept a byte: its widening is not scheduled at the load
  float c1v;
  u32x4 xa[kXLds ? 1 : 8];
};

// kFuse: T is formed in this grid, in three roles by work-group index.
//  - The first nprod = S ceil(r / 16) work groups each form one (slice, column
//    tile) of the slices with tpart::slice_tile (the arithmetic of the
//    stand-alone partial-sum kernel), store it to `part` and publish it by
//    writing `epoch` to its flag with release semantics at agent scope.
//  - The next ceil(r / 16) ("summers", one wave each) wait for the S flags of
//    their column tile, read the slices with agent-coherent (sc1) loads, which
//    bypass the other XCDs' non-coherent L2 copies, add them in order s = 0 ..
//    S-1, round T once to bf16, write T_out and publish T as 64-bit records
//    rec[m][c / 2] = {T[m][c], T[m][c + 1], low 32 bits of epoch}, each stored
//    by one single-copy-atomic 64-bit store.
//  - The rest take the 16-row tiles.  A tile's waves request their two records
//    before converting their last step and check the epoch of each at the end,
//    so no ordering between loads is needed and the round trip overlaps the
//    conversion.
// Every wait (a summer's for its flags, a tile's for its records) is bounded by
// `spins` polls: past it the wave forms the slices itself (tpart::slice_wave,
// same bits), so no work group ever depends on another being scheduled.  Flags
// and records carry the epoch of the call that wrote them (never repeated by
// the host), so they need no clearing between calls.
struct TFuse {
  const uint16_t* L1;
  int64_t rows;              // rows of K per slice (multiple of 32)
  int nprod;                 // slice work groups (S ceil(r / 16))
  float* part;               // [S][M][r] fp32 slices
  uint64_t* flags;           // [nprod]
  uint64_t* rec;             // [M][r / 2] T records
  uint64_t epoch;            // its low 32 bits are never 0
  uint32_t spins;
};

// T fragment of lane (g, col) of a wave working on column tile ct: the S slices
// of rows m = col, ranks 16 ct + 4 g .. + 3, added in order s = 0 .. S-1 (read
// once the S producers of the tile have published them, else formed here).
__device__ __forceinline__ f32x4 fused_t_sum(const TFuse& fz, const uint16_t* __restrict__ X, int64_t M, int64_t K,
                                             int r, int S, int ct, bool t_ok, uint32_t off, f32x4* slot) {
  const int l = threadIdx.x & 63;
  const int ctiles = (r + 15) / 16;
  bool ready = false;
  for (uint32_t it = 0;; ++it) {
    const uint64_t f = l < S ? __hip_atomic_load(fz.flags + l * ctiles + ct, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)
                             : fz.epoch;
    ready = __all(f == fz.epoch);
    if (ready || it >= fz.spins) break;
    __builtin_amdgcn_s_sleep(2);
  }
  asm volatile("" ::: "memory");             // the slices are requested after the flags have been seen
  f32x4 sum = {0.0f, 0.0f, 0.0f, 0.0f};
  if (ready) {
    const __amdgpu_buffer_rsrc_t rp = rsrc(fz.part, 4 * (uint64_t)S * M * r);
    f32x4 pv[kDecodeTSlices];
#pragma unroll
    for (int s = 0; s < kDecodeTSlices; ++s)
      pv[s] = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(
                                            rp, (t_ok && s < S) ? off + (uint32_t)(4 * s * M * r) : kOOB, 0,
                                            16 /* sc1: agent-coherent */));
#pragma unroll
    for (int s = 0; s < kDecodeTSlices; ++s)
      if (s < S) sum += pv[s];
  } else {
    for (int s = 0; s < S; ++s) sum += tpart::slice_wave(X, M, K, fz.L1, r, fz.rows, ct, s, slot);
  }
  return sum;
}

// kTPart: T is not given but formed here from the S fp32 slices Tp[s][m][c]
// (added in order s = 0 .. S-1, rounded once), and written to T (if not null)
// by work group 0.
// Stacked linears (G segments of seg_tiles 16-row tiles each, sharing X): the
// work group's segment sg has its own T_sg (at T + sg M r; slices at
// Tp + sg S M r) and L2_sg [r, l2ld] at L2 + sg r l2ld, whose column is the row
// within the segment; Y [M, ld] spans all segments.  The first work group of
// each segment writes that segment's T.  One linear: seg_tiles >= the grid,
// l2ld = ld.
// Eight-wave work groups are held to six waves per SIMD (three work groups per
// CU, at most 80 VGPRs): given the registers, the compiler would otherwise keep
// more values live and fit only two.
template <bool kXLds, int kWv, int kXPer, bool kTPart, bool kFuse>
__global__ __launch_bounds__(64 * kWv, kWv == 8 ? 6 : 1) void k_qgemv_fwd(const uint16_t* __restrict__ X, int64_t M, int64_t K,
                                                        int64_t N, int64_t ld, const uint8_t* __restrict__ codes,
                                                        const uint8_t* __restrict__ c2,
                                                        const float* __restrict__ c1,
                                                        uint16_t* __restrict__ T, const float* __restrict__ Tp, int S,
                                                        const uint16_t* __restrict__ L2, int r, float scale,
                                                        uint16_t* __restrict__ Y, Nf4Params p, int seg_tiles,
                                                        int64_t l2ld, TFuse fz) {
  static_assert(!kFuse || (kXLds && kTPart), "slices formed in the grid: X staged in LDS, T from slices");
  constexpr int kThr = 64 * kWv;
  __shared__ __attribute__((aligned(16))) uint8_t lds[(kXLds ? kXBytes + kZeroBytes : 0) + kWv * 64 * 16];
  const int t = threadIdx.x;
  const int w = __builtin_amdgcn_readfirstlane(t >> 6), l = t & 63;
  const int g = l >> 4, col = l & 15;
  if constexpr (kFuse) {
    if ((int)blockIdx.x < fz.nprod) {
      // producer: one (slice, column tile) of T's slices, then its flag
      const int ctiles = (r + 15) / 16;
      tpart::slice_tile<kWv, 2>(X, M, K, fz.L1, r, fz.rows, fz.part, (int)blockIdx.x % ctiles,
                                (int)blockIdx.x / ctiles, (f32x4*)lds);
      if (t == 0) __hip_atomic_store(fz.flags + blockIdx.x, fz.epoch, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
      return;
    }
    if ((int)blockIdx.x < fz.nprod + (r + 15) / 16) {
      // summer of column tile ct (wave 0): T's records for ranks 16 ct .. 16 ct + 15
      if (w != 0) return;
      const int ct = (int)blockIdx.x - fz.nprod;
      const int rb = 16 * ct + 4 * g;
      const bool ok = rb < r && col < M;
      const int S_ = S;
      const f32x4 sum = fused_t_sum(fz, X, M, K, r, S_, ct, ok, (uint32_t)(4 * (col * r + rb)), (f32x4*)lds);
      uint32_t vt[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) vt[j] = qk::f32_to_bf16(sum[j]);
      if (ok) {
        if (T) {
#pragma unroll
          for (int j = 0; j < 4; ++j) T[col * r + rb + j] = (uint16_t)vt[j];
        }
        const uint64_t tag = (uint64_t)(uint32_t)fz.epoch << 32;
        uint64_t* rp = fz.rec + (col * r + rb) / 2;
        __hip_atomic_store(rp, tag | vt[0] | (vt[1] << 16), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __hip_atomic_store(rp + 1, tag | vt[2] | (vt[3] << 16), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
      return;
    }
  }
  const uint32_t tile = kFuse ? blockIdx.x - (uint32_t)(fz.nprod + (r + 15) / 16) : blockIdx.x;
  const int64_t n0 = (int64_t)tile * kRows;
  const int64_t nrow = n0 + col;
  const uint32_t sg = tile / (uint32_t)seg_tiles;               // segment of this work group
  const int64_t nloc = nrow - (int64_t)sg * seg_tiles * kRows;  // its row within the segment
  const bool seg_first = tile == sg * (uint32_t)seg_tiles;
  if (T) T += (int64_t)sg * M * r;                  // a null T (no T to write) stays null
  if (kTPart) Tp += (int64_t)sg * S * M * r;
  L2 += (int64_t)sg * r * l2ld;
  const bool row_ok = nrow < N;
  const bool m_ok = col < M;                       // A-operand row of this lane is X[col]
  const uint32_t kblocks = (uint32_t)(K / qk::kBlock);
  const SplitConst kc = split_const();

  // K is walked in steps of four blocks (256 columns); the waves take the steps
  // in turn, and in step s lane group g takes block 4 s + g, so the four lanes
  // of a row read 128 contiguous bytes of codes.  Step i of wave w is s = w + kWv i.
  const uint32_t nsteps = (kblocks + 3) / 4;
  const uint32_t nst = nsteps > (uint32_t)w ? (nsteps - (uint32_t)w + kWv - 1) / kWv : 0u;   // uniform
  const uint32_t kb0 = 4u * (uint32_t)w + (uint32_t)g;
  const uint32_t kbstep = 4u * kWv;
  const uint32_t kb_lim = row_ok ? kblocks : 0u;   // blocks valid for the lane's weight row
  // row offsets formed before any load is issued and made opaque: refolded into
  // a later add, the compiler's 64-bit multiply-add may take a register that a
  // pending load writes as its don't-care high half, and then wait for that load
  uint32_t code_row = (uint32_t)(nrow * (K / 2));
  uint32_t blk_row = (uint32_t)(nrow * kblocks);
  asm volatile("" : "+v"(code_row), "+v"(blk_row));

  const __amdgpu_buffer_rsrc_t rc = rsrc(codes, (uint64_t)N * (K / 2));
  const __amdgpu_buffer_rsrc_t r2 = rsrc(c2, (uint64_t)N * kblocks);
  const __amdgpu_buffer_rsrc_t r1 = rsrc(c1, 4 * (((uint64_t)N * kblocks + 255) / 256));
  const __amdgpu_buffer_rsrc_t rx = rsrc(X, (uint64_t)M * K * 2);

  // ---- small X: its loads are issued first, then the first step of the code
  // stream, then X is written to LDS (waiting for the X loads only).  Every
  // 16-byte group of eight columns is stored as (0, 2, 4, 6, 1, 3, 5, 7).
  LDS_AS uint8_t* xl = (LDS_AS uint8_t*)lds;
  u32x4 xr[kXLds ? kXPer : 1];
  const uint32_t xbytes = kXLds ? (uint32_t)(M * K * 2) : 0u;
  if (kXLds) {
#pragma unroll
    for (int j = 0; j < kXPer; ++j) {
      const uint32_t o = 16u * (uint32_t)(t + j * kThr);
      xr[j] = __builtin_amdgcn_raw_buffer_load_b128(rx, o < xbytes ? o : kOOB, 0, 0);
    }
  }
  // T slices (kTPart) next, ahead of the code stream, so that adding them waits
  // for these loads and X only
  const int rb = 16 * w + 4 * g;                   // first of this lane's four LoRA ranks
  const bool t_ok = rb < r && m_ok;                // r % 4 == 0 with kTPart: the four ranks are all in or all out
  f32x4 ps[kTPart ? kDecodeTSlices : 1];
  if (kTPart && !kFuse) {
    const __amdgpu_buffer_rsrc_t rp = rsrc(Tp, 4 * (uint64_t)S * M * r);
#pragma unroll
    for (int s = 0; s < kDecodeTSlices; ++s)
      ps[s] = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(
                                            rp, (t_ok && s < S) ? (uint32_t)(4 * (((int64_t)s * M + col) * r + rb)) : kOOB,
                                            0, 0));
  }
  // The LoRA operands next, still ahead of the code stream: L2[rb .. rb + 3][nrow]
  // and (T given) T[col][rb .. rb + 3], kept as loaded (16-bit) until their use at
  // the end, so that no wait for them covers the code stream.
  uint16_t vl[4], vt16[4];
  {
    const __amdgpu_buffer_rsrc_t rl = rsrc(L2, 2 * (uint64_t)r * l2ld);
    const __amdgpu_buffer_rsrc_t rt = rsrc(T, 2 * (uint64_t)M * r);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const bool rk = rb + j < r;
      const uint32_t ol = (rk && row_ok) ? (uint32_t)(2 * ((int64_t)(rb + j) * l2ld + nloc)) : kOOB;
      vl[j] = __builtin_amdgcn_raw_buffer_load_b16(rl, ol, 0, 0);
      if (!kTPart) {
        const uint32_t ot = (rk && m_ok) ? (uint32_t)(2 * (col * r + rb + j)) : kOOB;
        vt16[j] = __builtin_amdgcn_raw_buffer_load_b16(rt, ot, 0, 0);
      }
    }
  }
  __builtin_amdgcn_sched_barrier(0);
  // Step i >= nst lies past the wave's last step (kb >= kblocks): its loads read
  // zeros, so they are issued without a branch (a branch around a load makes the
  // compiler wait for it where the paths join).
  auto load_step = [&](uint32_t i, Step<kXLds>& st) {
    const uint32_t kb = kb0 + i * kbstep;
    const bool ok = kb < kb_lim;
    const uint32_t co = ok ? code_row + 32u * kb : kOOB;
    const uint32_t b = blk_row + kb;
    st.cw[0] = __builtin_amdgcn_raw_buffer_load_b128(rc, co, 0, 0);
    st.cw[1] = __builtin_amdgcn_raw_buffer_load_b128(rc, co + 16, 0, 0);
    st.c2b = __builtin_amdgcn_raw_buffer_load_b8(r2, ok ? b : kOOB, 0, 0);
    st.c1v = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(r1, ok ? 4 * (b >> 8) : kOOB, 0, 0));
    if (!kXLds) {
      const bool xok = m_ok && kb < kblocks;      // the lane's row of X (independent of its weight row)
      const uint32_t xo = xok ? (uint32_t)((col * K) * 2) + 128u * kb : kOOB;
#pragma unroll
      for (int d = 0; d < 8; ++d) st.xa[d] = __builtin_amdgcn_raw_buffer_load_b128(rx, xo + 16 * d, 0, 0);
    }
  };
  Step<kXLds> sa, sb;
  load_step(0, sa);                                // all-zero (out-of-range offsets) when the wave has no step
  __builtin_amdgcn_sched_barrier(0);

  // ---- T fragment: lane group g holds T[col][rb .. rb + 3]
  uint32_t lt[2];
  {
    uint32_t vt[4];
    if (kTPart && !kFuse) {
      // the slices added in order s = 0 .. S-1, rounded once
      f32x4 sum = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int s = 0; s < kDecodeTSlices; ++s)
        if (s < S) sum += ps[s];
#pragma unroll
      for (int j = 0; j < 4; ++j) vt[j] = qk::f32_to_bf16(sum[j]);
      if (T && seg_first && t_ok) {
#pragma unroll
        for (int j = 0; j < 4; ++j) T[col * r + rb + j] = (uint16_t)vt[j];
      }
      lt[0] = vt[0] | (vt[1] << 16);
      lt[1] = vt[2] | (vt[3] << 16);
    }
  }

  if (kXLds) {
#pragma unroll
    for (int j = 0; j < kXPer; ++j) {
      const uint32_t o = 16u * (uint32_t)(t + j * kThr);
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

  // kFuse: T's two records of this lane (see TFuse), requested before the last
  // step is converted: ra_ in the last pair, rb_ before an odd last step (or
  // when the wave has no steps)
  const __amdgpu_buffer_rsrc_t rrec = rsrc(kFuse ? (const void*)fz.rec : (const void*)Y, 4 * (uint64_t)M * r);
  const uint32_t rec_off = t_ok ? (uint32_t)(4 * (col * r + rb)) : kOOB;
  u32x2 ra0 = {0, 0}, ra1 = {0, 0}, rb0 = {0, 0}, rb1 = {0, 0};
  auto load_recs = [&](bool on, u32x2& v0, u32x2& v1) {
    const uint32_t o = on ? rec_off : kOOB;
    v0 = __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(rrec, o, 0, 16 /* sc1 */));
    v1 = __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(rrec, o + 8, 0, 16 /* sc1 */));
  };

  f32x4 acc = {0, 0, 0, 0};
  auto compute_step = [&](uint32_t i, const Step<kXLds>& st) {
    const uint32_t kb = kb0 + i * kbstep;
    const BlockLut L = make_lut(qk::e4m3fn_to_f32(st.c2b) * st.c1v, p);
    if (kXLds) {
      // X'[col][64 kb .. +64] (eight 16-byte groups), zeros for idle lanes
      const bool xok = m_ok && kb < kblocks;
      const LDS_AS u32x4* xs =
          (const LDS_AS u32x4*)(xl + (xok ? ((uint32_t)col * (uint32_t)K + 64u * kb) * 2u : (uint32_t)kXBytes));
#pragma unroll
      for (int d = 0; d < 8; ++d) {
        const u32x4 bv = dequant8_eo(L, st.cw[d >> 2][d & 3], kc);
        acc = mfma16(__builtin_bit_cast(bf16x8, xs[d]), __builtin_bit_cast(bf16x8, bv), acc);
      }
    } else {
#pragma unroll
      for (int d = 0; d < 8; ++d) {
        const u32x4 bv = dequant8(L, st.cw[d >> 2][d & 3], kc);
        acc = mfma16(__builtin_bit_cast(bf16x8, st.xa[d]), __builtin_bit_cast(bf16x8, bv), acc);
      }
    }
  };
  // steps in pairs, the next step's loads issued before the current one is
  // converted (no exit between the halves: the compiler's wait before each
  // conversion then covers exactly that step), then the odd last step
  uint32_t i = 0;
  for (; kFuse ? i + 2 < nst : i + 2 <= nst; i += 2) {
    load_step(i + 1, sb);
    __builtin_amdgcn_sched_barrier(0);
    compute_step(i, sa);
    load_step(i + 2, sa);
    __builtin_amdgcn_sched_barrier(0);
    compute_step(i + 1, sb);
  }
  if constexpr (kFuse) {
    // the last pair, with the records requested before its second step (a
    // reload in every pair would make each pair wait for the previous one)
    if (i + 2 == nst) {
      load_step(i + 1, sb);
      __builtin_amdgcn_sched_barrier(0);
      compute_step(i, sa);
      load_recs(true, ra0, ra1);
      __builtin_amdgcn_sched_barrier(0);
      compute_step(i + 1, sb);
    } else {
      // an odd last step (or none): the records requested before it
      load_recs(true, rb0, rb1);
      if (i < nst) compute_step(i, sa);
    }
  } else {
    if (i < nst) compute_step(i, sa);
  }
  const bool recs_late = (nst & 1u) != 0 || nst == 0;     // uniform

  {
    // the L2 (and given T) values are first used here: the empty volatile asm
    // keeps the wait for them at this point; the pairs are formed with the perm
    // builtin so that the compiler sees the VALU write ahead of the MFMA
    uint16_t a0 = vl[0], a1 = vl[1], a2 = vl[2], a3 = vl[3];
    asm volatile("" : "+v"(a0), "+v"(a1), "+v"(a2), "+v"(a3));
    const uint32_t ll0 = __builtin_amdgcn_perm(a1, a0, 0x05040100u);
    const uint32_t ll1 = __builtin_amdgcn_perm(a3, a2, 0x05040100u);
    if (!kTPart) {
      uint16_t b0 = vt16[0], b1 = vt16[1], b2 = vt16[2], b3 = vt16[3];
      asm volatile("" : "+v"(b0), "+v"(b1), "+v"(b2), "+v"(b3));
      lt[0] = __builtin_amdgcn_perm(b1, b0, 0x05040100u);
      lt[1] = __builtin_amdgcn_perm(b3, b2, 0x05040100u);
    }
    if constexpr (kFuse) {
      // T from the records published by this grid's summers (see TFuse)
      const uint32_t tag = (uint32_t)fz.epoch;
      u32x2 v0 = recs_late ? rb0 : ra0, v1 = recs_late ? rb1 : ra1;
      bool ok = !t_ok || (v0[1] == tag && v1[1] == tag);
      for (uint32_t it = 0; !__all(ok) && it < fz.spins; ++it) {
        __builtin_amdgcn_s_sleep(2);
        load_recs(true, v0, v1);
        ok = !t_ok || (v0[1] == tag && v1[1] == tag);
      }
      if (__all(ok)) {
        lt[0] = t_ok ? v0[0] : 0u;
        lt[1] = t_ok ? v1[0] : 0u;
      } else {
        // not published within the bound: the slices formed and added here (same bits)
        f32x4* slot = (f32x4*)(lds + (kXLds ? kXBytes + kZeroBytes : 0)) + w * 64;
        f32x4 sum = {0.0f, 0.0f, 0.0f, 0.0f};
        if (16 * w < r)
          for (int s = 0; s < S; ++s) sum += tpart::slice_wave(X, M, K, fz.L1, r, fz.rows, w, s, slot);
        uint32_t vt[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) vt[j] = qk::f32_to_bf16(sum[j]);
        lt[0] = t_ok ? (vt[0] | (vt[1] << 16)) : 0u;
        lt[1] = t_ok ? (vt[2] | (vt[3] << 16)) : 0u;
      }
    }
    f32x4 zl = {0, 0, 0, 0};
    zl = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(s16x4, u32x2{lt[0], lt[1]}),
                                                   __builtin_bit_cast(s16x4, u32x2{ll0, ll1}), zl, 0, 0, 0);
    acc += scale * zl;
  }
  f32x4* red = (f32x4*)(lds + (kXLds ? kXBytes + kZeroBytes : 0));
  red[w * 64 + l] = acc;
  __syncthreads();
  if (w == 0) {
    f32x4 sum = red[l];
#pragma unroll
    for (int ww = 1; ww < kWv; ++ww) sum += red[ww * 64 + l];
    // lane l holds C[m = 4g + i][n = col]
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int m = 4 * g + i;
      if (m < M && row_ok) Y[(int64_t)m * ld + nrow] = qk::f32_to_bf16(sum[i]);
    }
  }
}

// ---------------------------------------------------------------------------
// X of 32 to 128 KB (e.g. M = 16 at K = 4096): one persistent work group of 8
// waves per CU stages all of X in LDS once (the same column order as above) and
// then takes 16-row tiles blockIdx.x, blockIdx.x + gridDim.x, ...; the waves
// split each tile's K as above.  A wave's (tile, step) items form one stream
// with the next item's codes in flight while the current one is converted, so
// the first step of the next tile is requested before the current tile's
// partial sums are added.  Per-work-group X reads in 16-byte pieces (the path
// above for larger X) are replaced by one staging pass per CU.  Eight waves
// (two steps each per tile at K = 4096) measured 3-11% ahead of sixteen (one).
constexpr int kXPersistBytes = 131072;

// One item of a wave's stream: its block's codes and scales.  The scale byte is
// kept as a byte so that its widening is not scheduled at the load.
struct PStep {
  u32x4 cw[2];
  uint8_t c2b;
  float c1v;
};

template <bool kTPart>
__global__ __launch_bounds__(512) void k_qgemv_persist(const uint16_t* __restrict__ X, int64_t M, int64_t K,
                                                        int64_t N, int64_t ld, const uint8_t* __restrict__ codes,
                                                        const uint8_t* __restrict__ c2,
                                                        const float* __restrict__ c1, uint16_t* __restrict__ T,
                                                        const float* __restrict__ Tp, int S,
                                                        const uint16_t* __restrict__ L2, int r, float scale,
                                                        uint16_t* __restrict__ Y, Nf4Params p) {
  constexpr int kWv = 8, kThr = 512, kXPer = kXPersistBytes / (16 * kThr);
  __shared__ __attribute__((aligned(16))) uint8_t lds[kXPersistBytes + kZeroBytes + kWv * 64 * 16];
  const int t = threadIdx.x;
  const int w = __builtin_amdgcn_readfirstlane(t >> 6), l = t & 63;
  const int g = l >> 4, col = l & 15;
  const bool m_ok = col < M;
  const uint32_t kblocks = (uint32_t)(K / qk::kBlock);
  const int64_t ntiles = (N + kRows - 1) / kRows;
  const int64_t my_tiles = ntiles > blockIdx.x ? (ntiles - blockIdx.x + gridDim.x - 1) / gridDim.x : 0;
  const SplitConst kc = split_const();
  const uint32_t nsteps = (kblocks + 3) / 4;
  const uint32_t nst = nsteps > (uint32_t)w ? (nsteps - (uint32_t)w + kWv - 1) / kWv : 0u;   // steps per tile, uniform
  const uint32_t kb0 = 4u * (uint32_t)w + (uint32_t)g;
  const uint32_t kbstep = 4u * kWv;

  const __amdgpu_buffer_rsrc_t rc = rsrc(codes, (uint64_t)N * (K / 2));
  const __amdgpu_buffer_rsrc_t r2 = rsrc(c2, (uint64_t)N * kblocks);
  const __amdgpu_buffer_rsrc_t r1 = rsrc(c1, 4 * (((uint64_t)N * kblocks + 255) / 256));
  const __amdgpu_buffer_rsrc_t rx = rsrc(X, (uint64_t)M * K * 2);
  const __amdgpu_buffer_rsrc_t rl = rsrc(L2, 2 * ((uint64_t)(r - 1) * ld + N));

  // ---- X (all of it) first, then the T slices, then the stream
  LDS_AS uint8_t* xl = (LDS_AS uint8_t*)lds;
  const uint32_t xbytes = (uint32_t)(M * K * 2);
  u32x4 xr[kXPer];
#pragma unroll
  for (int j = 0; j < kXPer; ++j) {
    const uint32_t o = 16u * (uint32_t)(t + j * kThr);
    xr[j] = __builtin_amdgcn_raw_buffer_load_b128(rx, o < xbytes ? o : kOOB, 0, 0);
  }
  const int rb = 16 * w + 4 * g;                   // first of this lane's four LoRA ranks
  const bool t_ok = rb < r && m_ok;
  f32x4 ps[kTPart ? kDecodeTSlices : 1];
  uint16_t vt16[4];                                // T[col][rb .. rb + 3] when T is given
  if (!kTPart) {
    const __amdgpu_buffer_rsrc_t rt = rsrc(T, 2 * (uint64_t)M * r);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const uint32_t ot = (rb + q < r && m_ok) ? (uint32_t)(2 * (col * r + rb + q)) : kOOB;
      vt16[q] = __builtin_amdgcn_raw_buffer_load_b16(rt, ot, 0, 0);
    }
  } else {
    const __amdgpu_buffer_rsrc_t rp = rsrc(Tp, 4 * (uint64_t)S * M * r);
#pragma unroll
    for (int s = 0; s < kDecodeTSlices; ++s)
      ps[s] = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(
                                            rp, (t_ok && s < S) ? (uint32_t)(4 * (((int64_t)s * M + col) * r + rb)) : kOOB,
                                            0, 0));
  }
  __builtin_amdgcn_sched_barrier(0);

  const uint32_t nq = nst * (uint32_t)my_tiles;
  // item q of this wave: tile j = q / nst of the work group, step i = q % nst.
  // Items past the end are requested too, at an offset that reads zeros: with no
  // branch around a load the compiler waits for exactly the step it converts.
  struct Offs {
    uint32_t co, o2, o1;
  };
  // 32-bit offsets: a launch covers fewer than 2^31 code bytes, and rows past N
  // (items past the end) stay below 2^32
  const uint32_t n32 = (uint32_t)N;
  auto item_offs = [&](uint32_t q) {
    const uint32_t j = nst ? q / nst : 0u, i = q - j * nst;
    const uint32_t nrow = (blockIdx.x + j * gridDim.x) * kRows + (uint32_t)col;
    const uint32_t kb = kb0 + i * kbstep;
    const bool ok = q < nq && nrow < n32 && kb < kblocks;
    // block index b; its 32 code bytes start at 32 b.  The product is written out
    // because the compiler's 64-bit multiply-add form borrows a register that may
    // still be waiting for a load.
    uint32_t nk;
    asm("v_mul_lo_u32 %0, %1, %2" : "=v"(nk) : "v"(nrow), "s"(kblocks));
    const uint32_t b = nk + kb;
    return Offs{ok ? 32u * b : kOOB, ok ? b : kOOB, ok ? 4 * (b >> 8) : kOOB};
  };
  auto issue = [&](const Offs& o, PStep& st) {
    st.cw[0] = __builtin_amdgcn_raw_buffer_load_b128(rc, o.co, 0, 0);
    st.cw[1] = __builtin_amdgcn_raw_buffer_load_b128(rc, o.co + 16, 0, 0);
    st.c2b = __builtin_amdgcn_raw_buffer_load_b8(r2, o.o2, 0, 0);
    st.c1v = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(r1, o.o1, 0, 0));
  };
  auto load_item = [&](uint32_t q, PStep& st) { issue(item_offs(q), st); };
  // LoRA L2 fragment of tile j (wave w covers ranks 16 w .. 16 w + 15), kept as
  // loaded until the tile's LoRA product so that nothing waits for it earlier
  uint16_t vl[4];
  auto load_l2 = [&](int64_t j) {
    const int64_t nrow = ((int64_t)blockIdx.x + j * gridDim.x) * kRows + col;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const uint32_t ol = (rb + q < r && nrow < N && j < my_tiles) ? (uint32_t)(2 * ((int64_t)(rb + q) * ld + nrow)) : kOOB;
      vl[q] = __builtin_amdgcn_raw_buffer_load_b16(rl, ol, 0, 0);
    }
  };
  // The first tile's L2 fragment is requested before its first codes (a wait for
  // it then leaves the codes in flight), their offsets formed before either.
  PStep sa, sb;
  const Offs o0 = item_offs(0);
  __builtin_amdgcn_sched_barrier(0);
  load_l2(0);
  issue(o0, sa);

  // ---- T fragment (the same for every tile)
  uint32_t lt[2];
  {
    uint32_t vt[4];
    if (kTPart) {
      f32x4 sum = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int s = 0; s < kDecodeTSlices; ++s)
        if (s < S) sum += ps[s];
#pragma unroll
      for (int q = 0; q < 4; ++q) vt[q] = qk::f32_to_bf16(sum[q]);
      if (T && blockIdx.x == 0 && t_ok) {
#pragma unroll
        for (int q = 0; q < 4; ++q) T[col * r + rb + q] = (uint16_t)vt[q];
      }
    } else {
#pragma unroll
      for (int q = 0; q < 4; ++q) vt[q] = vt16[q];
    }
    lt[0] = vt[0] | (vt[1] << 16);
    lt[1] = vt[2] | (vt[3] << 16);
  }

  // ---- X into LDS, eight-column groups as (0, 2, 4, 6, 1, 3, 5, 7)
#pragma unroll
  for (int j = 0; j < kXPer; ++j) {
    const uint32_t o = 16u * (uint32_t)(t + j * kThr);
    const u32x4 v = xr[j];
    u32x4 e;
    e[0] = __builtin_amdgcn_perm(v[1], v[0], 0x05040100u);
    e[1] = __builtin_amdgcn_perm(v[3], v[2], 0x05040100u);
    e[2] = __builtin_amdgcn_perm(v[1], v[0], 0x07060302u);
    e[3] = __builtin_amdgcn_perm(v[3], v[2], 0x07060302u);
    if (o < xbytes) *(LDS_AS u32x4*)(xl + o) = e;
  }
  if (t < kZeroBytes / 16) *(LDS_AS u32x4*)(xl + kXPersistBytes + 16 * t) = u32x4{0, 0, 0, 0};
  __syncthreads();

  f32x4* red = (f32x4*)(lds + kXPersistBytes + kZeroBytes);
  f32x4 acc = {0, 0, 0, 0};
  // tile j done by this wave: LoRA term, partial sums of the 8 waves added in
  // LDS in a fixed order, output row written; the next tile's L2 fragment requested
  auto finish_tile = [&](int64_t j) {
    // the two bf16 pairs of the L2 fragment, formed here: the empty volatile asm
    // keeps the first use of the loaded values (and the wait for them) at this point
    uint16_t a0 = vl[0], a1 = vl[1], a2 = vl[2], a3 = vl[3];
    asm volatile("" : "+v"(a0), "+v"(a1), "+v"(a2), "+v"(a3));
    const uint32_t ll0 = __builtin_amdgcn_perm(a1, a0, 0x05040100u);
    const uint32_t ll1 = __builtin_amdgcn_perm(a3, a2, 0x05040100u);
    f32x4 zl = {0, 0, 0, 0};
    zl = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(s16x4, u32x2{lt[0], lt[1]}),
                                                   __builtin_bit_cast(s16x4, u32x2{ll0, ll1}), zl, 0, 0, 0);
    acc += scale * zl;
    red[w * 64 + l] = acc;
    acc = f32x4{0, 0, 0, 0};
    __syncthreads();
    if (w == 0) {
      f32x4 sum = red[l];
#pragma unroll
      for (int ww = 1; ww < kWv; ++ww) sum += red[ww * 64 + l];
      const int64_t nrow = ((int64_t)blockIdx.x + j * gridDim.x) * kRows + col;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int m = 4 * g + i;
        if (m < M && nrow < N) Y[(int64_t)m * ld + nrow] = qk::f32_to_bf16(sum[i]);
      }
    }
    __syncthreads();                               // red is reused by the next tile
    load_l2(j + 1);
  };
  auto process = [&](uint32_t q, const PStep& st) {
    const uint32_t j = q / nst, i = q - j * nst;
    const uint32_t kb = kb0 + i * kbstep;
    const BlockLut L = make_lut(qk::e4m3fn_to_f32(st.c2b) * st.c1v, p);
    const bool xok = m_ok && kb < kblocks;
    const LDS_AS u32x4* xs =
        (const LDS_AS u32x4*)(xl + (xok ? ((uint32_t)col * (uint32_t)K + 64u * kb) * 2u : (uint32_t)kXPersistBytes));
#pragma unroll
    for (int d = 0; d < 8; ++d) {
      const u32x4 bv = dequant8_eo(L, st.cw[d >> 2][d & 3], kc);
      acc = mfma16(__builtin_bit_cast(bf16x8, xs[d]), __builtin_bit_cast(bf16x8, bv), acc);
    }
    if (i + 1 == nst) finish_tile((int64_t)j);
  };
  if (nst == 0) {
    for (int64_t j = 0; j < my_tiles; ++j) finish_tile(j);   // no steps here: the LoRA ranks and the barriers
  } else {
    // items in pairs (no exit between the two halves, so the compiler's wait
    // before each conversion covers exactly that item), then the odd last one
    uint32_t q = 0;
    for (; q + 2 <= nq; q += 2) {
      load_item(q + 1, sb);
      __builtin_amdgcn_sched_barrier(0);         // requested before this item's work is scheduled
      process(q, sa);
      load_item(q + 2, sa);
      __builtin_amdgcn_sched_barrier(0);
      process(q + 1, sb);
    }
    if (q < nq) process(q, sa);
  }
}

// ---------------------------------------------------------------------------
// X above 128 KB (e.g. M = 16 at 11008 -> 4096, or at 8192 -> 22016): one work
// group of 8 waves per CU stages X in LDS slice by slice (ksl columns at a time,
// a multiple of 4096, so that each wave has an even number of steps per slice)
// and, for each of its tiles b, b + G, .. (at most kT; G work groups), walks the
// slice's steps as above into that tile's own accumulator.  The next item's
// codes are in flight across tile and slice changes.  The tiles are finished
// after the last slice, by every wave at the same points.
template <int kT, bool kTPart>
__global__ __launch_bounds__(512) void k_qgemv_slices(const uint16_t* __restrict__ X, int64_t M, int64_t K,
                                                      int64_t N, int64_t ld, const uint8_t* __restrict__ codes,
                                                      const uint8_t* __restrict__ c2,
                                                      const float* __restrict__ c1, uint16_t* __restrict__ T,
                                                      const float* __restrict__ Tp, int S,
                                                      const uint16_t* __restrict__ L2, int r, float scale,
                                                      uint16_t* __restrict__ Y, int64_t ksl, Nf4Params p) {
  constexpr int kWv = 8, kThr = 512, kXPer = kXPersistBytes / (16 * kThr);
  __shared__ __attribute__((aligned(16))) uint8_t lds[kXPersistBytes + kZeroBytes + kWv * 64 * 16];
  const int t = threadIdx.x;
  const int w = __builtin_amdgcn_readfirstlane(t >> 6), l = t & 63;
  const int g = l >> 4, col = l & 15;
  const bool m_ok = col < M;
  const uint32_t kblocks = (uint32_t)(K / qk::kBlock);
  const uint32_t ntiles = (uint32_t)((N + kRows - 1) / kRows);
  // 1 .. kT (the grid has at most ntiles work groups); a constant for kT = 1,
  // so that no branch surrounds that kernel's step loop
  const uint32_t my_tiles = kT == 1 ? 1u : (ntiles - blockIdx.x + gridDim.x - 1) / gridDim.x;
  const uint32_t nrow0 = blockIdx.x * kRows + (uint32_t)col;          // this lane's row in its first tile
  const uint32_t trows = gridDim.x * kRows;                           // rows from one of its tiles to the next
  const SplitConst kc = split_const();
  const uint32_t nsteps = (kblocks + 3) / 4;
  const uint32_t nst = nsteps > (uint32_t)w ? (nsteps - (uint32_t)w + kWv - 1) / kWv : 0u;   // uniform
  const uint32_t kb0 = 4u * (uint32_t)w + (uint32_t)g;
  const uint32_t kbstep = 4u * kWv;
  const uint32_t per_slice = (uint32_t)(ksl / (256 * kWv));     // steps of a wave per slice (even)
  const int nsl = (int)((K + ksl - 1) / ksl);

  const __amdgpu_buffer_rsrc_t rc = rsrc(codes, (uint64_t)N * (K / 2));
  const __amdgpu_buffer_rsrc_t r2 = rsrc(c2, (uint64_t)N * kblocks);
  const __amdgpu_buffer_rsrc_t r1 = rsrc(c1, 4 * (((uint64_t)N * kblocks + 255) / 256));
  const __amdgpu_buffer_rsrc_t rx = rsrc(X, (uint64_t)M * K * 2);
  const __amdgpu_buffer_rsrc_t rl = rsrc(L2, 2 * ((uint64_t)(r - 1) * ld + N));
  LDS_AS uint8_t* xl = (LDS_AS uint8_t*)lds;

  // slice sl of X: row m's columns [sl ksl, sl ksl + ksl) at m ksl * 2 bytes; chunk
  // c of the thread-linear order holds row c / (ksl / 8), columns 8 (c % (ksl / 8)) ..
  const uint32_t cpr = (uint32_t)(ksl / 8);                       // 16-byte chunks per row
  const uint32_t nchunk = (uint32_t)M * cpr;
  auto load_x = [&](int sl, u32x4 (&xr)[kXPer]) {
#pragma unroll
    for (int j = 0; j < kXPer; ++j) {
      const uint32_t c = (uint32_t)(t + j * kThr);
      const uint32_t m = c / cpr, cg = c - m * cpr;
      const int64_t kc0 = (int64_t)sl * ksl + 8 * (int64_t)cg;
      const bool ok = c < nchunk && kc0 < K;
      xr[j] = __builtin_amdgcn_raw_buffer_load_b128(rx, ok ? (uint32_t)((m * K + kc0) * 2) : kOOB, 0, 0);
    }
  };
  auto store_x = [&](const u32x4 (&xr)[kXPer]) {
#pragma unroll
    for (int j = 0; j < kXPer; ++j) {
      const uint32_t c = (uint32_t)(t + j * kThr);
      const u32x4 v = xr[j];
      u32x4 e;
      e[0] = __builtin_amdgcn_perm(v[1], v[0], 0x05040100u);
      e[1] = __builtin_amdgcn_perm(v[3], v[2], 0x05040100u);
      e[2] = __builtin_amdgcn_perm(v[1], v[0], 0x07060302u);
      e[3] = __builtin_amdgcn_perm(v[3], v[2], 0x07060302u);
      if (c < nchunk) *(LDS_AS u32x4*)(xl + 16 * c) = e;
    }
  };
  u32x4 xr[kXPer];
  load_x(0, xr);
  const int rb = 16 * w + 4 * g;                   // first of this lane's four LoRA ranks
  const bool t_ok = rb < r && m_ok;
  f32x4 ps[kTPart ? kDecodeTSlices : 1];
  uint16_t vt16[4], vl[kT][4];
  if (!kTPart) {
    const __amdgpu_buffer_rsrc_t rt = rsrc(T, 2 * (uint64_t)M * r);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const uint32_t ot = (rb + q < r && m_ok) ? (uint32_t)(2 * (col * r + rb + q)) : kOOB;
      vt16[q] = __builtin_amdgcn_raw_buffer_load_b16(rt, ot, 0, 0);
    }
  } else {
    const __amdgpu_buffer_rsrc_t rp = rsrc(Tp, 4 * (uint64_t)S * M * r);
#pragma unroll
    for (int s = 0; s < kDecodeTSlices; ++s)
      ps[s] = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(
                                            rp, (t_ok && s < S) ? (uint32_t)(4 * (((int64_t)s * M + col) * r + rb)) : kOOB,
                                            0, 0));
  }
#pragma unroll
  for (int jt = 0; jt < kT; ++jt) {
    const uint32_t nrow = nrow0 + (uint32_t)jt * trows;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const uint32_t ol = (rb + q < r && nrow < (uint32_t)N) ? (uint32_t)(2 * ((int64_t)(rb + q) * ld + nrow)) : kOOB;
      vl[jt][q] = __builtin_amdgcn_raw_buffer_load_b16(rl, ol, 0, 0);
    }
  }
  // row offsets before the code stream, opaque (see the main kernel)
  uint32_t blk_row = nrow0 * kblocks;
  asm volatile("" : "+v"(blk_row));
  const uint32_t tblk = trows * kblocks;           // blocks from one tile's row to the next tile's
  __builtin_amdgcn_sched_barrier(0);
  auto load_item = [&](uint32_t jn, uint32_t i, PStep& st) {   // tile jn's step i of this wave (past nst: zeros)
    const uint32_t kb = kb0 + i * kbstep;
    const bool ok = i < nst && nrow0 + jn * trows < (uint32_t)N && kb < kblocks;
    const uint32_t b = blk_row + jn * tblk + kb;
    const uint32_t co = ok ? 32u * b : kOOB;
    st.cw[0] = __builtin_amdgcn_raw_buffer_load_b128(rc, co, 0, 0);
    st.cw[1] = __builtin_amdgcn_raw_buffer_load_b128(rc, co + 16, 0, 0);
    st.c2b = __builtin_amdgcn_raw_buffer_load_b8(r2, ok ? b : kOOB, 0, 0);
    st.c1v = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(r1, ok ? 4 * (b >> 8) : kOOB, 0, 0));
  };
  PStep sa, sb;
  load_item(0, 0, sa);

  uint32_t lt[2];
  {
    uint32_t vt[4];
    if (kTPart) {
      f32x4 sum = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int s = 0; s < kDecodeTSlices; ++s)
        if (s < S) sum += ps[s];
#pragma unroll
      for (int q = 0; q < 4; ++q) vt[q] = qk::f32_to_bf16(sum[q]);
      if (T && blockIdx.x == 0 && t_ok) {
#pragma unroll
        for (int q = 0; q < 4; ++q) T[col * r + rb + q] = (uint16_t)vt[q];
      }
    } else {
#pragma unroll
      for (int q = 0; q < 4; ++q) vt[q] = vt16[q];
    }
    lt[0] = vt[0] | (vt[1] << 16);
    lt[1] = vt[2] | (vt[3] << 16);
  }
  store_x(xr);
  if (t < kZeroBytes / 16) *(LDS_AS u32x4*)(xl + kXPersistBytes + 16 * t) = u32x4{0, 0, 0, 0};
  __syncthreads();

  f32x4 acc[kT];
#pragma unroll
  for (int jt = 0; jt < kT; ++jt) acc[jt] = f32x4{0, 0, 0, 0};
  auto process = [&](f32x4& ac, uint32_t i, int sl, const PStep& st) {
    const uint32_t kb = kb0 + i * kbstep;
    const BlockLut L = make_lut(qk::e4m3fn_to_f32(st.c2b) * st.c1v, p);
    const bool xok = m_ok && kb < kblocks && i < nst;
    const uint32_t kl = kb - (uint32_t)sl * (uint32_t)(ksl / 64);  // block within the slice
    const LDS_AS u32x4* xs = (const LDS_AS u32x4*)(xl + (xok ? ((uint32_t)col * (uint32_t)ksl + 64u * kl) * 2u
                                                             : (uint32_t)kXPersistBytes));
#pragma unroll
    for (int d = 0; d < 8; ++d) {
      const u32x4 bv = dequant8_eo(L, st.cw[d >> 2][d & 3], kc);
      ac = mfma16(__builtin_bit_cast(bf16x8, xs[d]), __builtin_bit_cast(bf16x8, bv), ac);
    }
  };
  for (int sl = 0; sl < nsl; ++sl) {
    if (sl > 0) {
      load_x(sl, xr);
      __syncthreads();                             // every wave is done with slice sl - 1
      store_x(xr);
      __syncthreads();
    }
    // for each tile, this wave's steps of the slice in pairs (per_slice is
    // even); the item after a tile's last is the next tile's first of the
    // slice, or tile 0's first of the next slice, already requested into sa
    const uint32_t i0 = (uint32_t)sl * per_slice, i_end = i0 + per_slice;
#pragma unroll
    for (int jt = 0; jt < kT; ++jt) {
      if ((uint32_t)jt < my_tiles) {
        const bool last_t = (uint32_t)jt + 1 >= my_tiles;
        const uint32_t nj = last_t ? 0u : (uint32_t)jt + 1, ni = last_t ? i_end : i0;
        for (uint32_t i = i0; i < i_end; i += 2) {
          load_item((uint32_t)jt, i + 1, sb);
          __builtin_amdgcn_sched_barrier(0);
          process(acc[jt], i, sl, sa);
          const bool wrap = i + 2 >= i_end;
          load_item(wrap ? nj : (uint32_t)jt, wrap ? ni : i + 2, sa);
          __builtin_amdgcn_sched_barrier(0);
          process(acc[jt], i + 1, sl, sb);
        }
      }
    }
  }

  // each tile: LoRA term, the 8 waves' partial sums added in a fixed order
  f32x4* red = (f32x4*)(lds + kXPersistBytes + kZeroBytes);
#pragma unroll
  for (int jt = 0; jt < kT; ++jt) {
    if ((uint32_t)jt < my_tiles) {
      uint16_t a0 = vl[jt][0], a1 = vl[jt][1], a2 = vl[jt][2], a3 = vl[jt][3];
      asm volatile("" : "+v"(a0), "+v"(a1), "+v"(a2), "+v"(a3));
      const uint32_t ll0 = __builtin_amdgcn_perm(a1, a0, 0x05040100u);
      const uint32_t ll1 = __builtin_amdgcn_perm(a3, a2, 0x05040100u);
      f32x4 zl = {0, 0, 0, 0};
      zl = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(s16x4, u32x2{lt[0], lt[1]}),
                                                     __builtin_bit_cast(s16x4, u32x2{ll0, ll1}), zl, 0, 0, 0);
      f32x4 a = acc[jt];
      a += scale * zl;
      red[w * 64 + l] = a;
      __syncthreads();
      const uint32_t nrow = nrow0 + (uint32_t)jt * trows;
      if (w == 0) {
        f32x4 sum = red[l];
#pragma unroll
        for (int ww = 1; ww < kWv; ++ww) sum += red[ww * 64 + l];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int m = 4 * g + i;
          if (m < M && nrow < (uint32_t)N) Y[(int64_t)m * ld + nrow] = qk::f32_to_bf16(sum[i]);
        }
      }
      __syncthreads();                             // red is reused by the next tile
    }
  }
}

// One launch's operands besides the shape and the grid.
struct QgemvArgs {
  const uint16_t* X;
  int64_t M, K, rows, ld;
  const uint8_t* codes;
  const uint8_t* c2;
  const float* c1;
  uint16_t* T;
  const float* Tp;
  int S;
  const uint16_t* L2;
  int r;
  float scale;
  uint16_t* Y;
  int seg_tiles = 0x7fffffff;   // 16-row tiles per stacked segment (one linear: more than any grid)
  int64_t l2ld = 0;             // row stride of each segment's L2 (0: ld)
  TFuse fz = {};                // slices of T formed in the grid (k_qgemv_fwd only)
};

template <bool kTPart>
hipError_t launch_slices(int kt, unsigned grid, int64_t ksl, hipStream_t s, const QgemvArgs& a) {
#define QL_SLICES(KT)                                                                                              \
  hipLaunchKernelGGL((k_qgemv_slices<KT, kTPart>), dim3(grid), dim3(512), 0, s, a.X, a.M, a.K, a.rows, a.ld, a.codes, \
                     a.c2, a.c1, a.T, a.Tp, a.S, a.L2, a.r, a.scale, a.Y, ksl, nf4_params())
  if (kt <= 1)
    QL_SLICES(1);
  else if (kt <= 2)
    QL_SLICES(2);
  else if (kt <= 4)
    QL_SLICES(4);
  else
    QL_SLICES(8);
#undef QL_SLICES
  return hipGetLastError();
}

template <bool kXLds, int kWv, int kXPer, bool kTPart, bool kFuse = false>
hipError_t launch_one(dim3 grid, hipStream_t s, const QgemvArgs& a) {
  hipLaunchKernelGGL((k_qgemv_fwd<kXLds, kWv, kXPer, kTPart, kFuse>), grid, dim3(64 * kWv), 0, s, a.X, a.M, a.K,
                     a.rows, a.ld, a.codes, a.c2, a.c1, a.T, a.Tp, a.S, a.L2, a.r, a.scale, a.Y, nf4_params(),
                     a.seg_tiles, a.l2ld ? a.l2ld : a.ld, a.fz);
  return hipGetLastError();
}

// Small-X variant for kWv waves: the fewest X loads per thread (1, 2 or 4)
// that cover M * K * 2 bytes.
template <int kWv, bool kTPart, bool kFuse = false>
hipError_t launch_lds(dim3 grid, hipStream_t s, const QgemvArgs& a) {
  const int64_t per = (a.M * a.K * 2 + 16 * 64 * kWv - 1) / (16 * 64 * kWv);
  if (per <= 1) return launch_one<true, kWv, 1, kTPart, kFuse>(grid, s, a);
  if (per <= 2) return launch_one<true, kWv, 2, kTPart, kFuse>(grid, s, a);
  return launch_one<true, kWv, 4, kTPart, kFuse>(grid, s, a);
}

template <bool kTPart>
hipError_t launch_shape(const QgemvArgs& a0, int64_t N, hipStream_t s) {
  // Buffer offsets are 32-bit: X and the packed codes must each stay below 2^31
  // bytes (the library's shape check guarantees both).
  QgemvArgs a = a0;
  a.rows = N;
  a.ld = N;
  const int64_t K = a.K, M = a.M;
  if (M * K * 2 >= (int64_t(1) << 31) || N * (K / 2) >= (int64_t(1) << 31)) return hipErrorInvalidValue;
  const bool xlds = M * K * 2 <= kXBytes;
  const bool xpersist = !xlds && M * K * 2 <= kXPersistBytes;
  int cus = 0;
  if (!xlds) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) !=
                                                hipSuccess || cus < 1)
      cus = 256;
  }
  const int64_t wgs = (a.rows + kRows - 1) / kRows;
  dim3 grid((unsigned)wgs);
  // X read from global memory: 16 waves per work group when the grid alone
  // would leave SIMDs with fewer than two waves, else 4
  const bool wide = wgs <= 384;
  // X above 128 KB: the slice kernel, one work group per CU (cus >= 1 here)
  // with at most tpw tiles each, slices a multiple of 4096 columns wide.
  // Several tiles per work group are measured ahead of X read from global
  // memory from M = 6 (8192 <-> 22016), behind it at M = 4.
  const bool big = !xlds && !xpersist;
  const int64_t ksl = big ? (kXPersistBytes / (2 * M)) / 4096 * 4096 : 0;
  const int64_t sg = big ? (wgs < cus ? wgs : cus) : 1;
  const int64_t tpw = (wgs + sg - 1) / sg;
  if (big && ksl >= 4096 && (tpw == 1 || (tpw <= 8 && M >= 6))) return launch_slices<kTPart>((int)tpw, (unsigned)sg, ksl, s, a);
  if (xpersist) {
    const unsigned pg = (unsigned)(wgs < cus ? wgs : cus);
    hipLaunchKernelGGL((k_qgemv_persist<kTPart>), dim3(pg), dim3(512), 0, s, a.X, a.M, a.K, a.rows, a.ld, a.codes,
                       a.c2, a.c1, a.T, a.Tp, a.S, a.L2, a.r, a.scale, a.Y, nf4_params());
    return hipGetLastError();
  }
  if (xlds) return launch_lds<8, kTPart>(grid, s, a);     // 8 waves: measured ahead of 16 on small grids too
  // X read with each step (127 VGPRs): four waves keep four work groups per CU resident
  return wide ? launch_one<false, 16, 1, kTPart>(grid, s, a) : launch_one<false, 4, 1, kTPart>(grid, s, a);
}

}  // namespace

hipError_t launch_qgemv_fwd_tpart(const uint16_t* X, int64_t M, int64_t K, int64_t N, const uint8_t* codes,
                                  const uint8_t* c2, const float* c1, const float* Tpart, int S, uint16_t* T_out,
                                  const uint16_t* L2, int r, float scale, uint16_t* Y, hipStream_t s) {
  if (S < 1 || S > kDecodeTSlices || (r % 4) != 0 || ((uintptr_t)Tpart & 15) != 0) return hipErrorInvalidValue;
  const QgemvArgs a{X, M, K, 0, N, codes, c2, c1, T_out, Tpart, S, L2, r, scale, Y};
  return launch_shape<true>(a, N, s);
}

bool qgemv_fused_ok(int64_t M, int64_t K, int r) {
  return M >= 1 && M <= 16 && M * K * 2 <= kXBytes && (K % 64) == 0 && r >= 4 && r <= 64 && (r % 4) == 0;
}

size_t qgemv_fused_sync_bytes(int64_t M, int r) {
  return 8 * (size_t)kDecodeTSlices * ((r + 15) / 16) + 4 * (size_t)M * r;
}

hipError_t launch_qgemv_fwd_fused(const uint16_t* X, int64_t M, int64_t K, int64_t N, const uint8_t* codes,
                                  const uint8_t* c2, const float* c1, const uint16_t* L1, int r, float* part,
                                  void* sync, uint64_t epoch, uint32_t spins, uint16_t* T_out,
                                  const uint16_t* L2, float scale, uint16_t* Y, hipStream_t s) {
  if (!qgemv_fused_ok(M, K, r) || ((uintptr_t)part & 15) != 0 || ((uintptr_t)sync & 15) != 0 ||
      (uint32_t)epoch == 0 || N * (K / 2) >= (int64_t(1) << 31))
    return hipErrorInvalidValue;
  const int S = decode_t_slices(K);
  const int ctiles = (r + 15) / 16;
  QgemvArgs a{X, M, K, N, N, codes, c2, c1, T_out, part, S, L2, r, scale, Y};
  uint64_t* flags = (uint64_t*)sync;
  a.fz = TFuse{L1, decode_t_rows(K), S * ctiles, part, flags, flags + (size_t)kDecodeTSlices * ctiles, epoch, spins};
  const int64_t wgs = (N + kRows - 1) / kRows;
  return launch_lds<8, true, true>(dim3((unsigned)(a.fz.nprod + ctiles + wgs)), s, a);
}

bool qgemv_group_ok(int64_t M, int64_t K, int64_t N, int G) {
  return M >= 1 && M * K * 2 <= kXBytes && N % kRows == 0 && G >= 1 && (int64_t)G * N * (K / 2) < (int64_t(1) << 31);
}

hipError_t launch_qgemv_group_tpart(const uint16_t* X, int64_t M, int64_t K, int64_t N, int G, const uint8_t* codes,
                                    const uint8_t* c2, const float* c1, const float* Tpart, int S, uint16_t* T_out,
                                    const uint16_t* L2, int r, float scale, uint16_t* Y, hipStream_t s) {
  if (!qgemv_group_ok(M, K, N, G) || S < 1 || S > kDecodeTSlices || (r % 4) != 0 || ((uintptr_t)Tpart & 15) != 0)
    return hipErrorInvalidValue;
  QgemvArgs a{X, M, K, (int64_t)G * N, (int64_t)G * N, codes, c2, c1, T_out, Tpart, S, L2, r, scale, Y};
  a.seg_tiles = (int)(N / kRows);
  a.l2ld = N;
  return launch_lds<8, true>(dim3((unsigned)(G * (N / kRows))), s, a);
}

hipError_t launch_qgemv_fwd(const uint16_t* X, int64_t M, int64_t K, int64_t N, const uint8_t* codes,
                            const uint8_t* c2, const float* c1, const uint16_t* T, const uint16_t* L2, int r,
                            float scale, uint16_t* Y, hipStream_t s) {
  const QgemvArgs a{X, M, K, 0, N, codes, c2, c1, const_cast<uint16_t*>(T), nullptr, 0, L2, r, scale, Y};
  return launch_shape<false>(a, N, s);
}
