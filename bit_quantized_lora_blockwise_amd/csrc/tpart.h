// Decode-sized T = X L1 (M <= 16) as fp32 partial sums over S slices of the
// reduction, part[s][m][c] (layer formula: nlp-lineage milestone page on QLoRA,
// "The idea", notation paragraph; T is the rank-r product of the input with the
// first adapter).  Shared by the stand-alone partial-sum kernel (lora.hip) and
// the decode kernel that forms the slices in its first work groups
// (decode.hip), so that both produce the same bits.
//
// One column tile (16 of the r columns) of one slice: the slice's rows are cut
// into 32-row chunks; "virtual wave" v (0 .. 15) takes chunks v, v + 16, ... and
// chains one 16x16x32 MFMA per chunk (lane (g, col): X row col, L1 column
// 16 ctile + col, chunk rows 8 g .. 8 g + 7); the sixteen results are then added
// in the order v = 0 .. 15.  A work group of kReal waves runs 16 / kReal virtual
// waves per wave; one wave alone (slice_wave) runs all sixteen in turn.  The
// arithmetic, and so every bit of the result, is the same in all three cases.
#pragma once

#include "common.h"

namespace tpart {

constexpr int kVirt = 16;                 // virtual waves per column tile
constexpr int kCh = 4;                    // chunks in flight per wave
constexpr uint32_t kNone = 0x80000000u;   // buffer offset past every range: the load returns 0

__device__ __forceinline__ __amdgpu_buffer_rsrc_t buf(const void* p, uint64_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc((void*)p, (short)0, (int)(bytes < 0x7FFFFFFFull ? bytes : 0x7FFFFFFFull),
                                           0x00020000);
}

// Operands of chunk `chunk` (absolute index within the slice) for lane (g, col).
struct Op {
  u32x4 a, b;
};

__device__ __forceinline__ Op load_chunk(__amdgpu_buffer_rsrc_t ra, __amdgpu_buffer_rsrc_t rb, int64_t K, int r,
                                         int64_t k_beg, int64_t k_end, int64_t chunk, int g, int col, bool m_ok,
                                         int c, bool c_ok) {
  Op o;
  const int64_t k0 = k_beg + 32 * chunk + 8 * g;
  const bool ok = k0 < k_end;
  o.a = __builtin_amdgcn_raw_buffer_load_b128(ra, (ok && m_ok) ? (uint32_t)((col * K + k0) * 2) : kNone, 0, 0);
  // eight 2-byte loads down column c: one base offset per lane (out of range
  // for an idle lane, so every load returns 0), the row step as a uniform offset
  const uint32_t bo = (ok && c_ok) ? (uint32_t)((k0 * r + c) * 2) : kNone;
  uint32_t v[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) v[j] = __builtin_amdgcn_raw_buffer_load_b16(rb, bo, 2 * r * j, 0);
#pragma unroll
  for (int j = 0; j < 4; ++j) o.b[j] = v[2 * j] | (v[2 * j + 1] << 16);
  return o;
}

__device__ __forceinline__ f32x4 mfma(const Op& o, f32x4 acc) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, o.a), __builtin_bit_cast(bf16x8, o.b),
                                                 acc, 0, 0, 0);
}

// Work group of kReal waves (threadIdx.x < 64 kReal): column tile `ctile` of
// slice `slice` (rows slice * rows .. + rows of K, rows a multiple of 32) into
// part[slice][m][c], kChunks chunks in flight per wave (no effect on the
// result).  red: kVirt * 64 f32x4 of LDS.  Ends with a barrier after
// the stores of wave 0 (the only wave that stores).
template <int kReal, int kChunks = kCh>
__device__ __forceinline__ void slice_tile(const uint16_t* __restrict__ X, int64_t M, int64_t K,
                                           const uint16_t* __restrict__ L1, int r, int64_t rows,
                                           float* __restrict__ part, int ctile, int slice, f32x4* red) {
  static_assert(kVirt % kReal == 0, "virtual waves split evenly over the real ones");
  constexpr int kPer = kVirt / kReal;                      // virtual waves per real wave
  static_assert(kChunks % kPer == 0, "a chunk group holds whole rounds of virtual waves");
  const int t = threadIdx.x;
  const int w = __builtin_amdgcn_readfirstlane(t >> 6), l = t & 63;
  const int g = l >> 4, col = l & 15;
  const int c = ctile * 16 + col;
  const bool c_ok = c < r;
  const bool m_ok = col < M;
  const int64_t k_beg = (int64_t)slice * rows;
  const int64_t k_end = min(K, k_beg + rows);
  const int64_t nk = k_end > k_beg ? (k_end - k_beg) / 32 : 0;
  // chain step i of virtual wave v = w + j kReal is chunk v + i kVirt; the
  // wave's ops are o = i kPer + j, valid while chunk < nk
  const int64_t nst = nk > w ? (nk - w + kVirt - 1) / kVirt : 0;   // steps of virtual wave w (the longest)
  const int64_t nops = nst * kPer;
  const __amdgpu_buffer_rsrc_t ra = buf(X, (uint64_t)M * K * 2);
  const __amdgpu_buffer_rsrc_t rb = buf(L1, (uint64_t)K * r * 2);
  auto chunk_of = [&](int64_t o) { return (int64_t)(w + (int)(o % kPer) * kReal) + (o / kPer) * kVirt; };
  Op ca[kChunks], cb[kChunks];
#pragma unroll
  for (int j = 0; j < kChunks; ++j) ca[j] = load_chunk(ra, rb, K, r, k_beg, k_end, chunk_of(j), g, col, m_ok, c, c_ok);
  f32x4 acc[kPer];
#pragma unroll
  for (int j = 0; j < kPer; ++j) acc[j] = f32x4{0, 0, 0, 0};
  auto mul = [&](int64_t o0, const Op (&o)[kChunks]) {
#pragma unroll
    for (int j = 0; j < kChunks; ++j)
      if (o0 + j < nops && chunk_of(o0 + j) < nk) acc[j % kPer] = mfma(o[j], acc[j % kPer]);
  };
  for (int64_t o0 = 0; o0 < nops; o0 += 2 * kChunks) {
    if (o0 + kChunks < nops) {
#pragma unroll
      for (int j = 0; j < kChunks; ++j) cb[j] = load_chunk(ra, rb, K, r, k_beg, k_end, chunk_of(o0 + kChunks + j), g, col, m_ok, c, c_ok);
    }
    mul(o0, ca);
    if (o0 + kChunks >= nops) break;
    if (o0 + 2 * kChunks < nops) {
#pragma unroll
      for (int j = 0; j < kChunks; ++j) ca[j] = load_chunk(ra, rb, K, r, k_beg, k_end, chunk_of(o0 + 2 * kChunks + j), g, col, m_ok, c, c_ok);
    }
    mul(o0 + kChunks, cb);
  }
#pragma unroll
  for (int j = 0; j < kPer; ++j) red[(w + j * kReal) * 64 + l] = acc[j];
  __syncthreads();
  if (w == 0) {
    f32x4 sum = red[l];
#pragma unroll
    for (int v = 1; v < kVirt; ++v) sum += red[v * 64 + l];
    // lane l holds C[m = 4 g + i][c]
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int m = 4 * g + i;
      if (m < M && c_ok) part[((int64_t)slice * M + m) * r + c] = sum[i];
    }
  }
  __syncthreads();
}

// One wave alone: the same sums for column tile `ctile` of slice `slice`,
// returned transposed for lane (g, col) as part[slice][m = col][16 ctile + 4 g
// + i], i = 0 .. 3 (zeros outside M and r).  slot: 64 f32x4 of LDS owned by
// this wave (used to transpose).
__device__ __forceinline__ f32x4 slice_wave(const uint16_t* __restrict__ X, int64_t M, int64_t K,
                                            const uint16_t* __restrict__ L1, int r, int64_t rows, int ctile, int slice,
                                            f32x4* slot) {
  const int l = threadIdx.x & 63;
  const int g = l >> 4, col = l & 15;
  const int c = ctile * 16 + col;
  const bool c_ok = c < r;
  const bool m_ok = col < M;
  const int64_t k_beg = (int64_t)slice * rows;
  const int64_t k_end = min(K, k_beg + rows);
  const int64_t nk = k_end > k_beg ? (k_end - k_beg) / 32 : 0;
  const __amdgpu_buffer_rsrc_t ra = buf(X, (uint64_t)M * K * 2);
  const __amdgpu_buffer_rsrc_t rb = buf(L1, (uint64_t)K * r * 2);
  f32x4 sum = {0, 0, 0, 0};
  for (int v = 0; v < kVirt; ++v) {
    f32x4 acc = {0, 0, 0, 0};
    for (int64_t ch = v; ch < nk; ch += kVirt)
      acc = mfma(load_chunk(ra, rb, K, r, k_beg, k_end, ch, g, col, m_ok, c, c_ok), acc);
    if (v == 0) sum = acc;
    else sum += acc;
  }
  // lane (g, col) holds C[m = 4 g + i][c = 16 ctile + col]: transpose through the slot
  float* s = (float*)slot;
#pragma unroll
  for (int i = 0; i < 4; ++i) s[(4 * g + i) * 16 + col] = sum[i];
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  f32x4 out;
#pragma unroll
  for (int i = 0; i < 4; ++i) out[i] = s[col * 16 + 4 * g + i];
  __builtin_amdgcn_wave_barrier();
  return out;
}

}  // namespace tpart
