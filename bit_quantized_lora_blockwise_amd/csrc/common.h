// Shared device-side building blocks of the gfx950 kernels: vector types, the
// NF4 parameter block passed to kernels, LDS fragment loaders for the bf16
// MFMA (32x32x16) and small reductions.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

#define LDS_AS __attribute__((address_space(3)))

// NF4 levels (code k -> q[k], ascending) and encoder thresholds: thr[k] is the
// smallest fp32 strictly above the midpoint of q[k] and q[k+1], so that
// code(n) = #{k : n >= thr[k]} is the nearest level with ties to the smaller
// code.  Filled on the host from the level construction (see nf4_table.cpp).
struct Nf4Params {
  float q[16];
  float thr[15];
};

// Encoder lookup over 34 buckets of width 1/16 in n (index floor(16 n) + 17,
// n in [-1, 1]); each bucket holds at most one threshold.  For bucket i:
// t16[i] = 16 * (its threshold), or +inf when it has none; cnt[i] = the number
// of thresholds at or below the bucket's lower end.  An approximate 16 n' with
// |16 n' - t16| <= kNf4Near is too close to decide (+inf is never close).
// Built on the host (see nf4_table.cpp).
struct Nf4Buckets {
  float t16[34];
  uint32_t cnt[34];
  int ok;   // 1 when the construction's assumptions held
};

// The encoder's approximate quotient n' = w * (16 / a) (one reciprocal of at
// most 1 ulp and one rounded product) is within 2^-22 |16 n| of 16 n, n = fl(w / a),
// i.e. within 2^-18.2 of it wherever |16 n| <= 13.8 (the largest |t16|).  The
// margin below is 2.3 times that.
static constexpr float kNf4Near = 0x1p-17f;

namespace qk {

static constexpr int kBlock = 64;   // weights per first-level scale
static constexpr int kGroup = 256;  // first-level scales per second-level scale

__device__ __forceinline__ float bf16_to_f32(uint16_t h) {
  return __uint_as_float(((uint32_t)h) << 16);
}

// Two fp32 -> packed bf16 pair (round to nearest even; v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  bf16x2 p = {(__bf16)lo, (__bf16)hi};
  return __builtin_bit_cast(uint32_t, p);
}

__device__ __forceinline__ uint16_t f32_to_bf16(float x) {
  return __builtin_bit_cast(uint16_t, (__bf16)x);
}

// OCP E4M3FN byte -> fp32 (hardware conversion; gfx950 decodes the OCP format).
__device__ __forceinline__ float e4m3fn_to_f32(uint32_t byte) {
  return __builtin_amdgcn_cvt_f32_fp8((int)byte, 0);
}

// fragment loaders --------------------------------------------------------
// MFMA 32x32x16 bf16 operand layout: lane l holds 8 consecutive reduction
// indices k = 8*(l/32) + [0, 8) of row/column (l % 32).

// LDS tile laid out [row][k] (k contiguous, pitch in elements).
__device__ __forceinline__ bf16x8 frag_rowmajor(const LDS_AS uint16_t* base, int pitch, int row0, int k0) {
  const int l = threadIdx.x & 63;
  const LDS_AS uint16_t* p = base + (row0 + (l & 31)) * pitch + k0 + ((l >> 5) << 3);
  return *(const LDS_AS bf16x8*)p;
}

// LDS tile laid out [k][col] (col contiguous): transposed read with
// ds_read_b64_tr_b16.  In each group of 16 lanes, lane i addresses row i/4 and
// columns 4*(i%4)..+3 of a 4 x 16 block and receives column i of that block.
__device__ __forceinline__ bf16x8 frag_kmajor(const LDS_AS uint16_t* base, int pitch, int k0, int col0) {
  const int l = threadIdx.x & 63;
  const int G = l >> 4, i = l & 15;
  const int row = k0 + ((G >> 1) << 3) + (i >> 2);
  const int col = col0 + ((G & 1) << 4) + ((i & 3) << 2);
  const LDS_AS uint16_t* p = base + row * pitch + col;
  i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS_AS i16x4*)p);
  i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS_AS i16x4*)(p + 4 * pitch));
  u32x2 a = __builtin_bit_cast(u32x2, lo), b = __builtin_bit_cast(u32x2, hi);
  u32x4 v = {a[0], a[1], b[0], b[1]};
  return __builtin_bit_cast(bf16x8, v);
}

__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// Output element (row, col) of lane l, accumulator index j, for a 32x32 tile:
// col = l % 32, row = 8*(j/4) + 4*(l/32) + (j%4).
__device__ __forceinline__ int acc_row(int j) {
  const int l = threadIdx.x & 63;
  return ((j >> 2) << 3) + ((l >> 5) << 2) + (j & 3);
}
__device__ __forceinline__ int acc_col() { return threadIdx.x & 31; }

// max over aligned groups of 8 lanes: swap neighbours, swap pairs, mirror halves of 8
__device__ __forceinline__ uint32_t dpp_max8(uint32_t v) {
  v = max(v, (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0xB1, 0xF, 0xF, true));   // quad_perm [1,0,3,2]
  v = max(v, (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x4E, 0xF, 0xF, true));   // quad_perm [2,3,0,1]
  v = max(v, (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x141, 0xF, 0xF, true));  // row_half_mirror
  return v;
}

// Nearest OCP E4M3FN magnitude code of t in [0, 464) (past 448 the nearest
// finite value is 448), ties to even.  Below 2^-6 the format is fixed-point
// with step 2^-9, so the code is rint(t * 512); above, the fp32 mantissa is
// rounded to 3 bits and the exponent rebased from 127 to 7.
__device__ __forceinline__ uint32_t e4m3fn_encode(float t) {
  if (t < 0.015625f) return (uint32_t)__builtin_rintf(t * 512.0f);
  const uint32_t u = __float_as_uint(t);
  const uint32_t r = u + 0x7FFFFu + ((u >> 20) & 1u);
  return (r >> 20) - (120u << 3);
}

__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
  for (int o = 32; o >= 1; o >>= 1) v = max(v, (uint32_t)__shfl_xor((int)v, o, 64));
  return v;
}

}  // namespace qk
