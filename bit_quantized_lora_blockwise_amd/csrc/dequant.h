// Dequantisation of one 64-weight block held in registers, shared by the fused
// GEMMs (gemm_big.hip) and the decode kernels (decode.hip): the block's sixteen
// values W'(v) = bf16(fl32(q[v] s')) (examadda page, "The Core Idea": the base
// is dequantised on the fly; rounding as the double-dequantisation of the
// nlp-lineage milestone page, "The idea") are built once as two byte planes and
// each 4-bit code is looked up with v_perm_b32, three byte selects per four
// codes and plane.
#pragma once

#include "common.h"

namespace nf4 {

// One block's table: byte planes, lo[j] byte i = low byte of W'(4 j + i), hi likewise.
struct BlockLut {
  uint32_t lo[4], hi[4];
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

// The constants materialised in VGPRs (a kernel does this once).
__device__ __forceinline__ SplitConst split_const() {
  SplitConst k;
  asm volatile("v_mov_b32 %0, 0x04040404" : "=v"(k.m4));
  asm volatile("v_mov_b32 %0, 0x03020100" : "=v"(k.b0));
  return k;
}

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

// Byte-plane lookups of the even elements (le, he) and odd elements (lo, ho).
struct Planes {
  uint32_t le, he, lo, ho;
};

__device__ __forceinline__ Planes lookup8(const BlockLut& L, uint32_t c, const SplitConst& k) {
  const Split sp = split8(c, k);
  Planes P;
  P.le = lut16(L.lo, sp.xe, sp.se);
  P.he = lut16(L.hi, sp.xe, sp.se);
  P.lo = lut16(L.lo, sp.xo, sp.so);
  P.ho = lut16(L.hi, sp.xo, sp.so);
  return P;
}

// Eight nibbles -> four packed bf16 pairs in element order (e0 e1, e2 e3, e4 e5, e6 e7).
__device__ __forceinline__ u32x4 dequant8(const BlockLut& L, uint32_t c, const SplitConst& k) {
  const Planes P = lookup8(L, c, k);
  const uint32_t e02 = __builtin_amdgcn_perm(P.he, P.le, 0x05010400u);   // [W'(e0), W'(e2)]
  const uint32_t e46 = __builtin_amdgcn_perm(P.he, P.le, 0x07030602u);   // [W'(e4), W'(e6)]
  const uint32_t o13 = __builtin_amdgcn_perm(P.ho, P.lo, 0x05010400u);   // [W'(e1), W'(e3)]
  const uint32_t o57 = __builtin_amdgcn_perm(P.ho, P.lo, 0x07030602u);   // [W'(e5), W'(e7)]
  u32x4 r;
  r[0] = __builtin_amdgcn_perm(o13, e02, 0x05040100u);   // e0, e1
  r[1] = __builtin_amdgcn_perm(o13, e02, 0x07060302u);   // e2, e3
  r[2] = __builtin_amdgcn_perm(o57, e46, 0x05040100u);   // e4, e5
  r[3] = __builtin_amdgcn_perm(o57, e46, 0x07060302u);   // e6, e7
  return r;
}

// Eight nibbles -> weights in the order (0, 2, 4, 6, 1, 3, 5, 7) of the word.
__device__ __forceinline__ u32x4 dequant8_eo(const BlockLut& L, uint32_t c, const SplitConst& k) {
  const Planes P = lookup8(L, c, k);
  u32x4 r;
  r[0] = __builtin_amdgcn_perm(P.he, P.le, 0x05010400u);   // W'(e0), W'(e2)
  r[1] = __builtin_amdgcn_perm(P.he, P.le, 0x07030602u);   // W'(e4), W'(e6)
  r[2] = __builtin_amdgcn_perm(P.ho, P.lo, 0x05010400u);   // W'(e1), W'(e3)
  r[3] = __builtin_amdgcn_perm(P.ho, P.lo, 0x07030602u);   // W'(e5), W'(e7)
  return r;
}

// Eight nibbles -> the low and high bytes of their bf16 values, each as eight
// bytes in the element order (0, 2, 4, 6, 1, 3, 5, 7).
__device__ __forceinline__ void dequant8_planes(const BlockLut& L, uint32_t c, const SplitConst& k, u32x2& lo8,
                                                u32x2& hi8) {
  const Planes P = lookup8(L, c, k);
  lo8 = u32x2{P.le, P.lo};
  hi8 = u32x2{P.he, P.ho};
}

}  // namespace nf4
