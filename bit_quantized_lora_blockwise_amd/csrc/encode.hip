// NF4 blockwise-absmax encoder, double quantization of the block scales and
// the bit-exact dequantizer.
//
// Method: nlp-lineage milestone page on QLoRA, section "The idea" (NF4 bullet
// and double-quantisation bullet); inferensys glossary entry "QLoRA",
// double-quantization paragraph (scales quantised to 8-bit floats).
#include "kernels.h"

namespace {

constexpr int kThreads = 256;
constexpr int kNT = 2;   // cache policy of the weight loads: nontemporal (each weight is read once)

__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void* p, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, (int)bytes, 0x00020000);
}

// 8 * floor(x) as int32 for the bucket address: one conversion (which
// saturates NaN and +-inf to INT_MAX / INT_MIN) and one 24-bit signed multiply
// (which reads the low 24 bits of its input).  Every finite x of the encoder has
// |x| <= 16 (1 + 2^-22), so floor(x) is in [-17, 16] and the result 8 floor(x)
// exactly; INT_MAX and INT_MIN give -8 and 0, still inside the table, so no
// clamp is needed.
__device__ __forceinline__ int bucket_offset(float x) {
  int r;
  asm("v_cvt_flr_i32_f32 %0, %1\n\tv_mul_i32_i24 %0, 8, %0" : "=v"(r) : "v"(x));
  return r;
}

struct RawOct {
  u32x4 v0, v1;
};

template <bool kBf16>
__device__ __forceinline__ void unpack_oct(const RawOct& r, float (&w)[8]) {
  if (kBf16) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      w[2 * j] = __uint_as_float(r.v0[j] << 16);
      w[2 * j + 1] = __uint_as_float(r.v0[j] & 0xFFFF0000u);
    }
  } else {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      w[j] = __uint_as_float(r.v0[j]);
      w[4 + j] = __uint_as_float(r.v1[j]);
    }
  }
}

// The largest |w| of the octet as fp32 bits (NaN above +inf).  For bf16 the
// 16-bit magnitudes of each word's two weights are compared in pairs (one
// packed max per word) and the larger half is moved to the top.
template <bool kBf16>
__device__ __forceinline__ uint32_t oct_absmax_bits(const RawOct& r) {
  if (kBf16) {
    typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));
    u16x2 h = __builtin_bit_cast(u16x2, r.v0[0] & 0x7FFF7FFFu);
#pragma unroll
    for (int j = 1; j < 4; ++j) h = __builtin_elementwise_max(h, __builtin_bit_cast(u16x2, r.v0[j] & 0x7FFF7FFFu));
    return (uint32_t)max(h.x, h.y) << 16;
  } else {
    uint32_t m = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) m = max(m, max(r.v0[j] & 0x7FFFFFFFu, r.v1[j] & 0x7FFFFFFFu));
    return m;
  }
}

// One thread encodes 8 consecutive weights; the 8 lanes of an aligned group
// cover one block of 64 and share its absmax through DPP.  Codes of the 8
// weights form one 32-bit word (element j in bits 4j..4j+3).
//
// The code of n = fl32(w / a) is #{k : n >= thr[k]}.  Instead of dividing and
// comparing with all 15 thresholds, each weight takes n' = w * (16 / a) from
// one reciprocal per block (within a few ulp of 16 n), finds its 1/16-wide
// bucket in a 34-entry LDS table (one 8-byte read: the bucket's threshold t16
// and the count of thresholds below the bucket), and compares once.  Weights
// whose 16 n' lies within kNf4Near of the bucket's threshold -- and
// all weights of blocks with a nonzero finite absmax outside [2^-123, 2^125),
// where 16 / absmax would not be a finite normal number -- are redone with the
// correctly rounded division, so the codes are exactly those of the definition.
// The eight weights of a thread -> eight packed codes; `a` returns the block's
// absmax (shared by the 8 lanes of an aligned group through DPP, so all eight
// lanes of a block must be active together).  tab: the bucket table in LDS,
// tab_base its LDS byte address.
template <bool kBf16>
__device__ __forceinline__ uint32_t encode8(const RawOct& r, const uint32_t* tab, uint32_t tab_base,
                                            float& a_out) {
  float w[8];
  unpack_oct<kBf16>(r, w);
  const uint32_t m = qk::dpp_max8(oct_absmax_bits<kBf16>(r));
  const float a = __uint_as_float(m);
  // 16 / a when it is a finite normal number, i.e. a in [2^-123, 2^125) (and, as
  // for any other input, for an infinite or NaN absmax); every other nonzero
  // absmax -- subnormal, or at either end of the normal range -- takes the exact
  // division below.  An all-zero block gives n' = 0 (codes 7).
  const bool a_fast = (m >= 0x02000000u && m < 0x7E000000u) || m >= 0x7F800000u;
  const float y16 = a_fast ? 16.0f * __builtin_amdgcn_rcpf(a) : 0.0f;
  // With d = 16 n' - t16: 16 n' >= t16 exactly when d >= 0 (the difference of
  // two floats is non-negative exactly when the first is not smaller); the
  // octet is redone when the smallest |d| of its eight weights is at most
  // kNf4Near (a bucket without threshold gives |d| = +inf, never near; a NaN d
  // from a NaN weight is passed over by the minimum).  The codes are gathered
  // from the last weight down, four bits at a time.
  float emin = __builtin_inff();
  uint32_t packed = 0;
#pragma unroll
  for (int j = 7; j >= 0; --j) {
    const float n16 = w[j] * y16;
    // bucket floor(n16) + 17 in [0, 33]: the +17 is folded into the address
    const uint32_t addr = tab_base + 8u * 17u + (uint32_t)bucket_offset(n16);
    const float t16 = __uint_as_float(*(const LDS_AS uint32_t*)(uintptr_t)addr);
    const uint32_t cnt = *(const LDS_AS uint32_t*)(uintptr_t)(addr + 4);
    const float d = n16 - t16;
    emin = __builtin_fminf(emin, __builtin_fabsf(d));
    packed = (packed << 4) + cnt + (d >= 0.0f ? 1u : 0u);
  }
  const bool redo = (m != 0 && !a_fast) || emin <= kNf4Near;
  if (redo) {
    // correctly rounded quotients for the whole octet (the same codes wherever
    // the approximate one was decided)
    packed = 0;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const float n = (m == 0) ? 0.0f : w[j] / a;
      const float n16 = 16.0f * n;                            // exact
      const int bi = min(max((int)__builtin_floorf(n16) + 17, 0), 33);
      const float t16 = __uint_as_float(tab[2 * bi]);
      const uint32_t c = tab[2 * bi + 1] + (n16 >= t16 ? 1u : 0u);
      packed |= c << (4 * j);
    }
  }
  a_out = a;
  return packed;
}

// Encoder, with double quantization in the same pass (kDq): a work group owns
// whole groups of 256 blocks (2048 octets, eight per thread, all requested up
// front).  With kDq the group's max is reduced across the work group, the
// blocks' absmax values are parked in LDS, and each thread then forms one
// block's scale code (the results equal those of the encoder alone followed by
// k_double_quant); without it each block's absmax is written as it is found.
template <bool kBf16, bool kDq = true>
__global__ __launch_bounds__(kThreads) void k_nf4_encode_dq(const void* __restrict__ W, int64_t n_oct,
                                                            uint32_t* __restrict__ codes,
                                                            float* __restrict__ absmax, uint8_t* __restrict__ c2,
                                                            float* __restrict__ c1, int64_t ngroups,
                                                            Nf4Buckets bk) {
  // one LDS array with the bucket table first, at LDS address 0 (its addresses
  // are then 8 bi plus a constant offset), then the wave maxima and the group's
  // block absmax values
  __shared__ __attribute__((aligned(16))) uint32_t lds[34 * 2 + kThreads / 64 + qk::kGroup];
  uint32_t* tab = lds;
  uint32_t* red = lds + 34 * 2;
  float* absm = (float*)(lds + 34 * 2 + kThreads / 64);
  if (threadIdx.x < 34) {
    tab[2 * threadIdx.x] = __float_as_uint(bk.t16[threadIdx.x]);
    tab[2 * threadIdx.x + 1] = bk.cnt[threadIdx.x];
  }
  __syncthreads();
  const uint32_t tab_base = (uint32_t)(uintptr_t)(LDS_AS uint32_t*)tab;
  const int t = threadIdx.x;
  constexpr int kIt = qk::kGroup * 8 / kThreads;    // octets per thread per group (8)
  constexpr uint32_t kOctB = kBf16 ? 16u : 32u;     // bytes of weights per octet
  for (int64_t g = blockIdx.x; g < ngroups; g += gridDim.x) {
    // the group's weights and codes through descriptors based at its first
    // octet and sized to its octets (fewer in the last group): loads past the
    // end return zeros (blocks of zeros, absmax 0, codes that are not kept) and
    // stores past the end are dropped, so no lane needs a branch or a 64-bit
    // address
    const int64_t ob = g * qk::kGroup * 8;
    const uint32_t noct = (uint32_t)min(n_oct - ob, (int64_t)(qk::kGroup * 8));
    const __amdgpu_buffer_rsrc_t rw = rsrc((const char*)W + ob * kOctB, noct * kOctB);
    const __amdgpu_buffer_rsrc_t rc = rsrc(codes + ob, 4u * noct);
    RawOct raw[kIt];
#pragma unroll
    for (int it = 0; it < kIt; ++it) {
      raw[it].v0 = __builtin_amdgcn_raw_buffer_load_b128(rw, kOctB * t, kOctB * kThreads * it, kNT);
      raw[it].v1 = kBf16 ? u32x4{0, 0, 0, 0}
                         : __builtin_amdgcn_raw_buffer_load_b128(rw, kOctB * t + 16, kOctB * kThreads * it, kNT);
    }
    uint32_t m = 0;
#pragma unroll
    for (int it = 0; it < kIt; ++it) {
      float a;
      const uint32_t packed = encode8<kBf16>(raw[it], tab, tab_base, a);
      __builtin_amdgcn_raw_buffer_store_b32(packed, rc, 4 * t, 4 * kThreads * it, 0);
      if (!kDq) {
        // block (t / 8) + 32 it of the group, dropped past the end
        if ((t & 7) == 0)
          __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(a), rsrc(absmax + g * qk::kGroup, noct / 2),
                                                (uint32_t)(t >> 3) * 4u, 128u * it, 0);
        continue;
      }
      if ((t & 7) == 0) absm[(t >> 3) + 32 * it] = a; // block (t / 8) + 32 it of the group
      m = max(m, __float_as_uint(a));
    }
    if (!kDq) continue;
    m = qk::wave_max_u32(m);
    if ((t & 63) == 0) red[t >> 6] = m;
    __syncthreads();
    uint32_t gm = red[0];
#pragma unroll
    for (int i = 1; i < kThreads / 64; ++i) gm = max(gm, red[i]);
    const float cmax = __uint_as_float(gm);
    // one block per thread; blocks past the end are dropped by the descriptors
    const uint32_t nb = noct / 8;
    const float a = absm[t];
    __builtin_amdgcn_raw_buffer_store_b8((uint8_t)qk::e4m3fn_encode(gm == 0 ? 0.0f : a / cmax),
                                         rsrc(c2 + g * qk::kGroup, nb), t, 0, 0);
    if (absmax)
      __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(a), rsrc(absmax + g * qk::kGroup, 4u * nb), 4 * t, 0, 0);
    if (t == 0) c1[g] = cmax;
    __syncthreads();                                  // red and absm are reused by the next group
  }
}

// One wavefront per group of 256 scales; lane l owns scales 4l..4l+3.
__global__ __launch_bounds__(kThreads) void k_double_quant(const float* __restrict__ absmax, int64_t nb,
                                                           uint8_t* __restrict__ c2, float* __restrict__ c1,
                                                           int64_t ngroups) {
  const int lane = threadIdx.x & 63;
  const int64_t wstride = (int64_t)gridDim.x * (kThreads / 64);
  for (int64_t g = (int64_t)blockIdx.x * (kThreads / 64) + (threadIdx.x >> 6); g < ngroups; g += wstride) {
    const int64_t base = g * qk::kGroup + 4 * lane;
    float v[4];
    uint32_t m = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      v[j] = (base + j < nb) ? absmax[base + j] : 0.0f;
      m = max(m, __float_as_uint(v[j]));
    }
    m = qk::wave_max_u32(m);
    const float cmax = __uint_as_float(m);
    if (lane == 0) c1[g] = cmax;
    uint32_t packed = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float t = (m == 0) ? 0.0f : v[j] / cmax;
      packed |= qk::e4m3fn_encode(t) << (8 * j);
    }
    if (base + 4 <= nb) {
      *(uint32_t*)(c2 + base) = packed;
    } else {
      for (int j = 0; j < 4; ++j)
        if (base + j < nb) c2[base + j] = (uint8_t)(packed >> (8 * j));
    }
  }
}

// W'[e] = bf16(fl32(q[code_e] * s'_b)), s'_b = fl32(dec(c2_b) * c1_{b/256}).
// One thread per 8 elements (one 32-bit word of codes -> 16 bytes of bf16).
__global__ __launch_bounds__(kThreads) void k_dequant(const uint32_t* __restrict__ codes,
                                                      const uint8_t* __restrict__ c2,
                                                      const float* __restrict__ c1, int64_t n_oct,
                                                      u32x4* __restrict__ out, Nf4Params p) {
  __shared__ float q[16];
  if (threadIdx.x < 16) q[threadIdx.x] = p.q[threadIdx.x];
  __syncthreads();
  const int64_t stride = (int64_t)gridDim.x * kThreads;
  for (int64_t o = (int64_t)blockIdx.x * kThreads + threadIdx.x; o < n_oct; o += stride) {
    const int64_t b = o >> 3;
    const float s = qk::e4m3fn_to_f32(c2[b]) * c1[b >> 8];
    const uint32_t cw = codes[o];
    u32x4 r;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float lo = q[(cw >> (8 * j)) & 15] * s;
      const float hi = q[(cw >> (8 * j + 4)) & 15] * s;
      r[j] = qk::pack_bf16x2(lo, hi);
    }
    out[o] = r;
  }
}

int grid_for(int64_t items, int per_block) {
  int64_t g = (items + per_block - 1) / per_block;
  if (g > 8192) g = 8192;
  if (g < 1) g = 1;
  return (int)g;
}

}  // namespace

hipError_t launch_nf4_encode(const void* W, bool bf16, int64_t elems, uint8_t* codes, float* absmax,
                             hipStream_t s) {
  const int64_t n_oct = elems / 8;
  const int64_t ngroups = (elems / qk::kBlock + qk::kGroup - 1) / qk::kGroup;
  if (!nf4_buckets().ok) return hipErrorInvalidValue;   // table assumptions (checked once on the host)
  const unsigned grid = (unsigned)(ngroups < 65536 ? ngroups : 65536);
  if (bf16)
    hipLaunchKernelGGL((k_nf4_encode_dq<true, false>), dim3(grid), dim3(kThreads), 0, s, W, n_oct, (uint32_t*)codes,
                       absmax, nullptr, nullptr, ngroups, nf4_buckets());
  else
    hipLaunchKernelGGL((k_nf4_encode_dq<false, false>), dim3(grid), dim3(kThreads), 0, s, W, n_oct, (uint32_t*)codes,
                       absmax, nullptr, nullptr, ngroups, nf4_buckets());
  return hipGetLastError();
}

hipError_t launch_double_quant(const float* absmax, int64_t n_blocks, uint8_t* c2, float* c1, hipStream_t s) {
  const int64_t ngroups = (n_blocks + qk::kGroup - 1) / qk::kGroup;
  const int grid = grid_for(ngroups, kThreads / 64);
  hipLaunchKernelGGL(k_double_quant, dim3(grid), dim3(kThreads), 0, s, absmax, n_blocks, c2, c1, ngroups);
  return hipGetLastError();
}

hipError_t launch_dequant(const uint8_t* codes, const uint8_t* c2, const float* c1, int64_t elems, uint16_t* out,
                          hipStream_t s) {
  const int64_t n_oct = elems / 8;
  const int grid = grid_for(n_oct, kThreads);
  hipLaunchKernelGGL(k_dequant, dim3(grid), dim3(kThreads), 0, s, (const uint32_t*)codes, c2, c1, n_oct,
                     (u32x4*)out, nf4_params());
  return hipGetLastError();
}

hipError_t launch_nf4_encode_dq(const void* W, bool bf16, int64_t elems, uint8_t* codes, float* absmax, uint8_t* c2,
                                float* c1, hipStream_t s) {
  const int64_t n_oct = elems / 8;
  const int64_t nblocks = elems / qk::kBlock;
  const int64_t ngroups = (nblocks + qk::kGroup - 1) / qk::kGroup;
  if (!nf4_buckets().ok) return hipErrorInvalidValue;
  const unsigned grid = (unsigned)(ngroups < 65536 ? ngroups : 65536);
  if (bf16)
    hipLaunchKernelGGL(k_nf4_encode_dq<true>, dim3(grid), dim3(kThreads), 0, s, W, n_oct, (uint32_t*)codes, absmax,
                       c2, c1, ngroups, nf4_buckets());
  else
    hipLaunchKernelGGL(k_nf4_encode_dq<false>, dim3(grid), dim3(kThreads), 0, s, W, n_oct, (uint32_t*)codes, absmax,
                       c2, c1, ngroups, nf4_buckets());
  return hipGetLastError();
}
