// NF4 blockwise-absmax encoder, double quantization of the block scales and
// the bit-exact dequantizer.
//
// Method: nlp-lineage milestone page on QLoRA, section "The idea" (NF4 bullet
// and double-quantisation bullet); inferensys glossary entry "QLoRA",
// double-quantization paragraph (scales quantised to 8-bit floats).
#include "kernels.h"

namespace {

constexpr int kThreads = 256;

// One thread encodes 8 consecutive weights; the 8 lanes of an aligned group
// cover one block of 64 and share its absmax through DPP.  Codes of the 8
// weights form one 32-bit word (element j in bits 4j..4j+3).
//
// The code of n = fl32(w / a) is #{k : n >= thr[k]}.  Instead of dividing and
// comparing with all 15 thresholds, each weight takes n' = w * (16 / a) from
// one reciprocal per block (within a few ulp of 16 n), finds its 1/16-wide
// bucket in a 34-entry LDS table (one 8-byte read: the bucket's threshold, a
// margin and the count of thresholds below the bucket), and compares once.
// Weights whose n' lies within the margin of the bucket's threshold -- and
// all weights of blocks with a nonzero finite absmax outside [2^-123, 2^125),
// where 16 / absmax would not be a finite normal number -- are redone with the
// correctly rounded division, so the codes are exactly those of the definition.
// The eight weights of a thread -> eight packed codes; `a` returns the block's
// absmax (shared by the 8 lanes of an aligned group through DPP, so all eight
// lanes of a block must be active together).  tab: the bucket table in LDS.
// floor(x) as int32 in one instruction (the compiler emits a floor and a
// conversion); non-finite x gives an out-of-range index that the caller clamps.
__device__ __forceinline__ int cvt_floor_i32(float x) {
  int r;
  asm("v_cvt_flr_i32_f32 %0, %1" : "=v"(r) : "v"(x));
  return r;
}

__device__ __forceinline__ uint32_t encode8(const float (&w)[8], const uint32_t* tab, uint32_t tab_base,
                                            float& a_out) {
  uint32_t m = 0;
#pragma unroll
  for (int j = 0; j < 8; ++j) m = max(m, __float_as_uint(w[j]) & 0x7FFFFFFFu);
  m = qk::dpp_max8(m);
  const float a = __uint_as_float(m);
  // 16 / a when it is a finite normal number, i.e. a in [2^-123, 2^125) (and, as
  // for any other input, for an infinite or NaN absmax); every other nonzero
  // absmax -- subnormal, or at either end of the normal range -- takes the exact
  // division below.  An all-zero block gives n' = 0 (codes 7).
  const bool a_fast = (m >= 0x02000000u && m < 0x7E000000u) || m >= 0x7F800000u;
  const float y16 = a_fast ? 16.0f * __builtin_amdgcn_rcpf(a) : 0.0f;
  uint32_t packed = 0;
  // a weight is near its bucket's threshold when |n16 - t16| <= margin, i.e. when
  // fl(|n16 - t16| - margin) <= 0 (exact: the difference of two floats is
  // non-positive exactly when the first is not larger); the octet is redone when
  // the smallest of the eight is.  A NaN difference never counts as near, as
  // before, since the minimum passes over it.
  float emin = __builtin_inff();
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const float n16 = w[j] * y16;
    // bucket floor(n16) + 17 in [1, 33] for finite weights; the unsigned min keeps
    // a non-finite input inside the table
    const uint32_t bi = min((uint32_t)(cvt_floor_i32(n16) + 17), 33u);
    const uint32_t addr = tab_base + 8u * bi;
    const float t16 = __uint_as_float(*(const LDS_AS uint32_t*)(uintptr_t)addr);
    const uint32_t mb = *(const LDS_AS uint32_t*)(uintptr_t)(addr + 4);
    const uint32_t c = (mb & 15u) + (n16 >= t16 ? 1u : 0u);
    emin = __builtin_fminf(emin, __builtin_fabsf(n16 - t16) - __uint_as_float(mb));
    packed |= c << (4 * j);
  }
  const bool redo = (m != 0 && !a_fast) || emin <= 0.0f;
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
      const uint32_t c = (tab[2 * bi + 1] & 15u) + (n16 >= t16 ? 1u : 0u);
      packed |= c << (4 * j);
    }
  }
  a_out = a;
  return packed;
}

struct RawOct {
  u32x4 v0, v1;
};

template <bool kBf16>
__device__ __forceinline__ RawOct load_oct(const void* __restrict__ W, int64_t o) {
  RawOct r;
  if (kBf16) {
    r.v0 = __builtin_nontemporal_load((const u32x4*)W + o);
    r.v1 = u32x4{0, 0, 0, 0};
  } else {
    r.v0 = __builtin_nontemporal_load((const u32x4*)W + 2 * o);
    r.v1 = __builtin_nontemporal_load((const u32x4*)W + 2 * o + 1);
  }
  return r;
}

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

template <bool kBf16>
__global__ __launch_bounds__(kThreads) void k_nf4_encode(const void* __restrict__ W, int64_t n_oct,
                                                         uint32_t* __restrict__ codes,
                                                         float* __restrict__ absmax, Nf4Buckets bk) {
  __shared__ __attribute__((aligned(8))) uint32_t tab[34 * 2];
  if (threadIdx.x < 34) {
    tab[2 * threadIdx.x] = __float_as_uint(bk.t16[threadIdx.x]);
    tab[2 * threadIdx.x + 1] = bk.mb[threadIdx.x];
  }
  __syncthreads();
  const uint32_t tab_base = (uint32_t)(uintptr_t)(LDS_AS uint32_t*)tab;
  const int64_t stride = (int64_t)gridDim.x * kThreads;
  for (int64_t o = (int64_t)blockIdx.x * kThreads + threadIdx.x; o < n_oct; o += stride) {
    float w[8];
    unpack_oct<kBf16>(load_oct<kBf16>(W, o), w);
    float a;
    codes[o] = encode8(w, tab, tab_base, a);
    if ((threadIdx.x & 7) == 0) absmax[o >> 3] = a;
  }
}

// Encoder and double quantization in one pass: a work group owns whole groups
// of 256 blocks (2048 octets, eight per thread, all requested up front); the
// group's max is reduced across the work group and every block's scale code
// follows at once.  Results equal those of k_nf4_encode then k_double_quant.
template <bool kBf16>
__global__ __launch_bounds__(kThreads) void k_nf4_encode_dq(const void* __restrict__ W, int64_t n_oct,
                                                            uint32_t* __restrict__ codes,
                                                            float* __restrict__ absmax, uint8_t* __restrict__ c2,
                                                            float* __restrict__ c1, int64_t ngroups,
                                                            Nf4Buckets bk) {
  __shared__ __attribute__((aligned(8))) uint32_t tab[34 * 2];
  __shared__ uint32_t red[kThreads / 64];
  if (threadIdx.x < 34) {
    tab[2 * threadIdx.x] = __float_as_uint(bk.t16[threadIdx.x]);
    tab[2 * threadIdx.x + 1] = bk.mb[threadIdx.x];
  }
  __syncthreads();
  const uint32_t tab_base = (uint32_t)(uintptr_t)(LDS_AS uint32_t*)tab;
  const int t = threadIdx.x;
  constexpr int kIt = qk::kGroup * 8 / kThreads;    // octets per thread per group (8)
  for (int64_t g = blockIdx.x; g < ngroups; g += gridDim.x) {
    const int64_t o0 = g * qk::kGroup * 8 + t;
    RawOct raw[kIt];
#pragma unroll
    for (int it = 0; it < kIt; ++it) {
      const int64_t o = o0 + (int64_t)it * kThreads;
      raw[it] = load_oct<kBf16>(W, o < n_oct ? o : 0);
    }
    float a[kIt];
    uint32_t m = 0;
#pragma unroll
    for (int it = 0; it < kIt; ++it) {
      const int64_t o = o0 + (int64_t)it * kThreads;
      a[it] = 0.0f;
      if (o < n_oct) {                                // whole blocks (8 lanes) are in or out together
        float w[8];
        unpack_oct<kBf16>(raw[it], w);
        codes[o] = encode8(w, tab, tab_base, a[it]);
      }
      m = max(m, __float_as_uint(a[it]));
    }
    m = qk::wave_max_u32(m);
    if ((t & 63) == 0) red[t >> 6] = m;
    __syncthreads();
    uint32_t gm = red[0];
#pragma unroll
    for (int i = 1; i < kThreads / 64; ++i) gm = max(gm, red[i]);
    __syncthreads();                                  // red is reused by the next group
    const float cmax = __uint_as_float(gm);
    if ((t & 7) == 0) {
#pragma unroll
      for (int it = 0; it < kIt; ++it) {
        const int64_t o = o0 + (int64_t)it * kThreads;
        if (o < n_oct) {
          const int64_t b = o >> 3;
          c2[b] = (uint8_t)qk::e4m3fn_encode(gm == 0 ? 0.0f : a[it] / cmax);
          if (absmax) absmax[b] = a[it];
        }
      }
    }
    if (t == 0) c1[g] = cmax;
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
  const int grid = grid_for(n_oct, kThreads);
  if (!nf4_buckets().ok) return hipErrorInvalidValue;   // table assumptions (checked once on the host)
  if (bf16)
    hipLaunchKernelGGL(k_nf4_encode<true>, dim3(grid), dim3(kThreads), 0, s, W, n_oct, (uint32_t*)codes, absmax,
                       nf4_buckets());
  else
    hipLaunchKernelGGL(k_nf4_encode<false>, dim3(grid), dim3(kThreads), 0, s, W, n_oct, (uint32_t*)codes, absmax,
                       nf4_buckets());
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
