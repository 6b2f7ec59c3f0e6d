// Host-side construction of the NF4 code book and the encoder thresholds.
//
// NF4 (nlp-lineage milestone page on QLoRA, section "The idea", NF4 bullet):
// 16 values placed so that each covers an equal share of a standard normal
// distribution, one of them exactly zero.  The pages do not print the level
// formula; the construction used here places each side's levels at normal
// quantiles evenly spaced in probability between 1/2 and an outer probability
// delta = 1 - (1/32 + 1/30) / 2 (8 levels on the positive side, 7 on the
// negative side, plus zero), scaled so the outermost levels are exactly -1 and
// +1, then rounded once to fp32.  The inverse normal CDF is evaluated here by
// bisection on erfc in long double.
#include <algorithm>
#include <cmath>
#include <cstring>
#include <mutex>

#include "common.h"

namespace {

long double phi_inv(long double p) {
  long double lo = -12.0L, hi = 12.0L;
  for (int it = 0; it < 400; ++it) {
    long double mid = 0.5L * (lo + hi);
    if (mid == lo || mid == hi) break;
    long double cdf = 0.5L * std::erfc(-mid / std::sqrt(2.0L));
    if (cdf < p) lo = mid; else hi = mid;
  }
  return 0.5L * (lo + hi);
}

// Levels and the encoder thresholds: thr[k] is the smallest fp32 strictly
// above the midpoint of q[k] and q[k + 1] (exact in double).
Nf4Params from_levels(const float* q) {
  Nf4Params p;
  for (int k = 0; k < 16; ++k) p.q[k] = q[k];
  for (int k = 0; k < 15; ++k) {
    const double m = ((double)p.q[k] + (double)p.q[k + 1]) * 0.5;
    float f = (float)m;
    if ((double)f <= m) f = std::nextafter(f, 2.0f);
    p.thr[k] = f;
  }
  return p;
}

Nf4Params build() {
  const long double delta = 1.0L - 0.5L * (1.0L / 32.0L + 1.0L / 30.0L);
  const long double top = phi_inv(delta);
  long double v[16];
  int n = 0;
  for (int j = 0; j < 8; ++j) v[n++] = phi_inv(delta - j * (delta - 0.5L) / 8.0L) / top;
  for (int j = 0; j < 7; ++j) v[n++] = -phi_inv(delta - j * (delta - 0.5L) / 7.0L) / top;
  v[n++] = 0.0L;
  std::sort(v, v + 16);
  float q[16];
  for (int k = 0; k < 16; ++k) q[k] = (float)v[k];
  return from_levels(q);
}

// 4-bit float: OCP E2M1 (sign, 2 exponent bits with bias 1, 1 mantissa bit,
// exponent 0 subnormal) divided by its largest value 6.  4-bit integer: k / 7
// for k = -7..7.  Both have 15 distinct values; code 15 repeats +1 and is
// never the nearest (ties go to the smaller code).
Nf4Params build_fp4() {
  double v[16];
  int n = 0;
  for (int c = 0; c < 8; ++c) {               // non-negative patterns; the sign bit mirrors them
    const int e = (c >> 1) & 3, m = c & 1;
    const double mag = e == 0 ? 0.5 * m : (1.0 + 0.5 * m) * std::ldexp(1.0, e - 1);
    v[n++] = mag / 6.0;
    if (c) v[n++] = -mag / 6.0;
  }
  std::sort(v, v + 15);
  float q[16];
  for (int k = 0; k < 15; ++k) q[k] = (float)v[k];
  q[15] = 1.0f;
  return from_levels(q);
}

Nf4Params build_int4() {
  float q[16];
  for (int k = 0; k < 15; ++k) q[k] = (float)((k - 7) / 7.0);
  q[15] = 1.0f;
  return from_levels(q);
}

// Bucket table of the encoder.  Its approximate 16 n' is within 2^-22 |16 n|
// of 16 n (common.h); the table is accepted when that error stays below half
// the margin kNf4Near at every threshold (|t16| <= 16) and every threshold lies
// farther than four margins from its bucket's ends, so that a quotient placed
// in a neighbouring bucket still gets the right count.
Nf4Buckets build_buckets(const Nf4Params& p) {
  Nf4Buckets b;
  b.ok = 1;
  for (int i = 0; i < 34; ++i) {
    const double lo = i - 17, hi = i - 16;      // bucket covers 16 n in [lo, hi)
    int base = 0, inside = 0;
    float t = INFINITY;
    for (int k = 0; k < 15; ++k) {
      const double t16 = 16.0 * (double)p.thr[k];
      if (t16 <= lo) ++base;
      else if (t16 < hi) { ++inside; t = (float)t16; }
    }
    if (inside > 1) b.ok = 0;
    if (inside == 1) {
      const double m = (double)kNf4Near;
      if (2.0 * std::ldexp(std::fabs((double)t), -22) > m) b.ok = 0;
      if ((double)t - lo <= 4.0 * m || hi - (double)t <= 4.0 * m) b.ok = 0;
    }
    b.t16[i] = t;
    b.cnt[i] = (uint32_t)base;
  }
  return b;
}

}  // namespace

const Nf4Params& nf4_params() {
  static const Nf4Params p = build();
  return p;
}

const Nf4Buckets& nf4_buckets() {
  static const Nf4Buckets b = build_buckets(nf4_params());
  return b;
}

const Nf4Params* codebook_params(int codebook) {
  static const Nf4Params fp4 = build_fp4(), int4 = build_int4();
  switch (codebook) {
    case 0: return &nf4_params();
    case 1: return &fp4;
    case 2: return &int4;
    default: return nullptr;
  }
}
