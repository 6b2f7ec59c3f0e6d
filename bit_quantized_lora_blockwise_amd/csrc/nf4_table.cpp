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

Nf4Params build() {
  Nf4Params p;
  const long double delta = 1.0L - 0.5L * (1.0L / 32.0L + 1.0L / 30.0L);
  const long double top = phi_inv(delta);
  long double v[16];
  int n = 0;
  for (int j = 0; j < 8; ++j) v[n++] = phi_inv(delta - j * (delta - 0.5L) / 8.0L) / top;
  for (int j = 0; j < 7; ++j) v[n++] = -phi_inv(delta - j * (delta - 0.5L) / 7.0L) / top;
  v[n++] = 0.0L;
  std::sort(v, v + 16);
  for (int k = 0; k < 16; ++k) p.q[k] = (float)v[k];
  for (int k = 0; k < 15; ++k) {
    // midpoint of two fp32 levels: exact in double
    double m = ((double)p.q[k] + (double)p.q[k + 1]) * 0.5;
    float f = (float)m;
    if ((double)f <= m) f = std::nextafter(f, 2.0f);
    p.thr[k] = f;
  }
  return p;
}

}  // namespace

const Nf4Params& nf4_params() {
  static const Nf4Params p = build();
  return p;
}
