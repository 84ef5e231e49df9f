// Host construction of the 4-bit levels and decision thresholds.
//
// Levels ("QLoRA: Fine-Tuning a 70B on One GPU", section "NF4 Quantization":
// a 16-entry table built from the normal CDF; inquiringlines note on QLoRA,
// mechanism paragraph: each bin an equal share of a zero-centred normal):
// 7 negative levels, an exact zero and 8 positive levels.  Each half sits at
// normal quantiles of equally spaced probabilities from 1/2 to P = 31/32 (the
// centre of the outermost sixteenth of the mass), scaled by 1/Phi^-1(P) so the
// ends are exactly -1 and +1.
//
// Phi^-1 here is Newton's method on Phi(x) = erfc(-x/sqrt 2)/2 started at 0;
// for p >= 1/2 Phi is concave on [0, inf), so the iterates rise monotonically
// to the root and stop when a step no longer moves x.
#include <cmath>
#include <cstring>
#include <mutex>

#include "launch.h"

namespace qnf4 {
namespace {

double normal_quantile_upper(double p) {  // p in [1/2, 1)
  const double inv_sqrt_2pi = 0.39894228040143267794;
  double x = 0.0;
  for (int it = 0; it < 200; ++it) {
    const double f = 0.5 * std::erfc(-x / std::sqrt(2.0)) - p;
    const double d = inv_sqrt_2pi * std::exp(-0.5 * x * x);
    const double nx = x - f / d;
    if (nx == x) break;
    if (it > 8 && std::fabs(nx - x) <= 2e-16 * std::fabs(x)) { x = nx; break; }
    x = nx;
  }
  return x;
}

NF4Tables build(int kind) {
  NF4Tables t;
  if (kind == kQuantInt4) {
    // the uniform table: k / 7 for the 4-bit integers k = -8..7 (section "NF4
    // Quantization: Beyond Standard INT4": 16 integer levels at uniform steps)
    for (int k = 0; k < 16; ++k) t.level[k] = (float)((double)(k - 8) / 7.0);
  } else {
    const double P = 31.0 / 32.0;
    const double z = normal_quantile_upper(P);
    t.level[7] = 0.0f;
    for (int j = 1; j <= 7; ++j) {
      const double p = 0.5 + (P - 0.5) * j / 7.0;
      t.level[7 - j] = (float)(-normal_quantile_upper(p) / z);
    }
    for (int j = 1; j <= 8; ++j) {
      const double p = 0.5 + (P - 0.5) * j / 8.0;
      t.level[7 + j] = (float)(normal_quantile_upper(p) / z);
    }
  }
  // thresholds: largest float <= exact midpoint (exact in double)
  for (int j = 0; j < 15; ++j) {
    const double m = 0.5 * ((double)t.level[j] + (double)t.level[j + 1]);
    float f = (float)m;
    if ((double)f > m) f = std::nextafterf(f, -INFINITY);
    t.thresh[j] = f;
  }
  // The quantiser finds codes through 256 buckets of [-1, 1]: bucket
  // floor(fma(x, 128, 128)), holding the count of thresholds below it and
  // the one threshold inside it.  Rounding is monotone, so a value can only
  // land one bucket too high, and only then miscount, if some threshold at
  // or above it sits below that bucket's edge: that needs a threshold t whose
  // own fma(t, 128, 128) rounds up onto an edge.  Exact when no threshold
  // does that and no bucket holds two thresholds.  (INT4 has one threshold
  // exactly on an edge, at 1/2, and one a float below another, at -1/2:
  // both exact.)
  t.bucket_ok = 1;
  int prev = -1000;
  for (int j = 0; j < 15; ++j) {
    const double u = 128.0 * (double)t.thresh[j] + 128.0;   // exact
    const float uf = std::fmaf(t.thresh[j], 128.0f, 128.0f);
    const int b = (int)std::floor(u);
    if ((int)std::floor((double)uf) != b) t.bucket_ok = 0;
    if (b == prev) t.bucket_ok = 0;
    prev = b;
  }
  return t;
}

}  // namespace

const NF4Tables& host_tables(int kind) {
  static NF4Tables tables[2];
  static std::once_flag once;
  std::call_once(once, [] {
    tables[kQuantNf4] = build(kQuantNf4);
    tables[kQuantInt4] = build(kQuantInt4);
  });
  return tables[kind == kQuantInt4 ? kQuantInt4 : kQuantNf4];
}

}  // namespace qnf4
