// Lloyd-Max levels of the standard normal density for the TurboQuant codec
// (host only).  The page "hipfire：为AMD RDNA GPU打造的Rust原生LLM推理引擎",
// section "3. TurboQuant KV缓存压缩", quantises each rotated coordinate to
// Lloyd-Max centroids; here they are the fixed point of the two optimality
// conditions -- each threshold halfway between its neighbouring levels, each
// level the mean of the density over its cell -- reached by iterating both
// from equally probable cells.  The cell mean of N(0,1) over (a, b) is
// (phi(a) - phi(b)) / (Phi(b) - Phi(a)).
#include <cmath>
#include <vector>

#include "turbo.h"

namespace hq {
namespace {

double pdf(double x) { return std::exp(-0.5 * x * x) / std::sqrt(2.0 * M_PI); }
double cdf(double x) { return 0.5 * std::erfc(-x / std::sqrt(2.0)); }

double cell_mean(double a, double b) {
  const double pa = std::isinf(a) ? 0.0 : pdf(a), pb = std::isinf(b) ? 0.0 : pdf(b);
  const double Pa = std::isinf(a) ? 0.0 : cdf(a), Pb = std::isinf(b) ? 1.0 : cdf(b);
  return (pa - pb) / (Pb - Pa);
}

// x with cdf(x) = p, by bisection
double quantile(double p) {
  double lo = -40.0, hi = 40.0;
  for (int i = 0; i < 200; ++i) {
    const double mid = 0.5 * (lo + hi);
    (cdf(mid) < p ? lo : hi) = mid;
  }
  return 0.5 * (lo + hi);
}

}  // namespace

void lloyd_max_normal(int bits, double* levels) {
  const int L = 1 << bits;
  std::vector<double> edge(L + 1);
  edge[0] = -INFINITY;
  edge[L] = INFINITY;
  for (int j = 1; j < L; ++j) edge[j] = quantile((double)j / L);
  for (int j = 0; j < L; ++j) levels[j] = cell_mean(edge[j], edge[j + 1]);
  for (int it = 0; it < 20000; ++it) {
    for (int j = 1; j < L; ++j) edge[j] = 0.5 * (levels[j - 1] + levels[j]);
    double moved = 0.0;
    for (int j = 0; j < L; ++j) {
      const double m = cell_mean(edge[j], edge[j + 1]);
      moved = std::fmax(moved, std::fabs(m - levels[j]));
      levels[j] = m;
    }
    if (moved < 1e-14) break;
  }
}

void turbo_table(int n, int bits, TurboTable* t) {
  const int L = 1 << bits;
  double lv[256];
  lloyd_max_normal(bits, lv);
  const double sc = 1.0 / std::sqrt((double)n);
  for (int j = 0; j < 256; ++j) t->cent[j] = j < L ? (float)(lv[j] * sc) : 0.f;
  for (int j = 0; j < 255; ++j)
    t->thr[j] = j < L - 1 ? (float)(0.5 * ((double)t->cent[j] + (double)t->cent[j + 1])) : INFINITY;
  // buckets for the encoder's search: turbo_lut_buckets(bits) - 2 across the
  // thresholds (thr[0] near bucket 1, thr[L - 2] near the last), each
  // narrower than half the smallest gap between two thresholds, so no two
  // thresholds share a bucket even after rounding (the kernel checks)
  const double lo = t->thr[0], hi = t->thr[L - 2];
  double gap = INFINITY;
  for (int j = 0; j + 1 < L - 1; ++j) gap = std::fmin(gap, (double)t->thr[j + 1] - (double)t->thr[j]);
  const double w = (hi - lo) / (turbo_lut_buckets(bits) - 2);
  t->lut_a = 0.f;
  t->lut_b = 0.f;
  t->lut_ok = 0;
  if (w > 0.0 && 2.0 * w < gap) {
    t->lut_a = (float)(1.0 / w);
    t->lut_b = (float)(1.0 - lo / w);
    t->lut_ok = 1;
  }
}

}  // namespace hq
