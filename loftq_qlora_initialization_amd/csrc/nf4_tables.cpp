// NF4 levels, decision thresholds and the encode grid, built once on the host.
//
// NF4 is a quantile quantizer for normally distributed weights: its levels are
// values of the standard normal quantile function ("QLoRA论文概述", NF4 bullet and
// the related blurb on quantile quantization), listed ascending from -1 to 1 on
// "QLoRA技术解析：量化与低秩适配在LLM微调中的突破" §2.1.  Levels: 8 positive values
// Phi^-1 at 9 evenly spaced probabilities from delta to 1/2 (the last, 1/2,
// dropped), 7 negative values -Phi^-1 at 8 evenly spaced probabilities from delta
// to 1/2 (last dropped), an exact zero, all divided by the largest magnitude;
// delta = 1 - (1/32 + 1/30)/2.  Nearest-level rounding (ties to the lower level)
// is decided against the midpoints of neighbouring levels, as the CUDA-matching
// re-implementation blurbed on "QLoRA论文概述" does.
#include <algorithm>
#include <cmath>
#include <cstring>
#include <limits>
#include <mutex>

#include "internal.h"

namespace loftq {
namespace {

double normal_cdf(double x) { return 0.5 * std::erfc(-x / std::sqrt(2.0)); }
double normal_pdf(double x) { return std::exp(-0.5 * x * x) / std::sqrt(2.0 * M_PI); }

// Phi^-1(p) for p in [1/2, 1) by Newton's method on Phi(x) - p from x = 0.
// Phi is concave on x > 0, so the iterates increase monotonically to the root.
double normal_quantile_upper(double p) {
  if (p == 0.5) return 0.0;
  double x = 0.0;
  for (int it = 0; it < 200; ++it) {
    double step = (normal_cdf(x) - p) / normal_pdf(x);
    double nx = x - step;
    if (nx == x || std::fabs(step) <= 1e-17 * std::fabs(nx)) { x = nx; break; }
    x = nx;
  }
  return x;
}

Nf4Tables build() {
  Nf4Tables t;
  std::memset(&t, 0, sizeof(t));
  const double delta = 1.0 - 0.5 * (1.0 / 32.0 + 1.0 / 30.0);
  double v[16];
  int n = 0;
  const double step9 = (0.5 - delta) / 8.0, step8 = (0.5 - delta) / 7.0;
  for (int i = 0; i < 8; ++i) v[n++] = normal_quantile_upper(delta + i * step9);
  for (int i = 0; i < 7; ++i) v[n++] = -normal_quantile_upper(delta + i * step8);
  v[n++] = 0.0;
  std::sort(v, v + 16);
  double vmax = 0.0;
  for (double x : v) vmax = std::max(vmax, std::fabs(x));
  for (int i = 0; i < 16; ++i) t.level[i] = static_cast<float>(v[i] / vmax);

  // Threshold j: the largest fp32 not above the exact midpoint m_j.  For any
  // fp32 x, x > thr[j] exactly when x > m_j (equality at m_j goes to the lower
  // level, i.e. argmin-first).
  double thr[15];
  for (int j = 0; j < 15; ++j) {
    double m = 0.5 * (static_cast<double>(t.level[j]) + static_cast<double>(t.level[j + 1]));
    float f = static_cast<float>(m);
    if (static_cast<double>(f) > m) f = std::nextafter(f, -std::numeric_limits<float>::infinity());
    t.thr[j] = f;
    thr[j] = f;
  }

  // Encode grid: 32 cells of width 1/16 over [-1, 1) plus cell 32 for x >= 1.
  // Invariants the kernel relies on: at most one threshold per cell, and every
  // threshold at least `margin` from its cell's edges (the cell index computed in
  // fp32 may be off by one only for x within ~2^-22 of an edge).
  const double margin = 1.0 / 4096.0;
  bool ok = true;
  for (int g = 0; g < 33; ++g) {
    t.cell_thr[g] = std::numeric_limits<float>::infinity();
    t.cell_base[g] = 0;
  }
  for (int g = 0; g < 33; ++g) {
    double lo = -1.0 + g / 16.0, hi = -1.0 + (g + 1) / 16.0;
    int inside = 0, below = 0;
    for (int j = 0; j < 15; ++j) {
      if (thr[j] < lo) {
        ++below;
      } else if (g < 32 && thr[j] < hi) {
        ++inside;
        t.cell_thr[g] = static_cast<float>(thr[j]);
        if (thr[j] - lo < margin || hi - thr[j] < margin) ok = false;
      }
    }
    if (inside > 1) ok = false;
    t.cell_base[g] = below;
  }
  // The encoder compares y = 16 x + 16 (computed in fp32) with fl32(16 thr + 16).
  for (int g = 0; g < 33; ++g)
    t.cell_thr16[g] = std::isinf(t.cell_thr[g]) ? t.cell_thr[g]
                                                : static_cast<float>(16.0 * static_cast<double>(t.cell_thr[g]) + 16.0);
  // Threshold ordering sanity (levels strictly increasing).
  for (int j = 0; j + 1 < 15; ++j)
    if (!(thr[j] < thr[j + 1])) ok = false;
  if (!(t.level[0] == -1.0f && t.level[7] == 0.0f && t.level[15] == 1.0f)) ok = false;
  t.valid = ok ? 1 : 0;
  return t;
}

}  // namespace

const Nf4Tables& nf4_tables() {
  static const Nf4Tables tables = build();
  return tables;
}

}  // namespace loftq
