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
//
// Lower-bit NormalFloat (k = 2, 3; the LoftQ blog reports 2- and 3-bit LoftQ but
// gives no codebook): the same construction with 2^(k-1) positive and
// 2^(k-1) - 1 negative levels and delta_k = 1 - (1/2^(k+1) + 1/(2 (2^k - 1)))/2,
// which is NF4's delta at k = 4.  Unused thresholds are +inf, so code counts
// stop at 2^k - 1 and the kernels need no other change.
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

Nf4Tables build(int bits) {
  Nf4Tables t;
  std::memset(&t, 0, sizeof(t));
  const int nlev = 1 << bits, npos = nlev / 2, nneg = npos - 1, nthr = nlev - 1;
  const double delta = 1.0 - 0.5 * (1.0 / static_cast<double>(2 * nlev) + 1.0 / (2.0 * (nlev - 1)));
  double v[16];
  int n = 0;
  // npos + 1 (resp. nneg + 1) evenly spaced probabilities from delta to 1/2, the last dropped
  const double step_p = (0.5 - delta) / npos, step_n = (0.5 - delta) / nneg;
  for (int i = 0; i < npos; ++i) v[n++] = normal_quantile_upper(delta + i * step_p);
  for (int i = 0; i < nneg; ++i) v[n++] = -normal_quantile_upper(delta + i * step_n);
  v[n++] = 0.0;
  std::sort(v, v + nlev);
  double vmax = 0.0;
  for (int i = 0; i < nlev; ++i) vmax = std::max(vmax, std::fabs(v[i]));
  for (int i = 0; i < 16; ++i) t.level[i] = i < nlev ? static_cast<float>(v[i] / vmax) : 1.0f;

  // Threshold j: the largest fp32 not above the exact midpoint m_j.  For any
  // fp32 x, x > thr[j] exactly when x > m_j (equality at m_j goes to the lower
  // level, i.e. argmin-first).  Thresholds past the last level are +inf.
  double thr[15];
  for (int j = 0; j < 15; ++j) {
    if (j >= nthr) {
      t.thr[j] = std::numeric_limits<float>::infinity();
      thr[j] = std::numeric_limits<double>::infinity();
      continue;
    }
    double m = 0.5 * (static_cast<double>(t.level[j]) + static_cast<double>(t.level[j + 1]));
    float f = static_cast<float>(m);
    if (static_cast<double>(f) > m) f = std::nextafter(f, -std::numeric_limits<float>::infinity());
    t.thr[j] = f;
    thr[j] = f;
  }

  // Encode grid: y = 16 x + origin falls in cell int(y) (0..32), cells of width
  // 1/16 in x.  Invariants the kernel relies on: at most one threshold per cell,
  // and every threshold at least `margin` from its cell's edges (the cell index
  // computed in fp32 may be off by one only for x within ~2^-22 of an edge).
  // NF4 uses origin 16 (cells over [-1, 1) and cell 32 for x >= 1); a codebook
  // with a threshold on an edge of that grid (NF2's -1/2) takes the first
  // shifted origin that satisfies the invariants.
  const double margin = 1.0 / 4096.0;
  auto make_grid = [&](double origin) {
    bool good = true;
    for (int g = 0; g < 33; ++g) {
      t.cell_thr[g] = std::numeric_limits<float>::infinity();
      t.cell_base[g] = 0;
    }
    for (int g = 0; g < 33; ++g) {
      const double lo = (g - origin) / 16.0;
      const double hi = g < 32 ? (g + 1 - origin) / 16.0 : std::numeric_limits<double>::infinity();
      int inside = 0, below = 0;
      for (int j = 0; j < nthr; ++j) {
        if (thr[j] < lo) {
          ++below;
        } else if (thr[j] < hi) {
          ++inside;
          t.cell_thr[g] = static_cast<float>(thr[j]);
          if (thr[j] - lo < margin || hi - thr[j] < margin) good = false;
        }
      }
      if (inside > 1) good = false;
      t.cell_base[g] = below;
    }
    return good;   // origin >= 16: cell 0 starts at or below x = -1, so no threshold is left out
  };
  bool ok = false;
  for (double origin : {16.0, 16.5, 16.25, 16.75}) {
    if (make_grid(origin)) {
      t.cell_origin = static_cast<float>(origin);
      ok = true;
      break;
    }
  }
  // The encoder compares y = 16 x + origin (computed in fp32) with fl32(16 thr + origin).
  for (int g = 0; g < 33; ++g)
    t.cell_thr16[g] = std::isinf(t.cell_thr[g])
                          ? t.cell_thr[g]
                          : static_cast<float>(16.0 * static_cast<double>(t.cell_thr[g]) + t.cell_origin);
  // Threshold ordering sanity (levels strictly increasing).
  for (int j = 0; j + 1 < nthr; ++j)
    if (!(thr[j] < thr[j + 1])) ok = false;
  if (!(t.level[0] == -1.0f && t.level[npos - 1] == 0.0f && t.level[nlev - 1] == 1.0f)) ok = false;
  t.valid = ok ? 1 : 0;
  return t;
}

}  // namespace

const Nf4Tables& nf_tables(int bits) {
  static const Nf4Tables t2 = build(2), t3 = build(3), t4 = build(4);
  return bits == 2 ? t2 : (bits == 3 ? t3 : t4);
}

const Nf4Tables& nf4_tables() { return nf_tables(4); }

}  // namespace loftq
