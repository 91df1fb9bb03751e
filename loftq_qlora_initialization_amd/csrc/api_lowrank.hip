// C-ABI entry points for the low-rank step and the whole alternating initialisation.
#include "lowrank.h"

namespace loftq {
namespace {

int64_t align256(int64_t x) { return (x + 255) / 256 * 256; }

// Validation of the low-rank step's shape parameters (shared by both calls).
loftq_status_t check_svd_shape(int64_t rows, int64_t cols, int32_t r, int32_t oversample, int32_t exact) {
  if (!shape_ok(rows, cols) || rows < 1 || cols < 1 || r < 1 || oversample < 0) return LOFTQ_ERR_INVALID_ARG;
  if (exact != 0 && exact != 1) return LOFTQ_ERR_INVALID_ARG;
  const int64_t mn = rows < cols ? rows : cols;
  if (exact) {
    if (r > mn) return LOFTQ_ERR_INVALID_ARG;
    if (mn > kMaxExact) return LOFTQ_ERR_UNSUPPORTED;
  } else {
    const int64_t l = static_cast<int64_t>(r) + oversample;
    if (l > mn) return LOFTQ_ERR_INVALID_ARG;
    if (l > kMaxL || r > kMaxR) return LOFTQ_ERR_UNSUPPORTED;
  }
  return LOFTQ_OK;
}

// Sketches drawn per launch: alternations t .. t + kSketchBatch - 1 at once.
constexpr int kSketchBatch = 8;

struct InitPlan {
  SvdPlan svd;
  int nparts;
  int64_t sketch_floats;   // one alternation's sketch in fragment order (0 for the exact SVD)
  int64_t off_e, off_parts, off_wparts, off_sketch, off_svd, bytes;
};

InitPlan make_init_plan(int64_t rows, int64_t cols, const loftq_config_t& c) {
  InitPlan p{};
  p.svd = make_svd_plan(rows, cols, c.rank, c.oversample, c.exact_svd != 0);
  const int64_t n = rows * cols;
  p.nparts = dequant_num_partials(n);
  p.sketch_floats = p.svd.exact ? 0 : p.svd.k_pad * 16 * p.svd.nt;
  const int batch = c.iterative_steps < kSketchBatch ? c.iterative_steps : kSketchBatch;
  int64_t off = 0;
  p.off_e = off;      off += align256(n * 4);
  p.off_parts = off;  off += align256(static_cast<int64_t>(p.nparts) * 8);
  p.off_wparts = off; off += align256(static_cast<int64_t>(p.nparts) * 8);
  p.off_sketch = off; off += align256(p.sketch_floats * 4 * (batch > 0 ? batch : 0));
  p.off_svd = off;    off += align256(p.svd.bytes);
  p.bytes = off;
  return p;
}

loftq_status_t check_config(int64_t rows, int64_t cols, const loftq_config_t* c) {
  if (c == nullptr) return LOFTQ_ERR_INVALID_ARG;
  if ((c->bits != 2 && c->bits != 3 && c->bits != 4) || c->blocksize != 64 || c->dq_blocksize != 256)
    return LOFTQ_ERR_UNSUPPORTED;
  if (c->iterative_steps < 0 || c->iterative_steps > 1000 || c->power_iters < 0 || c->power_iters > 64 ||
      (c->warm_start != 0 && c->warm_start != 1) || (c->double_quant != 0 && c->double_quant != 1))
    return LOFTQ_ERR_INVALID_ARG;
  return check_svd_shape(rows, cols, c->rank, c->oversample, c->exact_svd);
}

}  // namespace
}  // namespace loftq

using namespace loftq;

extern "C" {

size_t loftq_lowrank_svd_workspace_bytes(int64_t rows, int64_t cols, int32_t r, int32_t oversample, int32_t exact) {
  if (check_svd_shape(rows, cols, r, oversample, exact) != LOFTQ_OK) return 0;
  return static_cast<size_t>(make_svd_plan(rows, cols, r, oversample, exact != 0).bytes);
}

loftq_status_t loftq_lowrank_svd(const float* E, int64_t rows, int64_t cols, int32_t r, int32_t oversample,
                                 int32_t power_iters, int32_t exact, const float* omega, uint64_t seed, int32_t t,
                                 float* B, float* A, float* sigma, void* ws, size_t ws_bytes, void* stream) {
  loftq_status_t st = check_svd_shape(rows, cols, r, oversample, exact);
  if (st != LOFTQ_OK) return st;
  if (power_iters < 0 || power_iters > 64 || t < 1) return LOFTQ_ERR_INVALID_ARG;
  if (!E || !B || !A || !sigma || !ws) return LOFTQ_ERR_INVALID_ARG;
  if (!aligned16(E) || !aligned16(B) || !aligned16(A) || !aligned16(sigma) || !aligned16(ws) ||
      (omega && !aligned16(omega)))
    return LOFTQ_ERR_INVALID_ARG;
  const SvdPlan pl = make_svd_plan(rows, cols, r, oversample, exact != 0);
  if (ws_bytes < static_cast<size_t>(pl.bytes)) return LOFTQ_ERR_WORKSPACE;
  const ObjectiveArgs none{nullptr, 0, nullptr, 0, nullptr, nullptr};
  return from_hip(run_lowrank(E, pl, power_iters, omega, nullptr, seed, t, B, A, sigma, static_cast<char*>(ws), none,
                              static_cast<hipStream_t>(stream)));
}

size_t loftq_workspace_bytes(int64_t rows, int64_t cols, const loftq_config_t* cfg) {
  if (check_config(rows, cols, cfg) != LOFTQ_OK) return 0;
  return static_cast<size_t>(make_init_plan(rows, cols, *cfg).bytes);
}

loftq_status_t loftq_init(const void* W, loftq_dtype_t wdt, int64_t rows, int64_t cols, const loftq_config_t* cfg,
                          uint8_t* packed, float* absmax, int8_t* qabsmax, float* dq_scale, float* B, float* A,
                          double* objective, float* sigma, void* ws, size_t ws_bytes, void* stream) {
  loftq_status_t st = check_config(rows, cols, cfg);
  if (st != LOFTQ_OK) return st;
  if (wdt != LOFTQ_F32 && wdt != LOFTQ_BF16) return LOFTQ_ERR_INVALID_ARG;
  if (!nf_tables(cfg->bits).valid) return LOFTQ_ERR_UNSUPPORTED;
  const bool dq = cfg->double_quant != 0;
  if (!W || !packed || !absmax || !B || !A || !objective || !sigma || !ws) return LOFTQ_ERR_INVALID_ARG;
  if (dq && (!qabsmax || !dq_scale)) return LOFTQ_ERR_INVALID_ARG;
  const void* ptrs[] = {W, packed, absmax, B, A, objective, sigma, ws};
  for (const void* p : ptrs)
    if (!aligned16(p)) return LOFTQ_ERR_INVALID_ARG;
  if (dq && (!aligned16(qabsmax) || !aligned16(dq_scale))) return LOFTQ_ERR_INVALID_ARG;
  const InitPlan pl = make_init_plan(rows, cols, *cfg);
  if (ws_bytes < static_cast<size_t>(pl.bytes)) return LOFTQ_ERR_WORKSPACE;

  hipStream_t s = static_cast<hipStream_t>(stream);
  char* w = static_cast<char*>(ws);
  float* E = reinterpret_cast<float*>(w + pl.off_e);
  double* eparts = reinterpret_cast<double*>(w + pl.off_parts);
  double* wparts = reinterpret_cast<double*>(w + pl.off_wparts);
  char* svd_ws = w + pl.off_svd;
  const int64_t n = rows * cols;
  const int r = cfg->rank;
  const int T = cfg->iterative_steps;

  float* sketches = reinterpret_cast<float*>(w + pl.off_sketch);
  // the first dequant also leaves the partials of ||W||^2 (W is read there anyway)
  auto quant_step = [&](const float* Bp, const float* Ap, bool first) -> hipError_t {
    hipError_t x = launch_nf4_quantize(W, wdt, rows, cols, Bp, Ap, r, packed, absmax, s, cfg->bits);
    // the double quant of the absmax is derived (and written) inside the dequant
    if (x == hipSuccess)
      x = launch_nf4_dequantize(packed, absmax, nullptr, nullptr, n, cfg->dq_blocksize, W, wdt, E, eparts,
                                first ? wparts : nullptr, nullptr, s, dq ? qabsmax : nullptr, dq ? dq_scale : nullptr,
                                cfg->bits);
    return x;
  };
  hipError_t e = hipSuccess;
  if (T == 0) {
    const ObjectiveArgs obj0{eparts, pl.nparts, wparts, pl.nparts, objective, nullptr};
    if (e == hipSuccess) e = quant_step(nullptr, nullptr, true);
    if (e == hipSuccess) e = run_objective(obj0, s);
    if (e == hipSuccess) e = run_fill(B, rows * r, 0.f, s);
    if (e == hipSuccess) e = run_fill(A, static_cast<int64_t>(r) * cols, 0.f, s);
    if (e == hipSuccess) e = run_fill(sigma, r, 0.f, s);
    return from_hip(e);
  }
  for (int t = 1; t <= T && e == hipSuccess; ++t) {
    e = quant_step(t == 1 ? nullptr : B, t == 1 ? nullptr : A, t == 1);
    // alternation 1's solve also writes objective[0] (the error of plain NF4)
    const ObjectiveArgs objt{eparts, pl.nparts, wparts, pl.nparts, objective + t, t == 1 ? objective : nullptr};
    const float* om = nullptr;
    if (pl.sketch_floats > 0) {
      const int slot = (t - 1) % kSketchBatch;
      if (slot == 0 && e == hipSuccess) {
        const int count = (T - t + 1) < kSketchBatch ? (T - t + 1) : kSketchBatch;
        e = run_sketch(cfg->seed, t, count, cols, pl.svd.l, pl.svd.nt, pl.svd.k_pad, sketches, s);
      }
      om = sketches + slot * pl.sketch_floats;
      // warm start: from alternation 2 on, the first r columns come from the
      // previous alternation's A and sigma (still in their buffers here)
      if (cfg->warm_start != 0 && t > 1 && e == hipSuccess)
        e = run_warm_columns(A, sigma, cols, r, pl.svd.nt, sketches + slot * pl.sketch_floats, s);
    }
    if (e == hipSuccess)
      e = run_lowrank(E, pl.svd, cfg->power_iters, nullptr, om, cfg->seed, t, B, A, sigma, svd_ws, objt, s);
  }
  return from_hip(e);
}

}  // extern "C"
