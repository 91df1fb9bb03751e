// C-ABI entry points for the low-rank step and the whole alternating initialisation.
#include <algorithm>
#include <mutex>
#include <vector>

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
// Streams a batched call may spread its matrices over.
constexpr int kMaxBatchStreams = 16;

struct InitPlan {
  SvdPlan svd;
  int nparts;
  int64_t sketch_floats;   // one alternation's sketch in fragment order (0 for the exact SVD)
  int64_t off_e, off_parts, off_wparts, off_sketch, off_svd, off_ascale, off_nparts, bytes;
  int nn_parts;            // ||E||^2 partials of the first product E Omega (alternations after the first)
};

// Whether the products form E from W and the codes (E is then never stored).
bool formed_residual(int64_t cols, const loftq_config_t& c) {
  return c.materialize_residual == 0 && c.exact_svd == 0 && c.iterative_steps > 0 && (cols & 7) == 0;
}

InitPlan make_init_plan(int64_t rows, int64_t cols, const loftq_config_t& c) {
  InitPlan p{};
  p.svd = make_svd_plan(rows, cols, c.rank, c.oversample, c.exact_svd != 0);
  const int64_t n = rows * cols;
  p.nparts = dequant_num_partials(n);
  p.sketch_floats = p.svd.exact ? 0 : p.svd.k_pad * 16 * p.svd.nt;
  const int batch = c.iterative_steps < kSketchBatch ? c.iterative_steps : kSketchBatch;
  int64_t off = 0;
  p.off_e = off;      off += formed_residual(cols, c) ? 0 : align256(n * 4);
  p.off_parts = off;  off += align256(static_cast<int64_t>(p.nparts) * 8);
  p.off_wparts = off; off += align256(static_cast<int64_t>(p.nparts) * 8);
  p.off_sketch = off; off += align256(p.sketch_floats * 4 * (batch > 0 ? batch : 0));
  p.off_svd = off;    off += align256(p.svd.bytes);
  // formed residual with double quant: a' = fl32(qabsmax dq_scale) per block, written by the dequant
  p.off_ascale = off; off += (formed_residual(cols, c) && c.double_quant) ? align256(((n + 63) / 64) * 4) : 0;
  p.nn_parts = p.svd.exact ? 0 : p.svd.nn_row_blocks * p.svd.nn_splits;
  p.off_nparts = off; off += align256(static_cast<int64_t>(p.nn_parts) * 8);
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
  // resume: k completed alternations (k + T stays within the sketch counter's range)
  if (c->init_from_BA < 0 || c->init_from_BA > 1000000 || (c->init_from_BA > 0 && c->iterative_steps == 0))
    return LOFTQ_ERR_INVALID_ARG;
  if (c->materialize_residual != 0 && c->materialize_residual != 1) return LOFTQ_ERR_INVALID_ARG;
  return check_svd_shape(rows, cols, c->rank, c->oversample, c->exact_svd);
}

// The device buffers of one initialisation (see loftq_init).
struct InitArgs {
  const void* W;
  int64_t rows, cols;
  uint8_t* packed;
  float* absmax;
  int8_t* qabsmax;
  float* dq_scale;
  float* B;
  float* A;
  double* objective;
  float* sigma;
};

loftq_status_t check_init(const InitArgs& a, loftq_dtype_t wdt, const loftq_config_t* cfg, const void* ws,
                          size_t ws_bytes) {
  loftq_status_t st = check_config(a.rows, a.cols, cfg);
  if (st != LOFTQ_OK) return st;
  if (wdt != LOFTQ_F32 && wdt != LOFTQ_BF16) return LOFTQ_ERR_INVALID_ARG;
  if (!nf_tables(cfg->bits).valid) return LOFTQ_ERR_UNSUPPORTED;
  const bool dq = cfg->double_quant != 0;
  if (!a.W || !a.packed || !a.absmax || !a.B || !a.A || !a.objective || !a.sigma || !ws) return LOFTQ_ERR_INVALID_ARG;
  if (dq && (!a.qabsmax || !a.dq_scale)) return LOFTQ_ERR_INVALID_ARG;
  const void* ptrs[] = {a.W, a.packed, a.absmax, a.B, a.A, a.objective, a.sigma, ws};
  for (const void* p : ptrs)
    if (!aligned16(p)) return LOFTQ_ERR_INVALID_ARG;
  if (dq && (!aligned16(a.qabsmax) || !aligned16(a.dq_scale))) return LOFTQ_ERR_INVALID_ARG;
  if (ws_bytes < static_cast<size_t>(make_init_plan(a.rows, a.cols, *cfg).bytes)) return LOFTQ_ERR_WORKSPACE;
  return LOFTQ_OK;
}

// The alternation loop of one validated initialisation, enqueued on stream s.
hipError_t run_init(const InitArgs& a, loftq_dtype_t wdt, const loftq_config_t& c, char* w, hipStream_t s,
                    SideLane* side = nullptr) {
  const loftq_config_t* cfg = &c;
  const void* W = a.W;
  const int64_t rows = a.rows, cols = a.cols;
  uint8_t* packed = a.packed;
  float* absmax = a.absmax;
  int8_t* qabsmax = a.qabsmax;
  float* dq_scale = a.dq_scale;
  float* B = a.B;
  float* A = a.A;
  double* objective = a.objective;
  float* sigma = a.sigma;
  const bool dq = cfg->double_quant != 0;
  const InitPlan pl = make_init_plan(rows, cols, *cfg);
  const bool formed = formed_residual(cols, *cfg);
  float* E = formed ? nullptr : reinterpret_cast<float*>(w + pl.off_e);
  float* ascale = formed && dq ? reinterpret_cast<float*>(w + pl.off_ascale) : nullptr;
  VirtualE ve{W, wdt == LOFTQ_BF16 ? 1 : 0, packed, dq ? ascale : absmax, {}};
  for (int i = 0; i < 16; ++i) ve.level[i] = nf_tables(cfg->bits).level[i];
  double* eparts = reinterpret_cast<double*>(w + pl.off_parts);
  double* wparts = reinterpret_cast<double*>(w + pl.off_wparts);
  char* svd_ws = w + pl.off_svd;
  const int64_t n = rows * cols;
  const int r = cfg->rank;
  const int T = cfg->iterative_steps;
  float* sketches = reinterpret_cast<float*>(w + pl.off_sketch);
  double* nparts = reinterpret_cast<double*>(w + pl.off_nparts);
  // ||E||^2 of an alternation of the randomized path comes from its first product
  // E Omega, which forms (or reads) every element of E anyway; the dequant sums it
  // only for T = 0 and the exact SVD.  So the dequant runs in the call's first
  // alternation (for the partials of ||W||^2, W being read there anyway) and
  // wherever E is stored; with E formed in the products the later alternations
  // only need the double quant (with each block's a').
  const bool dq_norms = T == 0 || pl.svd.exact;
  auto quant_step = [&](const float* Bp, const float* Ap, bool first) -> hipError_t {
    hipError_t x = launch_nf4_quantize(W, wdt, rows, cols, Bp, Ap, r, packed, absmax, s, cfg->bits);
    if (x != hipSuccess) return x;
    if (!first && formed)
      return dq ? launch_double_quant(absmax, (n + 63) / 64, cfg->dq_blocksize, qabsmax, dq_scale, s, ascale)
                : hipSuccess;
    // the double quant of the absmax is derived (and written) inside the dequant
    return launch_nf4_dequantize(packed, absmax, nullptr, nullptr, n, cfg->dq_blocksize, W, wdt, E,
                                 dq_norms ? eparts : nullptr, first ? wparts : nullptr, nullptr, s,
                                 dq ? qabsmax : nullptr, dq ? dq_scale : nullptr, cfg->bits, ascale);
  };
  hipError_t e = hipSuccess;
  if (T == 0) {
    const ObjectiveArgs obj0{eparts, pl.nparts, wparts, pl.nparts, objective, nullptr};
    if (e == hipSuccess) e = quant_step(nullptr, nullptr, true);
    if (e == hipSuccess) e = run_objective(obj0, s);
    if (e == hipSuccess) e = run_fill(B, rows * r, 0.f, s);
    if (e == hipSuccess) e = run_fill(A, static_cast<int64_t>(r) * cols, 0.f, s);
    if (e == hipSuccess) e = run_fill(sigma, r, 0.f, s);
    return e;
  }
  // alternations k0+1 .. k0+T; with k0 > 0 (resume) the first one starts from the caller's B, A
  const int k0 = cfg->init_from_BA;
  for (int i = 1; i <= T && e == hipSuccess; ++i) {
    const int t = k0 + i;   // the alternation's number: its sketch is that of (seed, t)
    const bool fresh = (t == 1);
    e = quant_step(fresh ? nullptr : B, fresh ? nullptr : A, i == 1);
    // the call's first solve also writes objective[0] (the error of its first quantization)
    const ObjectiveArgs objt{dq_norms ? eparts : nparts, dq_norms ? pl.nparts : pl.nn_parts, wparts, pl.nparts,
                             objective + i, i == 1 ? objective : nullptr};
    const float* om = nullptr;
    const uint16_t* om_split = nullptr;
    if (pl.sketch_floats > 0) {
      const int slot = (i - 1) % kSketchBatch;
      // without warm start the +-1 sketches go straight to the products' split layout
      const bool split = cfg->warm_start == 0;
      if (slot == 0 && e == hipSuccess) {
        const int count = (T - i + 1) < kSketchBatch ? (T - i + 1) : kSketchBatch;
        e = split ? run_sketch_split(cfg->seed, t, count, cols, pl.svd.l, pl.svd.nt, pl.svd.k_pad,
                                     reinterpret_cast<uint16_t*>(sketches), s)
                  : run_sketch(cfg->seed, t, count, cols, pl.svd.l, pl.svd.nt, pl.svd.k_pad, sketches, s);
      }
      if (split) {
        om_split = reinterpret_cast<const uint16_t*>(sketches + slot * pl.sketch_floats);
      } else {
        om = sketches + slot * pl.sketch_floats;
        // warm start: from alternation 2 on, the first r columns come from the
        // previous alternation's A and sigma (still in their buffers here)
        if (t > 1 && e == hipSuccess)
          e = run_warm_columns(A, sigma, cols, r, pl.svd.nt, sketches + slot * pl.sketch_floats, s);
      }
    }
    if (e == hipSuccess)
      e = run_lowrank(E, pl.svd, cfg->power_iters, nullptr, om, cfg->seed, t, B, A, sigma, svd_ws, objt, s, side,
                      formed ? &ve : nullptr, om_split, dq_norms ? nullptr : nparts);
  }
  return e;
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
  const hipStream_t s = static_cast<hipStream_t>(stream);
  SideLane* side = side_lane_for(s);
  std::unique_lock<std::mutex> lk;
  if (side != nullptr) lk = std::unique_lock<std::mutex>(*side->mu);
  return from_hip(run_lowrank(E, pl, power_iters, omega, nullptr, seed, t, B, A, sigma, static_cast<char*>(ws), none,
                              s, side));
}

size_t loftq_workspace_bytes(int64_t rows, int64_t cols, const loftq_config_t* cfg) {
  if (check_config(rows, cols, cfg) != LOFTQ_OK) return 0;
  return static_cast<size_t>(make_init_plan(rows, cols, *cfg).bytes);
}

loftq_status_t loftq_init(const void* W, loftq_dtype_t wdt, int64_t rows, int64_t cols, const loftq_config_t* cfg,
                          uint8_t* packed, float* absmax, int8_t* qabsmax, float* dq_scale, float* B, float* A,
                          double* objective, float* sigma, void* ws, size_t ws_bytes, void* stream) {
  const InitArgs a{W, rows, cols, packed, absmax, qabsmax, dq_scale, B, A, objective, sigma};
  loftq_status_t st = check_init(a, wdt, cfg, ws, ws_bytes);
  if (st != LOFTQ_OK) return st;
  const hipStream_t s = static_cast<hipStream_t>(stream);
  SideLane* side = side_lane_for(s);
  std::unique_lock<std::mutex> lk;
  if (side != nullptr) lk = std::unique_lock<std::mutex>(*side->mu);
  return from_hip(run_init(a, wdt, *cfg, static_cast<char*>(ws), s, side));
}

size_t loftq_batch_workspace_bytes(const loftq_matrix_t* mats, int32_t count, const loftq_config_t* cfg) {
  if (mats == nullptr || count < 1 || cfg == nullptr) return 0;
  size_t need = 0;
  for (int32_t i = 0; i < count; ++i) {
    if (check_config(mats[i].rows, mats[i].cols, cfg) != LOFTQ_OK) return 0;
    const size_t b = static_cast<size_t>(make_init_plan(mats[i].rows, mats[i].cols, *cfg).bytes);
    need = b > need ? b : need;
  }
  return need;
}

loftq_status_t loftq_init_batch(const loftq_matrix_t* mats, int32_t count, loftq_dtype_t wdt,
                                const loftq_config_t* cfg, int32_t nstreams, void* const* streams,
                                void* const* ws, size_t ws_bytes) {
  if (mats == nullptr || count < 0 || cfg == nullptr) return LOFTQ_ERR_INVALID_ARG;
  if (count == 0) return LOFTQ_OK;
  if (nstreams < 1 || nstreams > kMaxBatchStreams || ws == nullptr) return LOFTQ_ERR_INVALID_ARG;
  for (int32_t j = 0; j < nstreams; ++j)
    for (int32_t i = 0; i < j; ++i)
      if (ws[i] == ws[j]) return LOFTQ_ERR_INVALID_ARG;   // each stream needs a workspace of its own
  // every matrix is validated (with every stream's workspace) before anything is enqueued
  for (int32_t i = 0; i < count; ++i) {
    const InitArgs a{mats[i].W, mats[i].rows, mats[i].cols, mats[i].packed, mats[i].absmax, mats[i].qabsmax,
                     mats[i].dq_scale, mats[i].B, mats[i].A, mats[i].objective, mats[i].sigma};
    for (int32_t j = 0; j < nstreams; ++j) {
      const loftq_status_t st = check_init(a, wdt, cfg, ws[j], ws_bytes);
      if (st != LOFTQ_OK) return st;
    }
  }
  // Enqueue order: the matrices sorted by descending element count (ties by index), taken one from
  // the front and two from the back in turn, each to the stream with the least work so far (the
  // streams are fed in turn and all start at once).  The products re-read W and the codes six times
  // per alternation, so the matrices in flight at one time share the 256 MB Infinity Cache; a mix of
  // large and small ones keeps more of their bytes there than the largest side by side, as a plain
  // longest-first order would run them (decoder batch, 3 streams: 178.1 -> 170.1 ms).
  std::vector<int32_t> sorted(count);
  for (int32_t i = 0; i < count; ++i) sorted[i] = i;
  std::stable_sort(sorted.begin(), sorted.end(), [&](int32_t x, int32_t y) {
    return mats[x].rows * mats[x].cols > mats[y].rows * mats[y].cols;
  });
  std::vector<int32_t> order;
  order.reserve(count);
  for (int32_t lo = 0, hi = count - 1; lo <= hi;) {
    order.push_back(sorted[lo++]);
    for (int t = 0; t < 2 && lo <= hi; ++t) order.push_back(sorted[hi--]);
  }
  std::vector<int64_t> load(nstreams, 0);
  for (int32_t idx : order) {
    int32_t j = 0;
    for (int32_t c = 1; c < nstreams; ++c)
      if (load[c] < load[j]) j = c;
    load[j] += mats[idx].rows * mats[idx].cols;
    const loftq_matrix_t& m = mats[idx];
    const InitArgs a{m.W, m.rows, m.cols, m.packed, m.absmax, m.qabsmax, m.dq_scale, m.B, m.A, m.objective, m.sigma};
    const hipError_t e = run_init(a, wdt, *cfg, static_cast<char*>(ws[j]),
                                  static_cast<hipStream_t>(streams ? streams[j] : nullptr));
    if (e != hipSuccess) return from_hip(e);
  }
  return LOFTQ_OK;
}

}  // extern "C"
