// Internal declarations for the low-rank step and the alternation driver.
#pragma once

#include "internal.h"

namespace loftq {

constexpr int kMaxL = 80;        // randomized sketch width l = r + p (fp64 l x l core lives in LDS)
constexpr int kMaxR = 64;        // rank limit of the randomized path's factor kernels
constexpr int kMaxExact = 512;   // exact SVD: min(rows, cols) limit
constexpr int kGramRows = 64;    // rows per workgroup (and fp64 Gram partial) of reduce_gram
constexpr int kReduceThreads = 512;
constexpr int kPanelRows = 64;   // rows per workgroup (and Gram partial) of the panel x small kernel

// Where the objective of an alternation goes: ||E||^2 and ||W||^2 arrive as
// per-workgroup partial sums (summed in a fixed order by the consumer);
// out = sqrt(max(||E||^2 - sum sigma^2, 0) / ||W||^2), and, when out0 is set,
// out0 = sqrt(||E||^2 / ||W||^2) (the plain-quantization error before any refit).
struct ObjectiveArgs {
  const double* e_parts;
  int ne;
  const double* w_parts;
  int nw;
  double* out;
  double* out0;
};

// Skinny panels that feed the thin products as their B operand (the sketch,
// Y and Z = E^T Q) are stored in fragment order: 16-row blocks, each
// a run of NT = ceil(l / 16) tiles of 16 x 16 floats, element (rho, c) of a
// tile at ((rho % 16) / 4) * 64 + (c % 16) * 4 + rho % 4.  Lane 16 g + i of a
// wave then finds the four K-steps it feeds to one MFMA group in a single
// float4.  Rows beyond the panel and columns beyond l are stored as zeros.
__host__ __device__ __forceinline__ int64_t frag_index(int64_t rho, int c, int nt) {
  return ((rho >> 4) * nt + (c >> 4)) * 256 + ((rho & 15) >> 2) * 64 + (c & 15) * 4 + (rho & 3);
}

// Workgroup tile of a thin product: rows (gemm_nn) or columns (gemm_tn) per
// workgroup, and the granularity of its split of the contracted dimension.
struct GemmShape {
  int tile;
  int unit;
};

// Workspace layout and launch shapes of one low-rank step (byte offsets into ws).
struct SvdPlan {
  int64_t d, k;
  int r, l, nt;
  bool exact;
  int nn_row_blocks, nn_splits;
  int64_t nn_kper;
  int tn_col_blocks, tn_splits;
  int64_t tn_rper;
  int gram_parts_d, gram_parts_k;
  bool ride;              // l <= 32 Cholesky rides along with E^T Y (see make_svd_plan)
  int64_t k_pad, d_pad;   // fragment-order panel rows: nn_splits * nn_kper and tn_splits * tn_rper
  int64_t off_omega, off_y, off_z, off_part, off_gram_parts, off_gram_total, off_rinv, off_sb, off_sa;
  int64_t off_stats, off_x;
  int64_t bytes;
};

SvdPlan make_svd_plan(int64_t d, int64_t k, int r, int oversample, bool exact);
// omega: caller's k x l sketch (row-major), or omega_frag: a sketch already in
// fragment order over k_pad rows, or neither: the sketch of alternation t is drawn.
hipError_t run_lowrank(const float* E, const SvdPlan& pl, int q, const float* omega, const float* omega_frag,
                       uint64_t seed, int t, float* B, float* A, float* sigma, char* ws, const ObjectiveArgs& obj,
                       hipStream_t s);
// Sketches of alternations t .. t + count - 1, each rows x 16 nt floats in fragment order, back to back.
hipError_t run_sketch(uint64_t seed, int t, int count, int64_t k, int l, int nt, int64_t rows, float* out,
                      hipStream_t s);
// Columns j < r of one fragment-order sketch (k rows) <- sqrt(k) A^T diag(sigma)^-1/2.
hipError_t run_warm_columns(const float* A, const float* sigma, int64_t k, int r, int nt, float* out, hipStream_t s);
hipError_t run_fill(float* p, int64_t n, float v, hipStream_t s);
hipError_t run_objective(const ObjectiveArgs& obj, hipStream_t s);
GemmShape gemm_shape(bool transposed, int nt);

// A Cholesky that rides along with a thin product E^T Y (l <= 32 only): one
// extra workgroup sums the P fp64 Gram partials of Y (parts) and writes
// X = R^-1 (fp32 l x l) while the other workgroups stream E.  parts == nullptr:
// no job.
struct CholJob {
  const double* parts;
  int P;
  int l;
  float* Xinv;
};
void launch_gemm(bool transposed, const float* E, int64_t d, int64_t k, const float* panel, const SvdPlan& pl,
                 float* part, const CholJob& job, hipStream_t s);

bool aligned16(const void* p);
bool shape_ok(int64_t rows, int64_t cols);
loftq_status_t from_hip(hipError_t e);

}  // namespace loftq
