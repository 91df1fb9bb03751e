// Internal declarations for the low-rank step and the alternation driver.
#pragma once

#include "internal.h"

namespace loftq {

constexpr int kMaxL = 96;        // randomized sketch width l = r + p (fp64 l x l core lives in LDS)
constexpr int kMaxR = 64;        // rank limit of the randomized path's factor kernels
constexpr int kMaxExact = 512;   // exact SVD: min(rows, cols) limit
constexpr int kGramRows = 128;   // rows per fp64 Gram partial of a reduced product
constexpr int kPanelRows = 64;   // rows per workgroup (and Gram partial) of the panel x small kernel

// Where the objective of an alternation goes: ||E||^2 and ||W||^2 arrive as
// per-workgroup partial sums; out = sqrt(max(||E||^2 - sum sigma^2, 0) / ||W||^2).
struct ObjectiveArgs {
  const double* e_parts;
  int ne;
  const double* w_parts;
  int nw;
  double* out;
};

__device__ inline void write_objective(const ObjectiveArgs& o, double sig2) {
  if (o.out == nullptr) return;
  double es = 0.0, ws = 0.0;
  for (int i = 0; i < o.ne; ++i) es += o.e_parts[i];
  for (int i = 0; i < o.nw; ++i) ws += o.w_parts[i];
  const double num = es - sig2;
  *o.out = ws > 0.0 ? sqrt((num > 0.0 ? num : 0.0) / ws) : 0.0;
}

// Workspace layout and launch shapes of one low-rank step (byte offsets into ws).
struct SvdPlan {
  int64_t d, k;
  int r, l, nt;
  bool exact;
  int nn_row_blocks, nn_splits;
  int64_t nn_kper;
  int tn_col_blocks, tn_splits;
  int64_t tn_rper;
  int gram_parts_d, gram_parts_k, gram_parts_qy;
  int64_t off_omega, off_y, off_qy, off_z, off_qz, off_part, off_gram1, off_gram2, off_rinv, off_sb, off_sa;
  int64_t off_stats, off_x;
  int64_t bytes;
};

SvdPlan make_svd_plan(int64_t d, int64_t k, int r, int oversample, bool exact);
hipError_t run_lowrank(const float* E, const SvdPlan& pl, int q, const float* omega, uint64_t seed, int t, float* B,
                       float* A, float* sigma, char* ws, const ObjectiveArgs& obj, hipStream_t s);
hipError_t run_sketch(uint64_t seed, int t, int64_t k, int l, float* out, hipStream_t s);
hipError_t run_fill(float* p, int64_t n, float v, hipStream_t s);
hipError_t run_objective(const ObjectiveArgs& obj, hipStream_t s);

bool aligned16(const void* p);
bool shape_ok(int64_t rows, int64_t cols);
loftq_status_t from_hip(hipError_t e);

}  // namespace loftq
