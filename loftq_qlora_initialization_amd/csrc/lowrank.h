// Internal declarations for the low-rank step and the alternation driver.
#pragma once

#include <mutex>

#include "internal.h"

namespace loftq {

constexpr int kMaxL = 80;        // randomized sketch width l = r + p (fp64 l x l core lives in LDS)
constexpr int kMaxR = 64;        // rank limit of the randomized path's factor kernels
constexpr int kMaxExact = 512;   // exact SVD: min(rows, cols) limit
constexpr int kGramRows = 64;    // rows per workgroup (and fp64 Gram partial) of reduce_gram
constexpr int kReduceThreads = 512;
constexpr int kPanelRows = 64;   // rows per workgroup (and Gram partial) of the panel x small kernel
// Orthonormalisation solves on a side stream (SideLane) for E of at least this
// many elements; below kSideFullGridElems E^T Y then keeps a CU free for them.
constexpr int64_t kSideMinElems = int64_t(1) << 25;
constexpr int64_t kSideFullGridElems = int64_t(1) << 27;

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

// Split panels feed the bf16 matrix-core products of wide panels: each fp32 value
// v is stored as two bf16 pieces, hi = bf16(v) and lo = bf16(v - hi) (nearest,
// ties to even), in 32-row K steps laid out as the operands of
// v_mfma_f32_16x16x32_bf16.  For K step s, tile c / 16 and part (0 hi, 1 lo),
// lane L = 16 g + li holds 8 bf16 (16 bytes): rows 8 g + e (e = 0..7) of the
// step, column 16 (c / 16) + li.  Same byte count as the fp32 panel.
__host__ __device__ __forceinline__ int64_t split_index(int64_t rho, int c, int nt, int part) {
  const int64_t step = rho >> 5;
  const int g = static_cast<int>((rho >> 3) & 3), e = static_cast<int>(rho & 7);
  return (((step * nt + (c >> 4)) * 2 + part) * 64 + 16 * g + (c & 15)) * 8 + e;
}
// The operand of E^T Y (Y, over the rows of E) uses the same pieces with the rows
// of each pair of K steps interleaved: row 64 m + 16 g + 8 h + e is element e of
// lane group g in step 2 m + h (measured faster for the product's reads of E).
// Row of a K step's lane group g, element e, in either layout:
__host__ __device__ __forceinline__ int64_t split_row(int64_t s, int g, int e, bool paired) {
  return paired ? 64 * (s >> 1) + 16 * g + 8 * (s & 1) + e : 32 * s + 8 * g + e;
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
  int64_t off_omega_s, off_y_s, off_z_s;   // split copies of the panels (split_index), read by the products
  int64_t off_stats, off_x;
  int64_t off_sync;       // exact SVD, block Jacobi: grid-barrier and sweep counters
  bool bj;                // exact SVD runs the block Jacobi (vectors fit its LDS tiles)
  int64_t bytes;
};

SvdPlan make_svd_plan(int64_t d, int64_t k, int r, int oversample, bool exact);
// omega: caller's k x l sketch (row-major), or omega_frag: a sketch already in
// fragment order over k_pad rows, or neither: the sketch of alternation t is drawn.
// The residual E = W - deq(Q) formed inside the thin products from the weight
// and the codes, element by element exactly as the dequant kernel forms it
// (d = fl32(level[code] a'), e = fl32(w - d)), instead of being read from a
// stored E: 2 + 0.5 bytes per element (bf16 W) instead of 4.  Needs
// cols % 8 == 0.
struct VirtualE {
  const void* W;
  int w_bf16;             // 1: W is bf16, 0: fp32
  const uint8_t* packed;
  const float* scale;     // a' per 64-block: absmax, or fl32(qabsmax dq_scale) with double quant
  float level[16];        // the codebook of the codes
};

// A second stream that takes the orthonormalisation solves (Gram sum, Cholesky,
// R^-1) off the main stream, so that each runs beside the E^T Y product that
// follows it; the product's split-K reduction, their first consumer, waits for
// `join`.  Both events are reused: each record is waited on before the next.
struct SideLane {
  hipStream_t stream;
  hipEvent_t fork, join;
  std::mutex* mu;   // held while a call enqueues through the lane (the events are shared)
};
// The side lane of main stream s on the current device (created on first use,
// kept until the process ends), or null if one cannot be created.
SideLane* side_lane_for(hipStream_t s);

// norm_parts (randomized path only, optional): the first product E Omega also leaves
// the partial sums of ||E||^2 there (nn_row_blocks x nn_splits fp64), which obj
// may then name as its e_parts.
hipError_t run_lowrank(const float* E, const SvdPlan& pl, int q, const float* omega, const float* omega_frag,
                       uint64_t seed, int t, float* B, float* A, float* sigma, char* ws, const ObjectiveArgs& obj,
                       hipStream_t s, SideLane* side = nullptr, const VirtualE* ve = nullptr,
                       const uint16_t* omega_split = nullptr, double* norm_parts = nullptr);
// Sketches of alternations t .. t + count - 1, each rows x 16 nt floats in fragment order, back to back;
// run_sketch_split writes them in the products' split layout instead (the same bytes per sketch).
hipError_t run_sketch(uint64_t seed, int t, int count, int64_t k, int l, int nt, int64_t rows, float* out,
                      hipStream_t s);
hipError_t run_sketch_split(uint64_t seed, int t, int count, int64_t k, int l, int nt, int64_t rows, uint16_t* out,
                            hipStream_t s);
// Columns j < r of one fragment-order sketch (k rows) <- sqrt(k) A^T diag(sigma)^-1/2.
hipError_t run_warm_columns(const float* A, const float* sigma, int64_t k, int r, int nt, float* out, hipStream_t s);
hipError_t run_fill(float* p, int64_t n, float v, hipStream_t s);
hipError_t run_objective(const ObjectiveArgs& obj, hipStream_t s);
// d, k: rows and columns of E (E P picks its kernel and tile by nn_direct and nn_staged_rt)
GemmShape gemm_shape(bool transposed, int nt, int64_t d, int64_t k);
// E P with every wave reading the panel itself (no LDS staging): for the narrow
// panels (l <= 32) while the split panel (k rows of 64 nt bytes) stays within
// 1 MiB; measured on MI355X, the staged kernel wins beyond (4096 x 11008 at
// l = 24, every l = 80 panel).
constexpr bool nn_direct(int nt, int64_t k) { return nt <= 2 && int64_t(64) * nt * k <= (int64_t(1) << 20); }
// 16-row tiles per wave of the staged E P: two for wide panels (l > 32) when the
// 32-row blocks with the most split-K ranges allowed (k_pad partials within ~8 % of
// a 4-byte E, whole 128-column steps) still give two workgroups per CU, else one
// (measured on MI355X: 8192 x 28672 at l = 80, 250 -> 235 us; 11008 x 4096 slower
// with two).
constexpr int nn_staged_rt(int nt, int64_t d, int64_t k) {
  return (nt >= 3 && ((d + 127) / 128) * (((k * 8) / (100 * 16 * nt)) < k / 128 ? (k * 8) / (100 * 16 * nt) : k / 128) >= 512)
             ? 2 : 1;
}

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
// panel: the split copy (split_index) of the skinny operand.  nparts (E P only,
// optional): the sums of squares of E's elements, one fp64 per workgroup tile
// (nn_row_blocks x nn_splits of them).
void launch_gemm(bool transposed, const float* E, int64_t d, int64_t k, const uint16_t* panel, const SvdPlan& pl,
                 float* part, const CholJob& job, hipStream_t s, const VirtualE* ve = nullptr,
                 double* nparts = nullptr);

bool aligned16(const void* p);
bool shape_ok(int64_t rows, int64_t cols);
loftq_status_t from_hip(hipError_t e);

}  // namespace loftq
