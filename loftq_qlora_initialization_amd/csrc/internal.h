// Internal declarations shared by the libloftq translation units.
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/loftq.h"

namespace loftq {

// While kernel timing is enabled (loftq_profile_enable), supplies a start/stop
// event pair that the launch itself records around the kernel's execution
// (hipExtLaunchKernel), and files it under the kernel's name; otherwise both
// events are null and the launch is a plain one.
class ProfScope {
 public:
  explicit ProfScope(const char* name);
  ~ProfScope();
  ProfScope(const ProfScope&) = delete;
  ProfScope& operator=(const ProfScope&) = delete;
  hipEvent_t start() const { return start_; }
  hipEvent_t stop() const { return stop_; }

 private:
  const char* name_;
  hipEvent_t start_;
  hipEvent_t stop_;
};

#define LQ_LAUNCH(NAME, KERNEL, GRID, BLOCK, SHMEM, STREAM, ...)                                             \
  do {                                                                                                     \
    ::loftq::ProfScope lq_prof_scope_(NAME);                                                               \
    hipExtLaunchKernelGGL(KERNEL, GRID, BLOCK, SHMEM, STREAM, lq_prof_scope_.start(), lq_prof_scope_.stop(), \
                          0, __VA_ARGS__);                                                                 \
  } while (0)

// NF4 tables handed to kernels by value (kernel arguments), built once on the
// host from the quantile definition of the levels.
//
// Encoding uses a 33-cell uniform grid over x in [-1, 1]: cell g covers
// [-1 + g/16, -1 + (g+1)/16) (cell 32 holds x >= 1).  Each cell contains at
// most one decision threshold; cell_base[g] counts the thresholds below the
// cell and cell_thr[g] is the threshold inside it (+inf if none), so the code
// of x in cell g is cell_base[g] + (x > cell_thr[g]).
struct Nf4Tables {
  float level[16];      // ascending NF4 levels, fp32
  float thr[15];        // thr[j]: for fp32 x, x > thr[j]  <=>  x > (level[j]+level[j+1])/2
  float cell_thr[33];
  float cell_thr16[33]; // fl32(16 cell_thr + cell_origin) (+inf where cell_thr is +inf)
  int32_t cell_base[33];
  float cell_origin;    // y = 16 x + cell_origin selects the cell (16 for NF4)
  int32_t valid;        // 1 if every grid invariant held at construction
};

const Nf4Tables& nf4_tables();
// k-bit NormalFloat tables, k = 2, 3 or 4 (4: the NF4 tables); codes are stored in nibbles either way.
const Nf4Tables& nf_tables(int bits);

// Window (absolute, in x units) inside which the fast path's x' = R * (1/a)
// may disagree with fl32(R / a) about a threshold; such elements are redone with
// an IEEE division.  |x' - fl32(R/a)| <= 3 * 2^-24 for |x| <= 1.
constexpr float kDangerWindow = 9.5367431640625e-07f;  // 2^-20
// The same window for the encoder's y = fma(R, 16 rcp(a), 16) against the
// cell thresholds fl32(16 thr + 16): |y - (16 fl32(R/a) + 16)| <= 2^-18 (rcp
// within 1 ulp, one rounding of the product-sum, 16 x the quotient's rounding)
// and |thr16 - (16 thr + 16)| <= 2^-19, both well inside 2^-16.
constexpr float kDangerWindow16 = 1.52587890625e-05f;  // 2^-16

// ---- launchers (quant_kernels.hip) ----
hipError_t launch_nf4_quantize(const void* W, loftq_dtype_t wdt, int64_t rows, int64_t cols,
                               const float* B, const float* A, int r, uint8_t* packed, float* absmax,
                               hipStream_t s, int bits = 4);
// a_out (optional): each block's dequantization scale a' = fl32(q scale) as well
hipError_t launch_double_quant(const float* absmax, int64_t nblocks, int dqbs, int8_t* q, float* scale,
                               hipStream_t s, float* a_out = nullptr);
// QLoRA forward Y = X bf16(deq(Q))^T + alpha (X bf16(A)^T) bf16(B)^T (forward_kernels.hip);
// Tws: up to 8 K-split partials of X A^T, n_tok x r fp32 each (qlora_forward_workspace_bytes);
// unused without B.
size_t qlora_forward_workspace_bytes(int64_t n_tok, int r);
// false when one of the call's launches would exceed 2^32 work-items
bool qlora_forward_shape_ok(int64_t n_tok, int64_t rows, int64_t cols, int r);
hipError_t launch_qlora_forward(const void* X, int64_t n_tok, int64_t rows, int64_t cols, const uint8_t* packed,
                                const float* absmax, const int8_t* qa, const float* dqs, int bits, const float* B,
                                const float* A, int r, float alpha, float* Y, float* Tws, hipStream_t s);
// Q' = NF4(deq(Q) + alpha B A); input scales absmax or (q, dqscale); output
// absmax_out and, with q_out / dqs_out, its double quant (dq_blocksize 256).
hipError_t launch_nf4_merge(const uint8_t* packed, const float* absmax, const int8_t* q, const float* dqscale,
                            int64_t rows, int64_t cols, const float* B, const float* A, int r, float alpha,
                            uint8_t* packed_out, float* absmax_out, int8_t* q_out, float* dqs_out, hipStream_t s);
// Sum of squares of the output: with `partials`, one fp64 partial per workgroup
// (dequant_num_partials(n) of them, summed in a fixed order by the consumer);
// otherwise, with `sumsq`, accumulated into *sumsq with atomics (after zeroing it).
// With W and `wpartials`, the same per-workgroup partials of sum W^2 as well.
// With q_out / dqs_out (dq_blocksize 256), the double quant of `absmax` is
// derived inside the dequant and written there (q and dqscale unused).
hipError_t launch_nf4_dequantize(const uint8_t* packed, const float* absmax, const int8_t* q,
                                 const float* dqscale, int64_t n, int dqbs, const void* W,
                                 loftq_dtype_t wdt, float* out, double* partials, double* wpartials,
                                 double* sumsq, hipStream_t s, int8_t* q_out = nullptr,
                                 float* dqs_out = nullptr, int bits = 4, float* a_out = nullptr);
int dequant_num_partials(int64_t n);
hipError_t launch_sumsq_weight(const void* W, loftq_dtype_t wdt, int64_t n, double* partials, unsigned* counter,
                               double* sumsq, hipStream_t s);

}  // namespace loftq
