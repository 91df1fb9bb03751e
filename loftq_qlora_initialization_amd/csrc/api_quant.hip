// C-ABI entry points for the NF4 codec and the adapter merge: argument validation, then launches.
#include <cmath>
#include <cstring>
#include <mutex>

#include "internal.h"

namespace loftq {

// Scratch of the allocation-free QLoRA forward (loftq_qlora_forward_noalloc): a
// file-scope device array, one copy per GPU the library runs on, held until the
// process ends.  Host code never passes `scratch` itself to a kernel (on the host it
// is only a stand-in for the symbol): its device address is looked up once per
// device, with that device current, and kept in scratch_ptr.
constexpr size_t kStaticScratchBytes = size_t(8) << 20;
__device__ __align__(256) char scratch[kStaticScratchBytes];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// The current device's copy of `scratch` (set up on the first call on that device).
hipError_t scratch_ptr(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return hipSuccess;
}
}  // namespace

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

bool shape_ok(int64_t rows, int64_t cols) {
  return rows >= 0 && cols >= 0 && rows < (int64_t(1) << 31) && cols < (int64_t(1) << 31);
}

loftq_status_t from_hip(hipError_t e) { return e == hipSuccess ? LOFTQ_OK : LOFTQ_ERR_HIP; }

}  // namespace loftq

using namespace loftq;

extern "C" {

const char* loftq_status_string(loftq_status_t status) {
  switch (status) {
    case LOFTQ_OK: return "ok";
    case LOFTQ_ERR_INVALID_ARG: return "invalid argument";
    case LOFTQ_ERR_UNSUPPORTED: return "unsupported configuration";
    case LOFTQ_ERR_WORKSPACE: return "workspace too small";
    case LOFTQ_ERR_HIP: return "HIP runtime error";
  }
  return "unknown status";
}

void loftq_nf4_codebook(float* out16) {
  if (out16) std::memcpy(out16, nf4_tables().level, 16 * sizeof(float));
}

loftq_status_t loftq_nf_codebook(int32_t bits, float* out) {
  if (bits != 2 && bits != 3 && bits != 4) return LOFTQ_ERR_UNSUPPORTED;
  if (!out) return LOFTQ_ERR_INVALID_ARG;
  if (!nf_tables(bits).valid) return LOFTQ_ERR_UNSUPPORTED;   // an encoder grid invariant failed
  std::memcpy(out, nf_tables(bits).level, (size_t(1) << bits) * sizeof(float));
  return LOFTQ_OK;
}

void loftq_default_config(loftq_config_t* cfg) {
  if (!cfg) return;
  std::memset(cfg, 0, sizeof(*cfg));
  cfg->bits = 4;
  cfg->iterative_steps = 5;
  cfg->rank = 16;
  cfg->blocksize = 64;
  cfg->double_quant = 1;
  cfg->dq_blocksize = 256;
  cfg->oversample = 8;
  cfg->power_iters = 2;
  cfg->exact_svd = 0;
  cfg->seed = 42;
}

loftq_status_t loftq_nf4_quantize(const void* W, loftq_dtype_t wdt, int64_t rows, int64_t cols, const float* B,
                                  const float* A, int32_t r, int32_t blocksize, uint8_t* packed, float* absmax,
                                  void* stream) {
  if (!shape_ok(rows, cols) || (wdt != LOFTQ_F32 && wdt != LOFTQ_BF16)) return LOFTQ_ERR_INVALID_ARG;
  if (blocksize != 64) return LOFTQ_ERR_UNSUPPORTED;
  if (!nf4_tables().valid) return LOFTQ_ERR_UNSUPPORTED;
  if ((B == nullptr) != (A == nullptr)) return LOFTQ_ERR_INVALID_ARG;
  if (B != nullptr && (r < 1 || r > 4096)) return LOFTQ_ERR_INVALID_ARG;
  const int64_t n = rows * cols;
  if (n == 0) return LOFTQ_OK;
  if (!W || !packed || !absmax) return LOFTQ_ERR_INVALID_ARG;
  if (!aligned16(W) || !aligned16(packed) || !aligned16(absmax)) return LOFTQ_ERR_INVALID_ARG;
  if (B && (!aligned16(B) || !aligned16(A))) return LOFTQ_ERR_INVALID_ARG;
  return from_hip(launch_nf4_quantize(W, wdt, rows, cols, B, A, r, packed, absmax,
                                      static_cast<hipStream_t>(stream)));
}

loftq_status_t loftq_double_quant(const float* absmax, int64_t nblocks, int32_t dq_blocksize, int8_t* qabsmax,
                                  float* dq_scale, void* stream) {
  if (nblocks < 0) return LOFTQ_ERR_INVALID_ARG;
  if (dq_blocksize != 256) return LOFTQ_ERR_UNSUPPORTED;
  if (nblocks == 0) return LOFTQ_OK;
  if (!absmax || !qabsmax || !dq_scale) return LOFTQ_ERR_INVALID_ARG;
  if (!aligned16(absmax) || !aligned16(qabsmax) || !aligned16(dq_scale)) return LOFTQ_ERR_INVALID_ARG;
  return from_hip(launch_double_quant(absmax, nblocks, dq_blocksize, qabsmax, dq_scale,
                                      static_cast<hipStream_t>(stream)));
}

loftq_status_t loftq_nf4_dequantize(const uint8_t* packed, const float* absmax, const int8_t* qabsmax,
                                    const float* dq_scale, int64_t rows, int64_t cols, int32_t blocksize,
                                    int32_t dq_blocksize, const void* W, loftq_dtype_t wdt, float* out,
                                    double* sumsq, void* stream) {
  if (!shape_ok(rows, cols)) return LOFTQ_ERR_INVALID_ARG;
  if (W && wdt != LOFTQ_F32 && wdt != LOFTQ_BF16) return LOFTQ_ERR_INVALID_ARG;
  if (blocksize != 64) return LOFTQ_ERR_UNSUPPORTED;
  if (!nf4_tables().valid) return LOFTQ_ERR_UNSUPPORTED;
  const bool dq = qabsmax != nullptr || dq_scale != nullptr;
  if (dq && (!qabsmax || !dq_scale)) return LOFTQ_ERR_INVALID_ARG;
  if (dq && dq_blocksize != 256) return LOFTQ_ERR_UNSUPPORTED;
  const int64_t n = rows * cols;
  if (n > 0) {
    if (!packed || !out || (!dq && !absmax)) return LOFTQ_ERR_INVALID_ARG;
    if (!aligned16(packed) || !aligned16(out) || (W && !aligned16(W))) return LOFTQ_ERR_INVALID_ARG;
    if (dq ? (!aligned16(qabsmax) || !aligned16(dq_scale)) : !aligned16(absmax)) return LOFTQ_ERR_INVALID_ARG;
  }
  if (sumsq && !aligned16(sumsq) && (reinterpret_cast<uintptr_t>(sumsq) & 7u)) return LOFTQ_ERR_INVALID_ARG;
  return from_hip(launch_nf4_dequantize(packed, dq ? nullptr : absmax, dq ? qabsmax : nullptr,
                                        dq ? dq_scale : nullptr, n, dq_blocksize, W, wdt, out, nullptr, nullptr,
                                        sumsq, static_cast<hipStream_t>(stream)));
}

static loftq_status_t merge_impl(const uint8_t* packed, const float* absmax, const int8_t* qabsmax,
                                 const float* dq_scale, int64_t rows, int64_t cols, int32_t blocksize,
                                 int32_t dq_blocksize, const float* B, const float* A, int32_t r, float alpha,
                                 uint8_t* packed_out, float* absmax_out, int8_t* qabsmax_out, float* dq_scale_out,
                                 void* stream) {
  if (!shape_ok(rows, cols)) return LOFTQ_ERR_INVALID_ARG;
  if (blocksize != 64) return LOFTQ_ERR_UNSUPPORTED;
  if (!nf4_tables().valid) return LOFTQ_ERR_UNSUPPORTED;
  const bool dq_in = qabsmax != nullptr || dq_scale != nullptr;
  const bool dq_out = qabsmax_out != nullptr || dq_scale_out != nullptr;
  if (dq_in && (!qabsmax || !dq_scale)) return LOFTQ_ERR_INVALID_ARG;
  if (dq_out && (!qabsmax_out || !dq_scale_out)) return LOFTQ_ERR_INVALID_ARG;
  if ((dq_in || dq_out) && dq_blocksize != 256) return LOFTQ_ERR_UNSUPPORTED;
  if ((B == nullptr) != (A == nullptr)) return LOFTQ_ERR_INVALID_ARG;
  if (B != nullptr && r < 1) return LOFTQ_ERR_INVALID_ARG;
  if (!std::isfinite(alpha)) return LOFTQ_ERR_INVALID_ARG;
  const int64_t n = rows * cols;
  if (n == 0) return LOFTQ_OK;
  if (cols % 64 != 0 || (B != nullptr && r > 64)) return LOFTQ_ERR_UNSUPPORTED;
  if (!packed || !packed_out || !absmax_out || (!dq_in && !absmax)) return LOFTQ_ERR_INVALID_ARG;
  if (!aligned16(packed) || !aligned16(packed_out) || !aligned16(absmax_out)) return LOFTQ_ERR_INVALID_ARG;
  if (dq_in ? (!aligned16(qabsmax) || !aligned16(dq_scale)) : !aligned16(absmax)) return LOFTQ_ERR_INVALID_ARG;
  if (dq_out && (!aligned16(qabsmax_out) || !aligned16(dq_scale_out))) return LOFTQ_ERR_INVALID_ARG;
  if (B && (!aligned16(B) || !aligned16(A))) return LOFTQ_ERR_INVALID_ARG;
  return from_hip(launch_nf4_merge(packed, dq_in ? nullptr : absmax, dq_in ? qabsmax : nullptr,
                                   dq_in ? dq_scale : nullptr, rows, cols, B, A, B ? r : 0, alpha, packed_out,
                                   absmax_out, dq_out ? qabsmax_out : nullptr, dq_out ? dq_scale_out : nullptr,
                                   static_cast<hipStream_t>(stream)));
}

loftq_status_t loftq_nf4_merge(const uint8_t* packed, const float* absmax, const int8_t* qabsmax,
                               const float* dq_scale, int64_t rows, int64_t cols, int32_t blocksize,
                               int32_t dq_blocksize, const float* B, const float* A, int32_t r, float alpha,
                               uint8_t* packed_out, float* absmax_out, int8_t* qabsmax_out, float* dq_scale_out,
                               void* stream) {
  return merge_impl(packed, absmax, qabsmax, dq_scale, rows, cols, blocksize, dq_blocksize, B, A, r, alpha,
                    packed_out, absmax_out, qabsmax_out, dq_scale_out, stream);
}

loftq_status_t loftq_nf4_unmerge(const uint8_t* packed, const float* absmax, const int8_t* qabsmax,
                                 const float* dq_scale, int64_t rows, int64_t cols, int32_t blocksize,
                                 int32_t dq_blocksize, const float* B, const float* A, int32_t r, float alpha,
                                 uint8_t* packed_out, float* absmax_out, int8_t* qabsmax_out, float* dq_scale_out,
                                 void* stream) {
  return merge_impl(packed, absmax, qabsmax, dq_scale, rows, cols, blocksize, dq_blocksize, B, A, r, -alpha,
                    packed_out, absmax_out, qabsmax_out, dq_scale_out, stream);
}

size_t loftq_qlora_forward_workspace_bytes(int64_t n_tok, int32_t r) {
  if (n_tok < 0 || n_tok >= (int64_t(1) << 31) || r < 0 || r > 64) return 0;
  return qlora_forward_workspace_bytes(n_tok, r);
}

}  // extern "C"

namespace {
// Every argument check of the QLoRA forward, before anything is enqueued; LOFTQ_OK
// also for the empty shapes (n_tok = 0 or rows = 0), which launch nothing.
loftq_status_t loftq_qlora_forward_check(const void* X, int64_t n_tok, int64_t rows, int64_t cols,
                                         const uint8_t* packed, const float* absmax, const int8_t* qabsmax,
                                         const float* dq_scale, int32_t bits, const float* B, const float* A,
                                         int32_t r, float alpha, float* Y, void* ws, size_t ws_bytes) {
  if (!shape_ok(rows, cols) || n_tok < 0 || n_tok >= (int64_t(1) << 31)) return LOFTQ_ERR_INVALID_ARG;
  if (bits != 2 && bits != 3 && bits != 4) return LOFTQ_ERR_UNSUPPORTED;
  if (!nf_tables(bits).valid) return LOFTQ_ERR_UNSUPPORTED;
  const bool dq = qabsmax != nullptr || dq_scale != nullptr;
  if (dq && (!qabsmax || !dq_scale)) return LOFTQ_ERR_INVALID_ARG;
  if ((B == nullptr) != (A == nullptr)) return LOFTQ_ERR_INVALID_ARG;
  if (B != nullptr && r < 1) return LOFTQ_ERR_INVALID_ARG;
  if (!std::isfinite(alpha)) return LOFTQ_ERR_INVALID_ARG;
  if (n_tok == 0 || rows == 0) return LOFTQ_OK;   // nothing to write
  if (cols == 0 || cols % 64 != 0 || (B != nullptr && r > 64)) return LOFTQ_ERR_UNSUPPORTED;
  if (!qlora_forward_shape_ok(n_tok, rows, cols, B ? r : 0)) return LOFTQ_ERR_UNSUPPORTED;   // launch sizes
  if (!X || !packed || !Y || (!dq && !absmax)) return LOFTQ_ERR_INVALID_ARG;
  if (!aligned16(X) || !aligned16(packed) || !aligned16(Y)) return LOFTQ_ERR_INVALID_ARG;
  if (dq ? (!aligned16(qabsmax) || !aligned16(dq_scale)) : !aligned16(absmax)) return LOFTQ_ERR_INVALID_ARG;
  if (B != nullptr) {
    if (!aligned16(B) || !aligned16(A) || !ws || !aligned16(ws)) return LOFTQ_ERR_INVALID_ARG;
    if (ws_bytes < qlora_forward_workspace_bytes(n_tok, r)) return LOFTQ_ERR_WORKSPACE;
  }
  return LOFTQ_OK;
}
}  // namespace

extern "C" {

loftq_status_t loftq_qlora_forward(const void* X, int64_t n_tok, int64_t rows, int64_t cols, const uint8_t* packed,
                                   const float* absmax, const int8_t* qabsmax, const float* dq_scale, int32_t bits,
                                   const float* B, const float* A, int32_t r, float alpha, float* Y, void* ws,
                                   size_t ws_bytes, void* stream) {
  const loftq_status_t st = loftq_qlora_forward_check(X, n_tok, rows, cols, packed, absmax, qabsmax, dq_scale, bits,
                                                      B, A, r, alpha, Y, ws, ws_bytes);
  if (st != LOFTQ_OK || n_tok == 0 || rows == 0) return st;
  const bool dq = qabsmax != nullptr || dq_scale != nullptr;
  return from_hip(launch_qlora_forward(X, n_tok, rows, cols, packed, dq ? nullptr : absmax, dq ? qabsmax : nullptr,
                                       dq ? dq_scale : nullptr, bits, B, A, B ? r : 0, alpha, Y,
                                       static_cast<float*>(ws), static_cast<hipStream_t>(stream)));
}

size_t loftq_qlora_forward_noalloc_max_bytes(void) { return kStaticScratchBytes; }

loftq_status_t loftq_qlora_forward_noalloc(const void* X, int64_t n_tok, int64_t rows, int64_t cols,
                                           const uint8_t* packed, const float* absmax, const int8_t* qabsmax,
                                           const float* dq_scale, int32_t bits, const float* B, const float* A,
                                           int32_t r, float alpha, float* Y, void* stream) {
  // the adapter's partial products go to the library's own scratch instead of a
  // caller workspace; every other check is loftq_qlora_forward's
  size_t need = 0;
  if (B != nullptr && A != nullptr && n_tok > 0 && n_tok < (int64_t(1) << 31) && r >= 1 && r <= 64) {
    need = qlora_forward_workspace_bytes(n_tok, r);
    if (need > kStaticScratchBytes) return LOFTQ_ERR_WORKSPACE;
  }
  // a stand-in for the workspace only to pass the shared validation, which never
  // dereferences it; the launch below gets the scratch's device address
  void* const probe = reinterpret_cast<void*>(uintptr_t(256));
  loftq_status_t st = loftq_qlora_forward_check(X, n_tok, rows, cols, packed, absmax, qabsmax, dq_scale, bits, B, A,
                                                r, alpha, Y, need > 0 ? probe : nullptr, need);
  if (st != LOFTQ_OK || n_tok == 0 || rows == 0) return st;
  void* ws = nullptr;
  if (B != nullptr) {
    const hipError_t e = scratch_ptr(&ws);
    if (e != hipSuccess) return LOFTQ_ERR_HIP;
  }
  const bool dq = qabsmax != nullptr;
  return from_hip(launch_qlora_forward(X, n_tok, rows, cols, packed, dq ? nullptr : absmax, dq ? qabsmax : nullptr,
                                       dq ? dq_scale : nullptr, bits, B, A, B ? r : 0, alpha, Y,
                                       static_cast<float*>(ws), static_cast<hipStream_t>(stream)));
}

}  // extern "C"
