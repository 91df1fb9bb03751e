// C-ABI entry points for the NF4 codec: argument validation, then launches.
#include <cstring>

#include "internal.h"

namespace loftq {

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

}  // extern "C"
