/*
 * libloftq: LoftQ initialisation (NF4 + double quant + rank-r SVD) on one
 * AMD Instinct MI355X (gfx950).  C ABI.
 *
 * LoftQ initialises a quantized base Q and a LoRA adapter BA for each linear
 * layer W (d x k, y = W x) by alternately minimising ||W - (Q + BA)||_F:
 * quantize the residual W - BA with Delta = BA fixed, then refit BA as the
 * best rank-r approximation of W - Q with Q fixed ("LoftQ：协同优化量化与LoRA，
 * 实现高效大语言模型微调", §2.2-2.3).  Q is QLoRA's 4-bit NormalFloat with
 * blockwise absmax scaling and optional double quantization of the absmax
 * constants ("QLoRA论文概述", NF4 and double-quantization bullets; PEFT guide
 * "量化", BitsAndBytesConfig bullets).  Around the initialisation the library
 * also merges an adapter into the quantized weights and takes it out again
 * (PEFT guide "量化"), and runs the QLoRA forward of an adapted layer on the
 * bf16 matrix cores ("参数高效微调：LoRA、Adapter 与 QLoRA", §2.2 and §4.3).
 *
 * Conventions for every call:
 *   - Matrices are row-major.  W is rows x cols (d x k); B is rows x r and A is
 *     r x cols (LoRA's B in R^{d x r}, A in R^{r x k}, "参数高效微调：LoRA、Adapter
 *     与 QLoRA", §2.2).
 *   - Pointers marked [device] are device memory on the current HIP device;
 *     [host] pointers are host memory.  Device pointers must be 16-byte aligned.
 *   - The caller owns every buffer.  The library allocates no device memory on
 *     any call; scratch comes from the caller's workspace.
 *   - `stream` is a hipStream_t (NULL = the null stream).  Work is enqueued
 *     asynchronously; outputs are valid once the caller synchronises the
 *     stream.  Calls on different streams share no mutable state.
 *   - Arguments are validated before anything is enqueued; on any error no
 *     output is written.
 *   - Inputs must be finite (NaN/Inf give unspecified codes, never a fault).
 *   - NF4 block size is 64 consecutive elements of the row-major flattening;
 *     a ragged last block is allowed.  Packed codes hold two per byte, element
 *     2i in the high nibble; the byte count is ceil(rows*cols / 2).
 */
#ifndef LOFTQ_H
#define LOFTQ_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  LOFTQ_OK = 0,
  LOFTQ_ERR_INVALID_ARG = 1,  /* null pointer, bad size/shape, misalignment */
  LOFTQ_ERR_UNSUPPORTED = 2,  /* bits != 4, blocksize != 64, dq_blocksize != 256, too-large exact SVD */
  LOFTQ_ERR_WORKSPACE = 3,    /* workspace smaller than the *_workspace_bytes query */
  LOFTQ_ERR_HIP = 4           /* a HIP runtime call or kernel launch failed */
} loftq_status_t;

typedef enum { LOFTQ_F32 = 0, LOFTQ_BF16 = 1 } loftq_dtype_t;

/* Mirrors loftq_config {bits, iterative_steps, seed} and LoraConfig.r from the
 * LoftQ blog (§3.2) and bnb_4bit_use_double_quant from the PEFT guide. */
typedef struct {
  int32_t bits;             /* 4 (NF4), or 3 / 2 for lower-bit LoftQ (see loftq_nf_codebook) */
  int32_t iterative_steps;  /* T >= 0 alternations; 0 = plain NF4 (B = A = 0) */
  int32_t rank;             /* r >= 1 */
  int32_t blocksize;        /* must be 64 */
  int32_t double_quant;     /* 0 or 1 */
  int32_t dq_blocksize;     /* must be 256 */
  int32_t oversample;       /* p >= 0; sketch width l = r + p (randomized SVD) */
  int32_t power_iters;      /* q >= 0 subspace iterations (randomized SVD) */
  int32_t exact_svd;        /* 1: exact SVD (min(rows, cols) <= 512); 0: randomized */
  int32_t warm_start;       /* 0: a fresh +-1 sketch every alternation (the pages' method);
                               1: alternations t >= 2 start the subspace iteration from the
                               previous right singular vectors, Omega_t = [sqrt(cols) V_{t-1} |
                               the last oversample columns of the fresh sketch] (a variant, to be
                               paired with fewer power_iters; ignored with exact_svd) */
  uint64_t seed;            /* sketch seed (loftq_config seed, default 42) */
  int32_t init_from_BA;     /* 0: start from Delta_0 = 0.  k >= 1: resume after k completed
                               alternations (the LoftQ blog, §2.3, computes the initialisation once
                               and keeps the result): B and A hold B_k, A_k on entry (with
                               warm_start also sigma = sigma_k), and the call runs alternations
                               k+1 .. k+T with the sketch counter continuing at k+1, so k
                               alternations followed by a resumed call of T give the same results
                               as one call of k+T.  Requires T >= 1. */
  int32_t materialize_residual; /* 0 (default): the randomized SVD's products form E = W - deq(Q)
                               element by element from W and the codes as they stream them (cols
                               % 8 == 0; E is never stored, the workspace holds no copy of it);
                               1: the dequant stores E and the products read it.  Both give the
                               same results bit for bit; the exact SVD always stores E. */
} loftq_config_t;

/* Quantization step ("LoftQ...", §2.3: quantize the residual W - Delta; the
 * QLoRA blog "QLoRA技术解析...", §2.1: absmax-normalise then nearest codebook
 * entry).  R = W - B A (B, A both NULL: R = W), formed in fp32; per block of 64,
 * a = max |R| (absmax[b], fp32); x = fl32(R / a) (a = 0: x = 0); code = index of
 * the nearest NF4 level, ties to the lower index.
 *   W      [device] rows x cols of dtype wdt
 *   B, A   [device] fp32 rows x r and r x cols, or both NULL (then r is ignored)
 *   packed [device] ceil(rows*cols/2) bytes out
 *   absmax [device] ceil(rows*cols/64) fp32 out
 * Codes and absmax are bit-exact against an fp32 reference when B = A = NULL. */
loftq_status_t loftq_nf4_quantize(const void* W, loftq_dtype_t wdt, int64_t rows, int64_t cols,
                                  const float* B, const float* A, int32_t r, int32_t blocksize,
                                  uint8_t* packed, float* absmax, void* stream);

/* Double quantization ("QLoRA论文概述", double-quantization bullet: quantize the
 * quantization constants again).  Per group of dq_blocksize consecutive absmax
 * values (ragged last group allowed): s = fl32(max / 127),
 * q = clamp(rint_even(fl32(a / s)), 0, 127) (s = 0: q = 0); reconstruction
 * a' = fl32(q * s).
 *   absmax   [device] nblocks fp32 (non-negative)
 *   qabsmax  [device] nblocks int8 out
 *   dq_scale [device] ceil(nblocks/dq_blocksize) fp32 out */
loftq_status_t loftq_double_quant(const float* absmax, int64_t nblocks, int32_t dq_blocksize,
                                  int8_t* qabsmax, float* dq_scale, void* stream);

/* Dequantization, optionally fused with the subtraction W - deq(Q) that feeds
 * the low-rank step ("LoftQ...", §2.3: the SVD of W - Q).  deq = fl32(c[code]*a')
 * with a' = absmax[b] (qabsmax == NULL) or fl32(qabsmax[b] * dq_scale[b/dq_bs]);
 * out = deq (W == NULL) or fl32(W - deq).
 *   packed           [device] codes from loftq_nf4_quantize
 *   absmax           [device] or NULL when qabsmax/dq_scale are given
 *   qabsmax,dq_scale [device] or both NULL
 *   W                [device] or NULL
 *   out              [device] rows*cols fp32 out
 *   sumsq            [device] 1 double out (sum of out^2) or NULL */
loftq_status_t loftq_nf4_dequantize(const uint8_t* packed, const float* absmax, const int8_t* qabsmax,
                                    const float* dq_scale, int64_t rows, int64_t cols, int32_t blocksize,
                                    int32_t dq_blocksize, const void* W, loftq_dtype_t wdt, float* out,
                                    double* sumsq, void* stream);

/* Merging a LoRA adapter into NF4 weights and taking it out again (PEFT guide
 * "量化", merging adapters into quantized weights: dequantize the base weight, add
 * the adapter, quantize the sum again; unmerge does the reverse and is not an
 * exact inverse, so rounding accumulates over cycles).
 *   merge:   Q' = NF4(deq(Q) + alpha B A)        unmerge: Q' = NF4(deq(Q) - alpha B A)
 * deq(Q) as in loftq_nf4_dequantize; the sum is formed in fp32 (B A on fp32 matrix
 * cores) and quantized like any residual (blockwise-64 absmax, nearest level).
 *   packed                     [device] input codes
 *   absmax                     [device] input scales, or NULL when qabsmax/dq_scale are given
 *   qabsmax, dq_scale          [device] double-quantized input scales, or both NULL
 *   B, A                       [device] fp32 rows x r and r x cols (r <= 64), or both NULL
 *                              (then the codes are only requantized)
 *   alpha                      [host] adapter scale (finite)
 *   packed_out                 [device] ceil(rows*cols/2) bytes out; may be `packed`
 *   absmax_out                 [device] ceil(rows*cols/64) fp32 out (the new absmax); may be `absmax`
 *   qabsmax_out, dq_scale_out  [device] the double quant of absmax_out, or both NULL; may be
 *                              the input qabsmax / dq_scale
 * Buffers given as "may be" are either identical to the input or disjoint from it.
 * UNSUPPORTED: cols % 64 != 0, r > 64, blocksize != 64, dq_blocksize != 256. */
loftq_status_t loftq_nf4_merge(const uint8_t* packed, const float* absmax, const int8_t* qabsmax,
                               const float* dq_scale, int64_t rows, int64_t cols, int32_t blocksize,
                               int32_t dq_blocksize, const float* B, const float* A, int32_t r, float alpha,
                               uint8_t* packed_out, float* absmax_out, int8_t* qabsmax_out, float* dq_scale_out,
                               void* stream);
loftq_status_t loftq_nf4_unmerge(const uint8_t* packed, const float* absmax, const int8_t* qabsmax,
                                 const float* dq_scale, int64_t rows, int64_t cols, int32_t blocksize,
                                 int32_t dq_blocksize, const float* B, const float* A, int32_t r, float alpha,
                                 uint8_t* packed_out, float* absmax_out, int8_t* qabsmax_out, float* dq_scale_out,
                                 void* stream);

/* QLoRA forward of one adapted layer, the consumer of the initialisation
 * ("参数高效微调：LoRA、Adapter 与 QLoRA" §2.2: the adapter's output adds to the
 * frozen weight's, h = W x + B A x; §4.3: the 4-bit base computes in bfloat16):
 *   Y = X bf16(deq(Q))^T + alpha (X bf16(A)^T) bf16(B)^T
 * Tokens are rows.  deq(Q) is formed as in loftq_nf4_dequantize (bits-bit
 * NormalFloat codes in nibbles), then rounded to bf16; A and B are rounded to
 * bf16 (nearest, ties to even); products accumulate in fp32 on the bf16 matrix
 * cores; X A^T and Y stay fp32.
 *   X                  [device] n_tok x cols bf16, row-major
 *   packed             [device] codes of the rows x cols weight, as loftq_nf4_quantize
 *   absmax             [device] fp32 block scales, or NULL when qabsmax/dq_scale are given
 *   qabsmax, dq_scale  [device] double-quantized scales (groups of 256), or both NULL
 *   bits               [host] 2, 3 or 4 (the codebook of loftq_nf_codebook)
 *   B, A               [device] fp32 rows x r and r x cols (1 <= r <= 64), or both NULL
 *                      (then Y is the base product alone and ws may be NULL)
 *   alpha              [host] LoRA scaling (finite)
 *   Y                  [device] n_tok x rows fp32 out
 *   ws                 [device] loftq_qlora_forward_workspace_bytes(n_tok, r) bytes (partial
 *                      products X A^T over K ranges)
 * All device pointers 16-byte aligned.  n_tok = 0 or rows = 0 writes nothing.
 * UNSUPPORTED: cols % 64 != 0, r > 64, or a shape whose launches would exceed 2^32 work-items
 * (about 8.4 million tokens, or 2^26 output features with at most 64 tokens). */
loftq_status_t loftq_qlora_forward(const void* X, int64_t n_tok, int64_t rows, int64_t cols,
                                   const uint8_t* packed, const float* absmax, const int8_t* qabsmax,
                                   const float* dq_scale, int32_t bits, const float* B, const float* A,
                                   int32_t r, float alpha, float* Y, void* ws, size_t ws_bytes, void* stream);
size_t loftq_qlora_forward_workspace_bytes(int64_t n_tok, int32_t r);

/* loftq_qlora_forward for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc): the
 * same computation and arguments without the workspace.  The partial products of
 * X A^T go to a scratch array the library holds in device memory (one copy per
 * GPU, kept until the process ends); its device address is looked up on the first
 * call on each device.  Nothing is allocated or freed by any call.
 *   Limit: loftq_qlora_forward_workspace_bytes(n_tok, r) <= loftq_qlora_forward_noalloc_max_bytes()
 *          (8 MiB: n_tok * r <= 262144, e.g. 4096 tokens at r = 64); larger calls
 *          return LOFTQ_ERR_WORKSPACE and enqueue nothing.
 *   The current HIP device must be the one `stream` belongs to.  Calls on one GPU
 *   share its scratch: calls that may run at the same time on that GPU (other
 *   streams, other threads) race and must be ordered by the caller.  The scratch
 *   needs no clearing (each call writes every partial before reading it).
 * Errors otherwise as loftq_qlora_forward. */
loftq_status_t loftq_qlora_forward_noalloc(const void* X, int64_t n_tok, int64_t rows, int64_t cols,
                                           const uint8_t* packed, const float* absmax, const int8_t* qabsmax,
                                           const float* dq_scale, int32_t bits, const float* B, const float* A,
                                           int32_t r, float alpha, float* Y, void* stream);
size_t loftq_qlora_forward_noalloc_max_bytes(void);

/* Low-rank step ("LoftQ...", §2.3: best rank-r approximation of W - Q from its
 * r largest singular triplets, Delta = U_r S_r V_r^T).  exact = 1: the SVD of E
 * itself by one-sided (Hestenes) Jacobi on its min(rows, cols) <= 512 short-side
 * vectors (fp64), swept until a sweep finds every pair orthogonal to tol times the
 * product of their norms: when max(rows, cols) <= 576 the pairs are spread over
 * co-resident workgroups of one cooperative launch (tol = 1e-7), else one
 * workgroup runs them (tol = 1e-14).  exact = 0: randomized
 * subspace iteration with sketch width l = r + oversample (l <= min(rows, cols),
 * l <= 80, r <= 64) and power_iters rounds; the sketch is `omega` (cols x l fp32) or, if
 * NULL, the +-1 SplitMix64 sketch of (seed, t).  Outputs B = U_r S_r^{1/2},
 * A = S_r^{1/2} V_r^T, sigma = S_r (descending).
 * Accuracy of the randomized path: the products accumulate in fp32 and the range
 * panel is re-orthonormalised by one Cholesky-QR pass per power iteration (fp64
 * Gram and factor; E^T Q is never re-orthonormalised), so the weak directions of
 * the panel lose accuracy as the spectrum steepens.  The top-r singular values
 * stay within 1e-5 relative of the same algorithm in exact arithmetic while
 * sigma_1 / sigma_l <= 1e3 for l <= 32 (or power_iters >= 3) and <= 1e2 for
 * 32 < l <= 80 with power_iters = 2 (all three edges tested); past them the error
 * grows quickly (about 3e-4 at l = 80, q = 2, ratio 1e3).  Quantization
 * residuals lie far inside this range (nearly flat spectra).
 * An E of rank below l is supported: directions whose Cholesky pivot falls
 * under 1e-13 of the largest are dropped and their singular values come out 0.
 *   E      [device] rows x cols fp32
 *   B, A   [device] rows x r, r x cols fp32 out
 *   sigma  [device] r fp32 out
 *   ws     [device] loftq_lowrank_svd_workspace_bytes(...) bytes */
loftq_status_t loftq_lowrank_svd(const float* E, int64_t rows, int64_t cols, int32_t r, int32_t oversample,
                                 int32_t power_iters, int32_t exact, const float* omega, uint64_t seed,
                                 int32_t t, float* B, float* A, float* sigma, void* ws, size_t ws_bytes,
                                 void* stream);
size_t loftq_lowrank_svd_workspace_bytes(int64_t rows, int64_t cols, int32_t r, int32_t oversample,
                                         int32_t exact);

/* The whole initialisation ("LoftQ...", §2.3 and §3.2; PEFT guide "LoftQ 初始化"):
 * Delta_0 = 0; for t = 1..T: Q_t = NF4(W - B_{t-1} A_{t-1}) (+ double quant),
 * (B_t, A_t) = rank-r SVD of W - deq(Q_t).  Outputs the final Q_T (packed,
 * absmax, and qabsmax/dq_scale when double_quant), B_T, A_T, sigma of
 * alternation T, and objective[t] = ||W - deq(Q_t) - B_t A_t||_F / ||W||_F for
 * t = 1..T; objective[0] = ||W - deq(Q_first)|| / ||W|| for the call's first
 * quantization (the plain NF4 error when not resuming).  With cfg->init_from_BA
 * = k the alternations are numbered k+1 .. k+T and B, A (sigma) are read first.
 *   cfg               [host]
 *   packed, absmax    [device] as loftq_nf4_quantize
 *   qabsmax, dq_scale [device] as loftq_double_quant (ignored if !double_quant)
 *   B, A, sigma       [device] as loftq_lowrank_svd (also inputs when resuming)
 *   objective         [device] T+1 doubles out
 *   ws                [device] loftq_workspace_bytes(rows, cols, cfg) bytes
 * The randomized SVD's accuracy limit of loftq_lowrank_svd applies per alternation. */
loftq_status_t loftq_init(const void* W, loftq_dtype_t wdt, int64_t rows, int64_t cols,
                          const loftq_config_t* cfg, uint8_t* packed, float* absmax, int8_t* qabsmax,
                          float* dq_scale, float* B, float* A, double* objective, float* sigma, void* ws,
                          size_t ws_bytes, void* stream);
size_t loftq_workspace_bytes(int64_t rows, int64_t cols, const loftq_config_t* cfg);

/* One matrix of a batched initialisation: the device buffers loftq_init takes,
 * with the same meaning, shapes and alignment. */
typedef struct {
  const void* W;
  int64_t rows, cols;
  uint8_t* packed;
  float* absmax;
  int8_t* qabsmax;    /* and dq_scale: NULL unless cfg->double_quant */
  float* dq_scale;
  float* B;
  float* A;
  double* objective;  /* T+1 doubles */
  float* sigma;
} loftq_matrix_t;

/* LoftQ initialisation of every targeted linear layer of a model, one call for
 * the batch (PEFT guide "LoftQ 初始化": LoftQ applies to each linear layer the
 * LoRA config targets, all-linear advised; the LoftQ blog, §3.2, targets the
 * q/k/v/o/gate/up/down projections).  Each matrix gets exactly the results of
 * loftq_init with the same cfg (the same kernels; bit for bit).  The matrices
 * are spread over nstreams streams in an order that mixes large and small ones
 * (sorted by size, one from the large end and two from the small end in turn),
 * each to the stream with the least work so far; a stream runs its matrices one
 * after another in its own workspace, so one matrix's single-workgroup solves
 * overlap another's streaming kernels.  Nothing is synchronised: outputs are
 * valid once every stream is.
 *   mats      [host] count matrices; their output buffers must not overlap each
 *             other (W may be shared)
 *   wdt       storage type of every W
 *   cfg       [host] one configuration for all (rank, T, double quant, ...)
 *   nstreams  1 .. 16; all streams at the default priority
 *   streams   [host] nstreams hipStream_t, or NULL (then every matrix runs on the
 *             null stream, one after another)
 *   ws        [host] nstreams distinct device workspaces of ws_bytes each, ws_bytes
 *             >= loftq_batch_workspace_bytes(mats, count, cfg)
 * Every matrix is validated before anything is enqueued; any error from
 * loftq_init's list (for any matrix) returns that status and enqueues nothing. */
loftq_status_t loftq_init_batch(const loftq_matrix_t* mats, int32_t count, loftq_dtype_t wdt,
                                const loftq_config_t* cfg, int32_t nstreams, void* const* streams,
                                void* const* ws, size_t ws_bytes);
/* Bytes of one stream's workspace for loftq_init_batch (the largest loftq_workspace_bytes
 * over the batch); 0 if any matrix's shape or cfg is invalid. */
size_t loftq_batch_workspace_bytes(const loftq_matrix_t* mats, int32_t count, const loftq_config_t* cfg);

/* Fills cfg with the defaults (bits 4, T 5, r 16, blocksize 64, double quant on,
 * dq_blocksize 256, p 8, q 2, randomized, seed 42). [host] */
void loftq_default_config(loftq_config_t* cfg);

/* Static message for a status code. */
const char* loftq_status_string(loftq_status_t status);

/* The 16 NF4 levels the library uses, ascending (index 7 = 0). [host] out16 */
void loftq_nf4_codebook(float* out16);

/* The 2^bits k-bit NormalFloat levels (bits = 2, 3, 4; 4 is NF4), ascending, index
 * 2^(bits-1) - 1 = 0: NF4's quantile construction with 2^(bits-1) positive and
 * 2^(bits-1) - 1 negative levels and delta = 1 - (1/2^(bits+1) + 1/(2 (2^bits - 1)))/2
 * (the LoftQ blog, §3.2 and §4.3, reports 2- and 3-bit LoftQ without a codebook).
 * loftq_init with cfg->bits = 2 or 3 quantizes with these levels; each code is
 * stored in a nibble like an NF4 code. [host] out: 2^bits floats */
loftq_status_t loftq_nf_codebook(int32_t bits, float* out);

/* Kernel timing for measurement.  While enabled, every kernel the library
 * enqueues is bracketed by two HIP events recorded on that launch's stream
 * (no extra synchronisation is added to the stream).  loftq_profile_collect
 * waits for the recorded events, sums elapsed time per kernel name, clears the
 * records and returns the number of kernel names written (at most max_entries).
 *   names    [host] max_entries * 64 chars (NUL-terminated names), or NULL
 *   launches [host] max_entries launch counts, or NULL
 *   total_ms [host] max_entries summed durations in milliseconds, or NULL */
void loftq_profile_enable(int on);
int loftq_profile_collect(int max_entries, char* names, int64_t* launches, double* total_ms);
/* n launches of an empty kernel on `stream`, bracketed like the library's launches (recorded as
 * "event_overhead" while timing is enabled): the time a bracketed launch's events add to its kernel.
 * Returns 0, or 1 if a launch failed. */
int loftq_profile_calibrate(int n, void* stream);

#ifdef __cplusplus
}
#endif
#endif /* LOFTQ_H */
