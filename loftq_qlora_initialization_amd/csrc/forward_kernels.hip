// QLoRA forward of one adapted layer on gfx950, the consumer of LoftQ's Q, B, A:
//   Y = X bf16(deq(Q))^T + alpha (X bf16(A)^T) bf16(B)^T
// ("参数高效微调：LoRA、Adapter 与 QLoRA" §2.2: the LoRA output adds to the frozen
// weight's, h = W x + B A x; §4.3: the 4-bit base computes in bfloat16).
// Tokens are rows: X n x cols (bf16), Y n x rows (fp32), W = deq(Q) rows x cols.
//
// lora_down_kernel  T = X bf16(A)^T (n x r, fp32) on bf16 MFMA (16x16x32), one
//                   16-token tile and all r columns per wave, straight from global.
// nf4_gemm_kernel   Y = X bf16(W)^T + alpha T bf16(B)^T: a 128 x 128 output tile per
//                   workgroup of 4 waves (64 x 64 each, 4 x 4 MFMA tiles), K in
//                   steps of 32.  Each step the workgroup stages X (bf16) and the
//                   weight decoded from NF4 codes (deq = fl32(c[code] a') exactly as
//                   in the dequantization, then rounded to bf16) in LDS, double
//                   buffered with one barrier per step; the next step's global
//                   loads are in flight while the current step's MFMAs run.  The
//                   epilogue adds the LoRA term in fp32.
//
// v_mfma_f32_16x16x32_bf16: lane L supplies A[L%16][8(L/16) + j] and
// B[8(L/16) + j][L%16] (j = 0..7) and receives D[4(L/16) + v][L%16] in element v.
#include "internal.h"

namespace loftq {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float mfma_f4 __attribute__((ext_vector_type(4)));

constexpr int kBM = 128, kBN = 128, kBK = 32, kLdsRow = kBK + 8;   // +8 bf16 per row against bank conflicts
constexpr int kGemmThreads = 256;

__device__ __forceinline__ int nib_shift16(int e) { return 8 * ((e >> 1) & 3) + ((e & 1) ? 0 : 4); }

template <bool kDQ>
__global__ __launch_bounds__(kGemmThreads) void nf4_gemm_kernel(const __bf16* __restrict__ X, int64_t M, int64_t N,
                                                                int64_t K, const uint8_t* __restrict__ packed,
                                                                const float* __restrict__ absmax,
                                                                const int8_t* __restrict__ qa,
                                                                const float* __restrict__ dqs,
                                                                const float* __restrict__ T, const float* __restrict__ B,
                                                                int r, float alpha, float* __restrict__ Y, Nf4Tables tab) {
  __shared__ __align__(16) __bf16 Xs[2][kBM][kLdsRow];
  __shared__ __align__(16) __bf16 Ws[2][kBN][kLdsRow];
  __shared__ float lvl[16];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, wm = w & 1, wn = w >> 1;
  const int li = lane & 15, lg = lane >> 4;
  if (tid < 16) lvl[tid] = tab.level[tid];
  const int64_t m0 = static_cast<int64_t>(blockIdx.y) * kBM, n0 = static_cast<int64_t>(blockIdx.x) * kBN;
  // this thread's share of one step: row `row` of the X and W tiles, 16 elements at column 16 half
  const int row = tid >> 1, half = tid & 1;
  const int64_t xr = (m0 + row < M) ? m0 + row : M - 1;   // clamped rows: loaded, never stored
  const int64_t wr = (n0 + row < N) ? n0 + row : N - 1;
  const uint4* xsrc = reinterpret_cast<const uint4*>(X + xr * K + 16 * half);
  const int64_t we0 = wr * K + 16 * half;                  // element index of this thread's 16 weights
  uint4 xv[2];
  uint2 wc;
  float sc;
  auto load = [&](int kt) {
    const int64_t k0 = static_cast<int64_t>(kt) * kBK;
    xv[0] = xsrc[k0 / 8];
    xv[1] = xsrc[k0 / 8 + 1];
    const int64_t e = we0 + k0;
    wc = *reinterpret_cast<const uint2*>(packed + (e >> 1));
    const int64_t b = e >> 6;
    sc = kDQ ? static_cast<float>(qa[b]) * dqs[b >> 8] : absmax[b];
  };
  auto store = [&](int buf) {
    uint4* xd = reinterpret_cast<uint4*>(&Xs[buf][row][16 * half]);
    xd[0] = xv[0];
    xd[1] = xv[1];
    bf16x8 o[2];
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const uint32_t code = ((e < 8 ? wc.x : wc.y) >> nib_shift16(e)) & 0xFu;
      o[e >> 3][e & 7] = static_cast<__bf16>(lvl[code] * sc);   // exact fp32 deq, then RNE to bf16
    }
    bf16x8* wd = reinterpret_cast<bf16x8*>(&Ws[buf][row][16 * half]);
    wd[0] = o[0];
    wd[1] = o[1];
  };
  mfma_f4 acc[4][4];
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int b = 0; b < 4; ++b) acc[a][b] = mfma_f4{0.f, 0.f, 0.f, 0.f};
  const int KT = static_cast<int>(K / kBK);
  __syncthreads();   // lvl
  load(0);
  store(0);
  __syncthreads();
  for (int kt = 0; kt < KT; ++kt) {
    const int buf = kt & 1;
    if (kt + 1 < KT) load(kt + 1);
    bf16x8 af[4], bfr[4];
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) af[mt] = *reinterpret_cast<const bf16x8*>(&Xs[buf][wm * 64 + mt * 16 + li][8 * lg]);
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) bfr[nt] = *reinterpret_cast<const bf16x8*>(&Ws[buf][wn * 64 + nt * 16 + li][8 * lg]);
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
      for (int nt = 0; nt < 4; ++nt)
        acc[mt][nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[mt], bfr[nt], acc[mt][nt], 0, 0, 0);
    if (kt + 1 < KT) store(buf ^ 1);
    __syncthreads();
  }
  // Epilogue.  Element v of tile (mt, nt) is token m = .. + 4 lg + v, feature n = .. + li.
  // The LoRA term T bf16(B)^T of the same 16 x 16 tile is one fp32 MFMA (16x16x4)
  // per 4 of r: lane L supplies T[m0 + L%16][p0 + L/16] and bf16(B)[n0 + L%16][p0 + L/16].
  const int64_t mw = m0 + wm * 64, nw = n0 + wn * 64;
#pragma unroll
  for (int mt = 0; mt < 4; ++mt) {
    mfma_f4 lora[4];
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) lora[nt] = mfma_f4{0.f, 0.f, 0.f, 0.f};
    if (T != nullptr) {
      const int64_t tm = mw + mt * 16 + li;
      for (int p0 = 0; p0 < r; p0 += 4) {
        const int p = p0 + lg;
        const float tv = (tm < M && p < r) ? T[tm * r + p] : 0.f;
#pragma unroll
        for (int nt = 0; nt < 4; ++nt) {
          const int64_t bn = nw + nt * 16 + li;
          const float bv = (bn < N && p < r) ? static_cast<float>(static_cast<__bf16>(B[bn * r + p])) : 0.f;
          lora[nt] = __builtin_amdgcn_mfma_f32_16x16x4f32(tv, bv, lora[nt], 0, 0, 0);
        }
      }
    }
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int64_t m = mw + mt * 16 + 4 * lg + v;
      if (m >= M) continue;
#pragma unroll
      for (int nt = 0; nt < 4; ++nt) {
        const int64_t n = nw + nt * 16 + li;
        if (n < N) Y[m * N + n] = fmaf(alpha, lora[nt][v], acc[mt][nt][v]);
      }
    }
  }
}

// T = X bf16(A)^T: wave = one 16-token tile, NT 16-column tiles of r.
template <int NT>
__global__ __launch_bounds__(256) void lora_down_kernel(const __bf16* __restrict__ X, int64_t M, int64_t K,
                                                        const float* __restrict__ A, int r, float* __restrict__ T) {
  const int lane = threadIdx.x & 63, li = lane & 15, lg = lane >> 4;
  const int64_t tile = (static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x) >> 6;
  const int64_t m0 = tile * 16;
  if (m0 >= M) return;
  const int64_t xr = (m0 + li < M) ? m0 + li : M - 1;
  mfma_f4 acc[NT];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) acc[nt] = mfma_f4{0.f, 0.f, 0.f, 0.f};
  for (int64_t k0 = 0; k0 < K; k0 += 32) {
    const bf16x8 a = *reinterpret_cast<const bf16x8*>(X + xr * K + k0 + 8 * lg);
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      const int p = nt * 16 + li;
      bf16x8 b;
      if (p < r) {
        const float4* src = reinterpret_cast<const float4*>(A + static_cast<int64_t>(p) * K + k0 + 8 * lg);
        const float4 u = src[0], q = src[1];
        b[0] = static_cast<__bf16>(u.x); b[1] = static_cast<__bf16>(u.y);
        b[2] = static_cast<__bf16>(u.z); b[3] = static_cast<__bf16>(u.w);
        b[4] = static_cast<__bf16>(q.x); b[5] = static_cast<__bf16>(q.y);
        b[6] = static_cast<__bf16>(q.z); b[7] = static_cast<__bf16>(q.w);
      } else {
        for (int j = 0; j < 8; ++j) b[j] = static_cast<__bf16>(0.f);
      }
      acc[nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, acc[nt], 0, 0, 0);
    }
  }
#pragma unroll
  for (int nt = 0; nt < NT; ++nt)
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int64_t m = m0 + 4 * lg + v;
      const int p = nt * 16 + li;
      if (m < M && p < r) T[m * r + p] = acc[nt][v];
    }
}

}  // namespace

size_t qlora_forward_workspace_bytes(int64_t n_tok, int r) {
  return static_cast<size_t>((n_tok * r * 4 + 255) / 256 * 256);
}

hipError_t launch_qlora_forward(const void* X, int64_t n_tok, int64_t rows, int64_t cols, const uint8_t* packed,
                                const float* absmax, const int8_t* qa, const float* dqs, int bits, const float* B,
                                const float* A, int r, float alpha, float* Y, float* Tws, hipStream_t s) {
  if (n_tok == 0 || rows == 0) return hipSuccess;
  if (cols % 64 != 0 || cols == 0) return hipErrorInvalidValue;
  const __bf16* Xb = static_cast<const __bf16*>(X);
  if (B != nullptr) {
    const int64_t tiles = (n_tok + 15) / 16;
    const dim3 grid(static_cast<unsigned>((tiles + 3) / 4));
    if (r <= 16) LQ_LAUNCH("lora_down", lora_down_kernel<1>, grid, dim3(256), 0, s, Xb, n_tok, cols, A, r, Tws);
    else if (r <= 32) LQ_LAUNCH("lora_down", lora_down_kernel<2>, grid, dim3(256), 0, s, Xb, n_tok, cols, A, r, Tws);
    else if (r <= 48) LQ_LAUNCH("lora_down", lora_down_kernel<3>, grid, dim3(256), 0, s, Xb, n_tok, cols, A, r, Tws);
    else LQ_LAUNCH("lora_down", lora_down_kernel<4>, grid, dim3(256), 0, s, Xb, n_tok, cols, A, r, Tws);
  }
  const dim3 grid(static_cast<unsigned>((rows + kBN - 1) / kBN), static_cast<unsigned>((n_tok + kBM - 1) / kBM));
  const Nf4Tables& tab = nf_tables(bits);
  const float* T = B != nullptr ? Tws : nullptr;
  if (qa != nullptr)
    LQ_LAUNCH("nf4_gemm", nf4_gemm_kernel<true>, grid, dim3(kGemmThreads), 0, s, Xb, n_tok, rows, cols, packed, absmax,
              qa, dqs, T, B, r, alpha, Y, tab);
  else
    LQ_LAUNCH("nf4_gemm", nf4_gemm_kernel<false>, grid, dim3(kGemmThreads), 0, s, Xb, n_tok, rows, cols, packed,
              absmax, qa, dqs, T, B, r, alpha, Y, tab);
  return hipGetLastError();
}

}  // namespace loftq
