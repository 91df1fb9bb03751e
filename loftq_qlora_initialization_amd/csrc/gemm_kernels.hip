// Thin products of the randomized SVD on fp32 MFMA (v_mfma_f32_16x16x4_f32):
//   gemm_nn: part[s] = E[:, K_s] X[K_s, :]      (E d x k row-major, X k x l)
//   gemm_tn: part[s] = E[R_s, :]^T Y[R_s, :]    (Y d x l)
// Both stream E exactly once per product.  The skinny operand (X or Y) is held
// in fragment order (frag_index), so the B operand of one MFMA K-step group is a
// single coalesced float4 load per lane, read straight from L2/L1 — no LDS
// staging and no barrier in the main loop.  Each wave keeps D steps of E and of
// the skinny operand in flight in a register ring.  Waves of a workgroup that
// share output rows split the contraction and are summed through LDS at the
// end; split-K partials across workgroups are summed in fixed order by
// reduce_gram.
//
// Out-of-range rows/columns of E are clamped to valid addresses rather than
// branched around: the matching rows of the skinny operand are zero (its
// buffers are zero-padded to the splits' full extent), and garbage output
// rows/columns are never stored.
#include "lowrank.h"
#include "small_solve.h"

namespace loftq {
namespace {

typedef float floatx4 __attribute__((ext_vector_type(4)));

// v_mfma_f32_16x16x4_f32: lane L supplies A[L%16][L/16] and B[L/16][L%16];
// lane L receives D[4*(L/16)+v][L%16] in accumulator component v.
__device__ __forceinline__ floatx4 mfma16x16x4(float a, float b, floatx4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ float comp(const float4& v, int j) {
  return j == 0 ? v.x : (j == 1 ? v.y : (j == 2 ? v.z : v.w));
}

// Four consecutive floats of row `p` starting at column c (c % 4 == 0 when VEC),
// columns clamped into [0, n).
template <bool VEC>
__device__ __forceinline__ float4 load_run4(const float* __restrict__ p, int64_t c, int64_t n) {
  if (VEC) {
    c = c < n - 4 ? c : n - 4;
    return *reinterpret_cast<const float4*>(p + c);
  }
  float o[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int64_t ci = c + i < n ? c + i : n - 1;
    o[i] = p[ci];
  }
  return make_float4(o[0], o[1], o[2], o[3]);
}

// Launch shapes (compile-time per tile count NT = ceil(l / 16)).
template <int NT>
struct NnCfg {
  static constexpr int RT = 2;                 // 16-row MFMA tiles per wave (each X fragment feeds both)
  static constexpr int D = NT <= 2 ? 3 : 2;    // register ring depth (K steps of 16)
  static constexpr int WR = NT <= 2 ? 4 : 2;   // waves along rows
  static constexpr int WK = NT <= 2 ? 1 : 2;   // waves splitting the workgroup's K range
};
template <int NT>
struct TnCfg {
  static constexpr int D = 2;
  static constexpr int CW = 1;                 // 64-column groups per wave (each Y fragment feeds all)
  static constexpr int WC = 2;                 // waves along columns
  static constexpr int WR = 2;                 // waves splitting the workgroup's rows
};

// ---------------------------------------------------------------------------
// gemm_nn.  Wave (wr, wk) owns rows row0 .. row0 + 16 RT and the K range
// [kb, kb + kper / WK).  K step j covers k = kb + 16 j .. + 15: lane (li, g)
// loads E[row][kb + 16 j + 4 g .. + 3] per row tile and the fragment-order X
// float4 of (step, tile); MFMA s of the step uses component s of both, i.e.
// K index g <-> k = kb + 16 j + 4 g + s.
template <int NT, bool VEC>
__global__ __launch_bounds__(64 * NnCfg<NT>::WR * NnCfg<NT>::WK) void gemm_nn_kernel(
    const float* __restrict__ E, int64_t d, int64_t k, const float* __restrict__ Xf, int64_t kper,
    float* __restrict__ part) {
  using C = NnCfg<NT>;
  constexpr int LP = 16 * NT, RT = C::RT, D = C::D, WR = C::WR, WK = C::WK;
  __shared__ float red[(WK > 1 ? WK - 1 : 1) * WR * 16 * RT * LP];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, wr = w % WR, wk = w / WR;
  const int g = lane >> 4, li = lane & 15;
  const int64_t row0 = (static_cast<int64_t>(blockIdx.x) * WR + wr) * 16 * RT;
  const int64_t kw = kper / WK;
  const int64_t kb = static_cast<int64_t>(blockIdx.y) * kper + wk * kw;
  const int nsteps = static_cast<int>(kw / 16);   // a multiple of D
  const float* erow[RT];
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    int64_t r = row0 + rt * 16 + li;
    r = r < d ? r : d - 1;
    erow[rt] = E + r * k;
  }
  const float* xp = Xf + (kb / 16) * NT * 256 + lane * 4;
  floatx4 acc[RT][NT];
#pragma unroll
  for (int a = 0; a < RT; ++a)
#pragma unroll
    for (int b = 0; b < NT; ++b) acc[a][b] = floatx4{0.f, 0.f, 0.f, 0.f};
  float4 eb[D][RT], xb[D][NT];
  auto load = [&](int u, int j) {
    const int64_t c = kb + 16 * j + 4 * g;
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) eb[u][rt] = load_run4<VEC>(erow[rt], c, k);
#pragma unroll
    for (int nt = 0; nt < NT; ++nt)
      xb[u][nt] = *reinterpret_cast<const float4*>(xp + (static_cast<int64_t>(j) * NT + nt) * 256);
  };
  auto compute = [&](int u) {
#pragma unroll
    for (int s = 0; s < 4; ++s)
#pragma unroll
      for (int rt = 0; rt < RT; ++rt)
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) acc[rt][nt] = mfma16x16x4(comp(eb[u][rt], s), comp(xb[u][nt], s), acc[rt][nt]);
  };
#pragma unroll
  for (int u = 0; u < D; ++u) load(u, u);
  const int rounds = nsteps / D;
  for (int rd = 0; rd + 1 < rounds; ++rd) {
#pragma unroll
    for (int u = 0; u < D; ++u) {
      compute(u);
      load(u, (rd + 1) * D + u);
      // keep the slot's reload here: left to itself the scheduler sinks every
      // load below the last compute of the round, and the ring then hides no
      // memory latency behind the MFMAs
      __builtin_amdgcn_sched_barrier(0);
    }
  }
#pragma unroll
  for (int u = 0; u < D; ++u) compute(u);
  if (WK > 1) {
    if (wk > 0) {
#pragma unroll
      for (int rt = 0; rt < RT; ++rt)
#pragma unroll
        for (int nt = 0; nt < NT; ++nt)
#pragma unroll
          for (int v = 0; v < 4; ++v)
            red[(((wk - 1) * WR + wr) * 16 * RT + rt * 16 + 4 * g + v) * LP + nt * 16 + li] = acc[rt][nt][v];
    }
    __syncthreads();
    if (wk > 0) return;
#pragma unroll
    for (int q = 1; q < WK; ++q)
#pragma unroll
      for (int rt = 0; rt < RT; ++rt)
#pragma unroll
        for (int nt = 0; nt < NT; ++nt)
#pragma unroll
          for (int v = 0; v < 4; ++v)
            acc[rt][nt][v] += red[(((q - 1) * WR + wr) * 16 * RT + rt * 16 + 4 * g + v) * LP + nt * 16 + li];
  }
#pragma unroll
  for (int rt = 0; rt < RT; ++rt)
#pragma unroll
    for (int nt = 0; nt < NT; ++nt)
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int64_t row = row0 + rt * 16 + 4 * g + v;
        if (row < d) part[(static_cast<int64_t>(blockIdx.y) * d + row) * LP + nt * 16 + li] = acc[rt][nt][v];
      }
}

// ---------------------------------------------------------------------------
// gemm_tn.  Wave (wc, wr) owns columns c0 .. c0 + 64 CW - 1 and its share of
// the workgroup's rows: [rb, rb + rper / WR).  In column group cw, lane (li, g)
// covers columns c0 + 64 cw + 4 li .. + 3, which belong to four interleaved
// 16-column MFMA tiles (tile jm holds columns c0 + 64 cw + 4 m + jm).  Row step
// j covers rows rb + 16 j .. + 15; MFMA i of the step takes rows
// rb + 16 j + 4 g + i (K index g), matching component i of the fragment-order
// Y float4, which serves all CW groups.
template <int NT, bool VEC, int LMJ>
__global__ __launch_bounds__(64 * TnCfg<NT>::WC * TnCfg<NT>::WR) void gemm_tn_kernel(
    const float* __restrict__ E, int64_t d, int64_t k, const float* __restrict__ Yf, int64_t rper,
    float* __restrict__ part, CholJob job) {
  using C = TnCfg<NT>;
  constexpr int LP = 16 * NT, D = C::D, CW = C::CW, WC = C::WC, WR = C::WR;
  constexpr int kRedFloats = (WR > 1 ? WR - 1 : 1) * WC * 64 * CW * LP;
  constexpr int kJobDoubles = LMJ > 0 ? 5 * (LMJ * (LMJ + 1) / 2) + 64 : 1;
  constexpr int kLdsBytes = 4 * kRedFloats > 8 * kJobDoubles ? 4 * kRedFloats : 8 * kJobDoubles;
  __shared__ __align__(16) char lds_raw[kLdsBytes];
  float* red = reinterpret_cast<float*>(lds_raw);
  // LMJ > 0: the extra last column of workgroups carries a Cholesky job; its
  // row 0 sums the Gram partials of Y and factors them (X = R^-1 for the
  // reduction that follows this product), l <= LMJ.  The plan leaves a CU free
  // for it.
  if constexpr (LMJ > 0) {
    if (blockIdx.x == gridDim.x - 1) {
      if (blockIdx.y == 0) {
        double* lds = reinterpret_cast<double*>(lds_raw);
        const double* gram = gram_sum_block<LMJ>(job.parts, job.P, job.l, lds);
        if (threadIdx.x < 64) chol_inv_to<LMJ>(gram, job.l, job.Xinv, lds);
      }
      return;
    }
  }
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, wc = w % WC, wr = w / WC;
  const int g = lane >> 4, li = lane & 15;
  const int64_t c0 = (static_cast<int64_t>(blockIdx.x) * WC + wc) * 64 * CW;
  const int64_t cl = c0 + 4 * li;
  const int64_t rw = rper / WR;
  const int64_t rb = static_cast<int64_t>(blockIdx.y) * rper + wr * rw;
  const int nsteps = static_cast<int>(rw / 16);   // a multiple of D
  const float* yp = Yf + (rb / 16) * NT * 256 + lane * 4;
  floatx4 acc[CW][4][NT];
#pragma unroll
  for (int cw = 0; cw < CW; ++cw)
#pragma unroll
    for (int a = 0; a < 4; ++a)
#pragma unroll
      for (int b = 0; b < NT; ++b) acc[cw][a][b] = floatx4{0.f, 0.f, 0.f, 0.f};
  float4 eb[D][CW][4], yb[D][NT];
  auto load = [&](int u, int j) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      int64_t r = rb + 16 * j + 4 * g + i;
      r = r < d ? r : d - 1;
#pragma unroll
      for (int cw = 0; cw < CW; ++cw) eb[u][cw][i] = load_run4<VEC>(E + r * k, cl + 64 * cw, k);
    }
#pragma unroll
    for (int nt = 0; nt < NT; ++nt)
      yb[u][nt] = *reinterpret_cast<const float4*>(yp + (static_cast<int64_t>(j) * NT + nt) * 256);
  };
  auto compute = [&](int u) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int cw = 0; cw < CW; ++cw)
#pragma unroll
        for (int jm = 0; jm < 4; ++jm)
#pragma unroll
          for (int nt = 0; nt < NT; ++nt)
            acc[cw][jm][nt] = mfma16x16x4(comp(eb[u][cw][i], jm), comp(yb[u][nt], i), acc[cw][jm][nt]);
  };
#pragma unroll
  for (int u = 0; u < D; ++u) load(u, u);
  const int rounds = nsteps / D;
  for (int rd = 0; rd + 1 < rounds; ++rd) {
#pragma unroll
    for (int u = 0; u < D; ++u) {
      compute(u);
      load(u, (rd + 1) * D + u);
      // keep the slot's reload here: left to itself the scheduler sinks every
      // load below the last compute of the round, and the ring then hides no
      // memory latency behind the MFMAs
      __builtin_amdgcn_sched_barrier(0);
    }
  }
#pragma unroll
  for (int u = 0; u < D; ++u) compute(u);
  // lane (li, g), group cw, tile jm, component v holds column c0 + 64 cw + 4 (4 g + v) + jm,
  // output n = 16 nt + li
  if (WR > 1) {
    if (wr > 0) {
#pragma unroll
      for (int cw = 0; cw < CW; ++cw)
#pragma unroll
        for (int jm = 0; jm < 4; ++jm)
#pragma unroll
          for (int nt = 0; nt < NT; ++nt)
#pragma unroll
            for (int v = 0; v < 4; ++v)
              red[(((wr - 1) * WC + wc) * 64 * CW + 64 * cw + 4 * (4 * g + v) + jm) * LP + nt * 16 + li] =
                  acc[cw][jm][nt][v];
    }
    __syncthreads();
    if (wr > 0) return;
#pragma unroll
    for (int q = 1; q < WR; ++q)
#pragma unroll
      for (int cw = 0; cw < CW; ++cw)
#pragma unroll
        for (int jm = 0; jm < 4; ++jm)
#pragma unroll
          for (int nt = 0; nt < NT; ++nt)
#pragma unroll
            for (int v = 0; v < 4; ++v)
              acc[cw][jm][nt][v] +=
                  red[(((q - 1) * WC + wc) * 64 * CW + 64 * cw + 4 * (4 * g + v) + jm) * LP + nt * 16 + li];
  }
#pragma unroll
  for (int cw = 0; cw < CW; ++cw)
#pragma unroll
    for (int jm = 0; jm < 4; ++jm)
#pragma unroll
      for (int nt = 0; nt < NT; ++nt)
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const int64_t col = c0 + 64 * cw + 4 * (4 * g + v) + jm;
          if (col < k) part[(static_cast<int64_t>(blockIdx.y) * k + col) * LP + nt * 16 + li] = acc[cw][jm][nt][v];
        }
}

template <int NT>
GemmShape shape_typed(bool transposed) {
  if (transposed) {
    using C = TnCfg<NT>;
    return GemmShape{64 * C::CW * C::WC, 16 * C::D * C::WR};
  }
  using C = NnCfg<NT>;
  return GemmShape{16 * C::RT * C::WR, 16 * C::D * C::WK};
}

template <int NT>
void gemm_typed(bool transposed, const float* E, int64_t d, int64_t k, const float* panel, const SvdPlan& pl,
                float* part, const CholJob& job, hipStream_t s) {
  const bool vec = (k & 3) == 0 && k >= 4;
  if (transposed) {
    constexpr int threads = 64 * TnCfg<NT>::WC * TnCfg<NT>::WR;
    const dim3 grid(pl.tn_col_blocks + (job.parts != nullptr ? 1 : 0), pl.tn_splits);
#define LQ_TN(V, LMJ) \
  LQ_LAUNCH("gemm_tn", (gemm_tn_kernel<NT, V, LMJ>), grid, dim3(threads), 0, s, E, d, k, panel, pl.tn_rper, part, job)
    // register tile of the ride-along Cholesky: the smallest of 16 / 24 / 32 rows that holds l
    const int lmj = job.parts == nullptr ? 0 : (job.l <= 16 ? 16 : (job.l <= 24 ? 24 : 32));
    if constexpr (NT == 1) {
      if (vec) { if (lmj) LQ_TN(true, 16); else LQ_TN(true, 0); }
      else { if (lmj) LQ_TN(false, 16); else LQ_TN(false, 0); }
    } else if constexpr (NT == 2) {
      if (vec) { if (lmj == 16) LQ_TN(true, 16); else if (lmj == 24) LQ_TN(true, 24); else if (lmj) LQ_TN(true, 32); else LQ_TN(true, 0); }
      else { if (lmj == 16) LQ_TN(false, 16); else if (lmj == 24) LQ_TN(false, 24); else if (lmj) LQ_TN(false, 32); else LQ_TN(false, 0); }
    } else {
      if (vec) LQ_TN(true, 0); else LQ_TN(false, 0);
    }
#undef LQ_TN
  } else {
    constexpr int threads = 64 * NnCfg<NT>::WR * NnCfg<NT>::WK;
    const dim3 grid(pl.nn_row_blocks, pl.nn_splits);
    if (vec) LQ_LAUNCH("gemm_nn", (gemm_nn_kernel<NT, true>), grid, dim3(threads), 0, s, E, d, k, panel, pl.nn_kper, part);
    else LQ_LAUNCH("gemm_nn", (gemm_nn_kernel<NT, false>), grid, dim3(threads), 0, s, E, d, k, panel, pl.nn_kper, part);
  }
}

}  // namespace

GemmShape gemm_shape(bool transposed, int nt) {
  switch (nt) {
    case 1: return shape_typed<1>(transposed);
    case 2: return shape_typed<2>(transposed);
    case 3: return shape_typed<3>(transposed);
    case 4: return shape_typed<4>(transposed);
    default: return shape_typed<5>(transposed);
  }
}

void launch_gemm(bool transposed, const float* E, int64_t d, int64_t k, const float* panel, const SvdPlan& pl,
                 float* part, const CholJob& job, hipStream_t s) {
  const CholJob none{nullptr, 0, 0, nullptr};
  const CholJob& j = (transposed && pl.nt <= 2) ? job : none;
  switch (pl.nt) {
    case 1: gemm_typed<1>(transposed, E, d, k, panel, pl, part, j, s); break;
    case 2: gemm_typed<2>(transposed, E, d, k, panel, pl, part, j, s); break;
    case 3: gemm_typed<3>(transposed, E, d, k, panel, pl, part, j, s); break;
    case 4: gemm_typed<4>(transposed, E, d, k, panel, pl, part, j, s); break;
    default: gemm_typed<5>(transposed, E, d, k, panel, pl, part, j, s); break;
  }
}

}  // namespace loftq
