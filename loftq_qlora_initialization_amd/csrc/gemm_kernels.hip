// Thin products of the randomized SVD on fp32 MFMA (v_mfma_f32_16x16x4_f32):
//   gemm_nn: part[s] = E[:, K_s] X[K_s, :]      (E d x k row-major, X k x l)
//   gemm_tn: part[s] = E[R_s, :]^T Y[R_s, :]    (Y d x l)
// Both stream E exactly once per product; the skinny operand (X or Y, at most a
// few MB) is staged through LDS and shared by the workgroup's waves.  E loads of
// the next chunk are issued before the MFMAs of the current one (register double
// buffering).  Split-K partials are summed in fixed order by reduce_gram.
#include "lowrank.h"

namespace loftq {
namespace {

typedef float floatx4 __attribute__((ext_vector_type(4)));

// v_mfma_f32_16x16x4_f32: lane L supplies A[L%16][L/16] and B[L/16][L%16];
// lane L receives D[4*(L/16)+v][L%16] in accumulator component v.
__device__ __forceinline__ floatx4 mfma16x16x4(float a, float b, floatx4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ float4 load4g(const float* __restrict__ M, int64_t row, int64_t nrows, int64_t ld,
                                         int64_t c0, int64_t cend, bool vec_ok) {
  if (row < nrows && vec_ok && c0 + 3 < cend) return *reinterpret_cast<const float4*>(M + row * ld + c0);
  float o[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) o[j] = (row < nrows && c0 + j < cend) ? M[row * ld + c0 + j] : 0.f;
  return make_float4(o[0], o[1], o[2], o[3]);
}

__device__ __forceinline__ float comp(const float4& v, int j) {
  return j == 0 ? v.x : (j == 1 ? v.y : (j == 2 ? v.z : v.w));
}

// ---------------------------------------------------------------------------
// gemm_nn: workgroup = 4 waves x (16 * RT) rows, one K split.  Per 128-wide K
// chunk a lane holds 8 float4 of E per row tile: float4 j covers k = kc + 16 j +
// 4 g .. +3 of row li (g = lane / 16, li = lane % 16).  MFMA step s of sub-chunk
// j uses component s, i.e. K index g <-> k = kc + 16 j + 4 g + s; the X operand
// is read from LDS with the same mapping.
template <int NT, int RT>
__global__ __launch_bounds__(256) void gemm_nn_kernel(const float* __restrict__ E, int64_t d, int64_t k,
                                                      const float* __restrict__ X, int l, int64_t kper,
                                                      float* __restrict__ part) {
  constexpr int LP = 16 * NT, XS = LP + 4, KC = kNnChunk, NJ = KC / 16;
  constexpr int XPER = (KC * LP + 255) / 256;
  __shared__ float Xs[KC * XS];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, g = lane >> 4, li = lane & 15;
  const int64_t row_base = static_cast<int64_t>(blockIdx.x) * (64 * RT) + wave * (16 * RT);
  const int64_t kb = static_cast<int64_t>(blockIdx.y) * kper;
  const int64_t ke = (kb + kper < k) ? kb + kper : k;
  const bool vec_ok = (k & 3) == 0;
  floatx4 acc[RT][NT];
#pragma unroll
  for (int a = 0; a < RT; ++a)
#pragma unroll
    for (int b = 0; b < NT; ++b) acc[a][b] = floatx4{0.f, 0.f, 0.f, 0.f};

  float4 ecur[RT][NJ], enext[RT][NJ];
  float xreg[XPER];
  auto load_e = [&](int64_t kc, float4 (&dst)[RT][NJ]) {
#pragma unroll
    for (int rt = 0; rt < RT; ++rt)
#pragma unroll
      for (int j = 0; j < NJ; ++j) dst[rt][j] = load4g(E, row_base + rt * 16 + li, d, k, kc + 16 * j + 4 * g, ke, vec_ok);
  };
  auto load_x = [&](int64_t kc) {
#pragma unroll
    for (int u = 0; u < XPER; ++u) {
      const int idx = tid + 256 * u;
      const int kk = idx / LP, n = idx - kk * LP;
      const int64_t gk = kc + kk;
      xreg[u] = (idx < KC * LP && gk < ke && n < l) ? X[gk * l + n] : 0.f;
    }
  };
  if (kb < ke) {
    load_e(kb, ecur);
    load_x(kb);
  }
  for (int64_t kc = kb; kc < ke; kc += KC) {
    __syncthreads();
#pragma unroll
    for (int u = 0; u < XPER; ++u) {
      const int idx = tid + 256 * u;
      if (idx < KC * LP) {
        const int kk = idx / LP, n = idx - kk * LP;
        Xs[kk * XS + n] = xreg[u];
      }
    }
    __syncthreads();
    const bool more = kc + KC < ke;
    if (more) {
      load_e(kc + KC, enext);
      load_x(kc + KC);
    }
#pragma unroll
    for (int j = 0; j < NJ; ++j)
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        float b[NT];
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) b[nt] = Xs[(16 * j + 4 * g + s) * XS + nt * 16 + li];
#pragma unroll
        for (int rt = 0; rt < RT; ++rt)
#pragma unroll
          for (int nt = 0; nt < NT; ++nt) acc[rt][nt] = mfma16x16x4(comp(ecur[rt][j], s), b[nt], acc[rt][nt]);
      }
    if (more) {
#pragma unroll
      for (int rt = 0; rt < RT; ++rt)
#pragma unroll
        for (int j = 0; j < NJ; ++j) ecur[rt][j] = enext[rt][j];
    }
  }
#pragma unroll
  for (int rt = 0; rt < RT; ++rt)
#pragma unroll
    for (int nt = 0; nt < NT; ++nt)
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int64_t row = row_base + rt * 16 + 4 * g + v;
        if (row < d) part[(static_cast<int64_t>(blockIdx.y) * d + row) * LP + nt * 16 + li] = acc[rt][nt][v];
      }
}

// ---------------------------------------------------------------------------
// gemm_tn: workgroup = 2 column tiles (64 columns each) x 2 row groups, one row
// split of `rper` rows; each row group walks half of the split's rows, and the
// two row groups' accumulators are summed through LDS at the end.  A lane's
// float4 covers 4 columns that belong to 4 interleaved 16-column MFMA tiles
// (tile j holds columns c0 + 4m + j); K index g <-> row r0 + 4 i + g.
template <int NT>
__global__ __launch_bounds__(256) void gemm_tn_kernel(const float* __restrict__ E, int64_t d, int64_t k,
                                                      const float* __restrict__ Y, int l, int64_t rper,
                                                      float* __restrict__ part) {
  constexpr int LP = 16 * NT, YS = (LP % 32 == 0) ? LP + 16 : LP, RC = kTnChunk, NI = RC / 4;
  constexpr int YPER = (RC * LP + 127) / 128;
  __shared__ float Ys[2][RC * YS];
  __shared__ float Red[2][64 * LP];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, g = lane >> 4, li = lane & 15;
  const int ct = wave & 1, rg = wave >> 1;       // column tile, row group
  const int ltid = tid & 127;                    // thread index within the row group's two waves
  const int64_t col_base = static_cast<int64_t>(blockIdx.x) * 128 + ct * 64;
  const int64_t rb = static_cast<int64_t>(blockIdx.y) * rper;
  const int64_t re_split = (rb + rper < d) ? rb + rper : d;
  const int64_t half = ((rper / 2) + RC - 1) / RC * RC;
  const int64_t r_lo = rb + rg * half;
  const int64_t r_hi = (rg == 0) ? ((rb + half < re_split) ? rb + half : re_split) : re_split;
  const bool vec_ok = (k & 3) == 0;
  floatx4 acc[4][NT];
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int b = 0; b < NT; ++b) acc[a][b] = floatx4{0.f, 0.f, 0.f, 0.f};

  float4 ecur[NI], enext[NI];
  float yreg[YPER];
  auto load_e = [&](int64_t rc, float4 (&dst)[NI]) {
#pragma unroll
    for (int i = 0; i < NI; ++i) dst[i] = load4g(E, rc + 4 * i + g, r_hi, k, col_base + 4 * li, k, vec_ok);
  };
  auto load_y = [&](int64_t rc) {
#pragma unroll
    for (int u = 0; u < YPER; ++u) {
      const int idx = ltid + 128 * u;
      const int rr = idx / LP, n = idx - rr * LP;
      const int64_t gr = rc + rr;
      yreg[u] = (idx < RC * LP && gr < r_hi && n < l) ? Y[gr * l + n] : 0.f;
    }
  };
  // both row groups run the same number of chunk iterations (barriers are uniform)
  const int64_t nchunks = (half + RC - 1) / RC;
  if (r_lo < r_hi) {
    load_e(r_lo, ecur);
    load_y(r_lo);
  }
  for (int64_t c = 0; c < nchunks; ++c) {
    const int64_t rc = r_lo + c * RC;
    const bool active = rc < r_hi;
    __syncthreads();
    if (active) {
#pragma unroll
      for (int u = 0; u < YPER; ++u) {
        const int idx = ltid + 128 * u;
        if (idx < RC * LP) {
          const int rr = idx / LP, n = idx - rr * LP;
          Ys[rg][rr * YS + n] = yreg[u];
        }
      }
    }
    __syncthreads();
    if (!active) continue;
    const bool more = rc + RC < r_hi;
    if (more) {
      load_e(rc + RC, enext);
      load_y(rc + RC);
    }
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      float b[NT];
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) b[nt] = Ys[rg][(4 * i + g) * YS + nt * 16 + li];
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) acc[j][nt] = mfma16x16x4(comp(ecur[i], j), b[nt], acc[j][nt]);
    }
    if (more) {
#pragma unroll
      for (int i = 0; i < NI; ++i) ecur[i] = enext[i];
    }
  }
  // row group 1 hands its accumulators to row group 0 through LDS
  __syncthreads();
  if (rg == 1) {
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int nt = 0; nt < NT; ++nt)
#pragma unroll
        for (int v = 0; v < 4; ++v) Red[ct][(4 * (4 * g + v) + j) * LP + nt * 16 + li] = acc[j][nt][v];
  }
  __syncthreads();
  if (rg == 0) {
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int nt = 0; nt < NT; ++nt)
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const int cl = 4 * (4 * g + v) + j;
          const int64_t col = col_base + cl;
          const float val = acc[j][nt][v] + Red[ct][cl * LP + nt * 16 + li];
          if (col < k) part[(static_cast<int64_t>(blockIdx.y) * k + col) * LP + nt * 16 + li] = val;
        }
  }
}

template <int NT>
void gemm_typed(bool transposed, const float* E, int64_t d, int64_t k, const float* panel, int l, const SvdPlan& pl,
                float* part, hipStream_t s) {
  if (transposed) {
    LQ_LAUNCH("gemm_tn", (gemm_tn_kernel<NT>), dim3(pl.tn_col_blocks, pl.tn_splits), dim3(256), 0, s, E, d, k,
              panel, l, pl.tn_rper, part);
  } else if (NT <= 2) {
    LQ_LAUNCH("gemm_nn", (gemm_nn_kernel<NT, 1>), dim3(pl.nn_row_blocks, pl.nn_splits), dim3(256), 0, s, E, d, k,
              panel, l, pl.nn_kper, part);
  } else {
    LQ_LAUNCH("gemm_nn", (gemm_nn_kernel<NT, 2>), dim3(pl.nn_row_blocks, pl.nn_splits), dim3(256), 0, s, E, d, k,
              panel, l, pl.nn_kper, part);
  }
}

}  // namespace

void launch_gemm(bool transposed, const float* E, int64_t d, int64_t k, const float* panel, int l, const SvdPlan& pl,
                 float* part, hipStream_t s) {
  switch (pl.nt) {
    case 1: gemm_typed<1>(transposed, E, d, k, panel, l, pl, part, s); break;
    case 2: gemm_typed<2>(transposed, E, d, k, panel, l, pl, part, s); break;
    case 3: gemm_typed<3>(transposed, E, d, k, panel, l, pl, part, s); break;
    case 4: gemm_typed<4>(transposed, E, d, k, panel, l, pl, part, s); break;
    default: gemm_typed<5>(transposed, E, d, k, panel, l, pl, part, s); break;
  }
}

}  // namespace loftq
