// Rank-r SVD of the quantization residual E (d x k, fp32, row-major) on gfx950.
//
// The low-rank step of LoftQ takes the r largest singular triplets of W - Q
// ("LoftQ：协同优化量化与LoRA，实现高效大语言模型微调", §2.3).  Large matrices use
// randomized subspace iteration (Halko, Martinsson and Tropp 2011, Alg. 4.4/5.1):
//   Y = E Omega;  Q = orth(Y);  repeat q: Z = orth(E^T Q), Q = orth(E Z);
//   C = E^T Q;  the SVD of Q^T E = C^T comes from the eigen-decomposition of
//   C^T C (l x l, fp64), corrected for any residual non-orthogonality of Q.
// Tiny matrices use an exact one-sided Jacobi SVD of E itself.
//
// Kernels:
//   sketch        counter-based +-1 test matrix (SplitMix64)
//   gemm_nn       split-K partials of E X   (X: k x l), fp32 MFMA 16x16x4
//   gemm_tn       split-K partials of E^T Y (Y: d x l), fp32 MFMA 16x16x4
//   reduce_gram   sum of the split-K partials (fixed order) + fp64 Gram partials
//   chol_inv      fp64 Cholesky of a Gram matrix and the inverse of its factor
//   small_svd     single-workgroup fp64 Jacobi eigen-solver on the l x l core
//   panel_small   Q = P R^-1, B = Q S_B and A = (C S_A)^T (+ fp64 Gram partials)
//   exact_jacobi  single-workgroup one-sided Jacobi SVD for tiny matrices
// Every reduction runs in a fixed order, so results are deterministic.
#include "lowrank.h"

namespace loftq {
namespace {

typedef float floatx4 __attribute__((ext_vector_type(4)));

// v_mfma_f32_16x16x4_f32: lane L supplies A[L%16][L/16] and B[L/16][L%16];
// lane L receives D[4*(L/16)+v][L%16] in accumulator component v.
__device__ __forceinline__ floatx4 mfma16x16x4(float a, float b, floatx4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ void load4(const float* __restrict__ M, int64_t row, int64_t nrows, int64_t ld,
                                      int64_t c0, int64_t cend, bool vec_ok, float out[4]) {
  if (row < nrows && vec_ok && c0 + 3 < cend) {
    const float4 v = *reinterpret_cast<const float4*>(M + row * ld + c0);
    out[0] = v.x; out[1] = v.y; out[2] = v.z; out[3] = v.w;
  } else {
#pragma unroll
    for (int j = 0; j < 4; ++j) out[j] = (row < nrows && c0 + j < cend) ? M[row * ld + c0 + j] : 0.f;
  }
}

// ---------------------------------------------------------------------------
__global__ void sketch_kernel(uint64_t seed, int t, int64_t k, int l, float* __restrict__ out) {
  const int64_t idx = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (idx >= k * l) return;
  const uint64_t c = static_cast<uint64_t>(t - 1) * static_cast<uint64_t>(k) * static_cast<uint64_t>(l) +
                     static_cast<uint64_t>(idx);
  uint64_t z = seed + (c + 1) * 0x9E3779B97F4A7C15ull;
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  z ^= z >> 31;
  out[idx] = (z >> 63) ? -1.f : 1.f;
}

// ---------------------------------------------------------------------------
// part[s][i][n] = sum_{j in split s} E[i][j] X[j][n].  A workgroup is 4 waves on
// 64*RT consecutive rows and one K split; X's chunk is staged once in LDS and
// shared by the 4 waves.  Each lane loads 4 consecutive k of one row per 16-k
// sub-chunk and feeds them to 4 MFMAs (the k order inside a sub-chunk is a
// permutation, matched on the X side).
constexpr int kNnKc = 64;

template <int NT, int RT>
__global__ __launch_bounds__(256) void gemm_nn_kernel(const float* __restrict__ E, int64_t d, int64_t k,
                                                      const float* __restrict__ X, int l, int64_t kper,
                                                      float* __restrict__ part) {
  constexpr int LP = 16 * NT, XS = LP + 4;
  __shared__ float Xs[kNnKc * XS];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63, g = lane >> 4, li = lane & 15;
  const int64_t row_base = static_cast<int64_t>(blockIdx.x) * (64 * RT) + wave * (16 * RT);
  const int64_t kb = static_cast<int64_t>(blockIdx.y) * kper;
  const int64_t ke = (kb + kper < k) ? kb + kper : k;
  const bool vec_ok = (k & 3) == 0;
  floatx4 acc[RT][NT];
#pragma unroll
  for (int a = 0; a < RT; ++a)
#pragma unroll
    for (int b = 0; b < NT; ++b) acc[a][b] = floatx4{0.f, 0.f, 0.f, 0.f};

  for (int64_t kc = kb; kc < ke; kc += kNnKc) {
    __syncthreads();
    for (int idx = threadIdx.x; idx < kNnKc * LP; idx += 256) {
      const int kk = idx / LP, n = idx - kk * LP;
      const int64_t gk = kc + kk;
      Xs[kk * XS + n] = (gk < ke && n < l) ? X[gk * l + n] : 0.f;
    }
    __syncthreads();
#pragma unroll
    for (int sc = 0; sc < kNnKc / 16; ++sc) {
      const int64_t k0 = kc + sc * 16 + 4 * g;
      float a[RT][4];
#pragma unroll
      for (int rt = 0; rt < RT; ++rt) load4(E, row_base + rt * 16 + li, d, k, k0, ke, vec_ok, a[rt]);
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        float b[NT];
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) b[nt] = Xs[(sc * 16 + 4 * g + s) * XS + nt * 16 + li];
#pragma unroll
        for (int rt = 0; rt < RT; ++rt)
#pragma unroll
          for (int nt = 0; nt < NT; ++nt) acc[rt][nt] = mfma16x16x4(a[rt][s], b[nt], acc[rt][nt]);
      }
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

// part[s][j][n] = sum_{i in split s} E[i][j] Y[i][n].  A workgroup is 4 waves on
// 256 consecutive columns (64 per wave) and one row split; Y's row chunk is
// staged once in LDS.  A lane's float4 covers 4 columns that belong to 4
// interleaved 16-column MFMA tiles (tile j holds columns c0 + 4m + j).
constexpr int kTnRc = 64;

template <int NT>
__global__ __launch_bounds__(256) void gemm_tn_kernel(const float* __restrict__ E, int64_t d, int64_t k,
                                                      const float* __restrict__ Y, int l, int64_t rper,
                                                      float* __restrict__ part) {
  constexpr int LP = 16 * NT, YS = (LP % 32 == 0) ? LP + 16 : LP;
  __shared__ float Ys[kTnRc * YS];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63, g = lane >> 4, li = lane & 15;
  const int64_t col_base = static_cast<int64_t>(blockIdx.x) * 256 + wave * 64;
  const int64_t rb = static_cast<int64_t>(blockIdx.y) * rper;
  const int64_t re = (rb + rper < d) ? rb + rper : d;
  const bool vec_ok = (k & 3) == 0;
  floatx4 acc[4][NT];
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int b = 0; b < NT; ++b) acc[a][b] = floatx4{0.f, 0.f, 0.f, 0.f};

  for (int64_t rc = rb; rc < re; rc += kTnRc) {
    __syncthreads();
    for (int idx = threadIdx.x; idx < kTnRc * LP; idx += 256) {
      const int rr = idx / LP, n = idx - rr * LP;
      const int64_t gr = rc + rr;
      Ys[rr * YS + n] = (gr < re && n < l) ? Y[gr * l + n] : 0.f;
    }
    __syncthreads();
#pragma unroll 4
    for (int sub = 0; sub < kTnRc / 4; ++sub) {
      float a[4];
      load4(E, rc + sub * 4 + g, re, k, col_base + 4 * li, k, vec_ok, a);
      float b[NT];
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) b[nt] = Ys[(sub * 4 + g) * YS + nt * 16 + li];
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) acc[j][nt] = mfma16x16x4(a[j], b[nt], acc[j][nt]);
    }
  }
#pragma unroll
  for (int j = 0; j < 4; ++j)
#pragma unroll
    for (int nt = 0; nt < NT; ++nt)
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int64_t col = col_base + 4 * (4 * g + v) + j;
        if (col < k) part[(static_cast<int64_t>(blockIdx.y) * k + col) * LP + nt * 16 + li] = acc[j][nt][v];
      }
}

// ---------------------------------------------------------------------------
// Gram partial of kRows rows held in LDS (row stride ld): entries a <= b, fp64.
__device__ void gram_from_lds(const float* rows, int ld, int nrows, int l, double* out) {
  const int total = l * l;
  for (int e = threadIdx.x; e < total; e += blockDim.x) {
    const int a = e / l, b = e - a * l;
    if (b < a) continue;
    double s = 0.0;
    for (int rr = 0; rr < nrows; ++rr) s += static_cast<double>(rows[rr * ld + a]) * static_cast<double>(rows[rr * ld + b]);
    out[a * l + b] = s;
    out[b * l + a] = s;
  }
}

template <int NT>
__global__ __launch_bounds__(256) void reduce_gram_kernel(const float* __restrict__ part, int S, int64_t m, int l,
                                                          float* __restrict__ out, double* __restrict__ gram_parts) {
  constexpr int LP = 16 * NT;
  __shared__ float rows[kGramRows * (LP + 1)];
  const int64_t r0 = static_cast<int64_t>(blockIdx.x) * kGramRows;
  for (int idx = threadIdx.x; idx < kGramRows * LP; idx += blockDim.x) {
    const int rr = idx / LP, n = idx - rr * LP;
    const int64_t row = r0 + rr;
    float s = 0.f;
    if (row < m && n < l) {
      for (int p = 0; p < S; ++p) s += part[(static_cast<int64_t>(p) * m + row) * LP + n];
      out[row * l + n] = s;
    }
    rows[rr * (LP + 1) + n] = s;
  }
  if (gram_parts == nullptr) return;
  __syncthreads();
  gram_from_lds(rows, LP + 1, kGramRows, l, gram_parts + static_cast<int64_t>(blockIdx.x) * l * l);
}

// ---------------------------------------------------------------------------
// fp64 dense helpers on LDS matrices (row stride ld), whole workgroup.
__device__ void sum_parts(const double* __restrict__ parts, int nparts, int l, double* M, int ld) {
  for (int e = threadIdx.x; e < l * l; e += blockDim.x) {
    double s = 0.0;
    for (int p = 0; p < nparts; ++p) s += parts[static_cast<int64_t>(p) * l * l + e];
    M[(e / l) * ld + (e % l)] = s;
  }
}

// In-place upper Cholesky G = R^T R.  R's strict upper triangle replaces G's;
// its diagonal goes to rdiag.  A pivot at or below 1e-13 of the largest diagonal
// gives a zero row (that direction of the panel is dropped).
__device__ void chol_upper(double* G, int ld, int l, double* rdiag, double* scratch1) {
  if (threadIdx.x == 0) {
    double m = 0.0;
    for (int a = 0; a < l; ++a) m = fmax(m, G[a * ld + a]);
    scratch1[0] = m;
  }
  __syncthreads();
  const double tol = 1e-13 * scratch1[0];
  for (int j = 0; j < l; ++j) {
    const double piv = G[j * ld + j];
    const double rjj = (piv > tol && piv > 0.0) ? sqrt(piv) : 0.0;
    for (int c = j + 1 + threadIdx.x; c < l; c += blockDim.x) G[j * ld + c] = rjj > 0.0 ? G[j * ld + c] / rjj : 0.0;
    if (threadIdx.x == 0) rdiag[j] = rjj;
    __syncthreads();
    const int rem = l - j - 1;
    for (int idx = threadIdx.x; idx < rem * rem; idx += blockDim.x) {
      const int a = j + 1 + idx / rem, b = j + 1 + idx % rem;
      if (b >= a) G[a * ld + b] -= G[j * ld + a] * G[j * ld + b];
    }
    __syncthreads();
  }
}

// X = R^-1 (upper triangular) from chol_upper's output; zero rows stay zero.
__device__ void inv_upper(const double* G, int ld, int l, const double* rdiag, double* X, int ldx) {
  for (int c = threadIdx.x; c < l; c += blockDim.x) {
    X[c * ldx + c] = rdiag[c] > 0.0 ? 1.0 / rdiag[c] : 0.0;
    for (int a = c - 1; a >= 0; --a) {
      double s = 0.0;
      for (int b = a + 1; b <= c; ++b) s += G[a * ld + b] * X[b * ldx + c];
      X[a * ldx + c] = rdiag[a] > 0.0 ? -s / rdiag[a] : 0.0;
    }
    for (int a = c + 1; a < l; ++a) X[a * ldx + c] = 0.0;
  }
  __syncthreads();
}

__global__ __launch_bounds__(256) void chol_inv_kernel(const double* __restrict__ parts, int nparts, int l,
                                                       float* __restrict__ Rinv) {
  __shared__ double G[kMaxL * kMaxL];
  __shared__ double X[kMaxL * kMaxL];
  __shared__ double rdiag[kMaxL];
  __shared__ double tmp[1];
  sum_parts(parts, nparts, l, G, l);
  __syncthreads();
  chol_upper(G, l, l, rdiag, tmp);
  inv_upper(G, l, l, rdiag, X, l);
  for (int e = threadIdx.x; e < l * l; e += blockDim.x) Rinv[e] = static_cast<float>(X[e]);
}

// ---------------------------------------------------------------------------
// Round-robin (circle) schedule: position 0 is fixed, the others rotate.
__device__ __forceinline__ int rr_player(int pos, int rnd, int n) {
  return pos == 0 ? 0 : 1 + (pos - 1 + rnd) % (n - 1);
}

// The l x l core.  Inputs: Gram partials of Q (G_Q = Q^T Q) and of C = E^T Q
// (M = C^T C).  With R the Cholesky factor of G_Q, Q R^-1 is orthonormal and
// H = R^-T M R^-1 = (Q R^-1)^T E E^T (Q R^-1).  Cyclic Jacobi (round-robin pairs,
// fp64) diagonalises H = U diag(lambda) U^T while the rotations accumulate onto
// R^-1, giving V = R^-1 U.  Then sigma = sqrt(lambda) (descending) and
//   S_B = V_r diag(sigma^1/2),  S_A = V_r diag(sigma^-1/2),
// so B = Q S_B and A = (C S_A)^T.
__global__ __launch_bounds__(256) void small_svd_kernel(const double* __restrict__ gq_parts, int ngq,
                                                        const double* __restrict__ m_parts, int nm, int l, int r,
                                                        float* __restrict__ SB, float* __restrict__ SA,
                                                        float* __restrict__ sigma, double* __restrict__ stats,
                                                        ObjectiveArgs obj) {
  __shared__ double H[kMaxL * kMaxL];
  __shared__ double V[kMaxL * kMaxL];
  __shared__ double rdiag[kMaxL];
  __shared__ double pc[kMaxL / 2], ps[kMaxL / 2];
  __shared__ int pp[kMaxL / 2], pq[kMaxL / 2];
  __shared__ int order[kMaxL];
  __shared__ int rotated;
  __shared__ double tmp[1];
  const int n = l + (l & 1);
  const int tid = threadIdx.x, bs = blockDim.x;
  for (int e = tid; e < n * n; e += bs) { H[e] = 0.0; V[e] = 0.0; }
  __syncthreads();
  sum_parts(gq_parts, ngq, l, H, n);
  __syncthreads();
  chol_upper(H, n, l, rdiag, tmp);
  inv_upper(H, n, l, rdiag, V, n);
  for (int e = tid; e < n * n; e += bs) H[e] = 0.0;
  __syncthreads();
  sum_parts(m_parts, nm, l, H, n);
  __syncthreads();
  // T = M X in place, row by row from the right (X upper triangular)
  for (int a = tid; a < l; a += bs)
    for (int c = l - 1; c >= 0; --c) {
      double s = 0.0;
      for (int b = 0; b <= c; ++b) s += H[a * n + b] * V[b * n + c];
      H[a * n + c] = s;
    }
  __syncthreads();
  // H = X^T T in place, column by column from the bottom
  for (int c = tid; c < l; c += bs)
    for (int a = l - 1; a >= 0; --a) {
      double s = 0.0;
      for (int b = 0; b <= a; ++b) s += V[b * n + a] * H[b * n + c];
      H[a * n + c] = s;
    }
  __syncthreads();
  for (int e = tid; e < l * l; e += bs) {
    const int a = e / l, b = e % l;
    if (a < b) {
      const double s = 0.5 * (H[a * n + b] + H[b * n + a]);
      H[a * n + b] = s;
      H[b * n + a] = s;
    }
  }
  __syncthreads();

  for (int sweep = 0; sweep < 40; ++sweep) {
    if (tid == 0) rotated = 0;
    __syncthreads();
    for (int rnd = 0; rnd < n - 1; ++rnd) {
      for (int i = tid; i < n / 2; i += bs) {
        const int pa = rr_player(i, rnd, n), pb = rr_player(n - 1 - i, rnd, n);
        const int p = min(pa, pb), q = max(pa, pb);
        double c = 1.0, s = 0.0;
        if (q < l) {
          const double app = H[p * n + p], aqq = H[q * n + q], apq = H[p * n + q];
          if (apq != 0.0 && fabs(apq) > 1e-14 * sqrt(fabs(app * aqq))) {
            const double theta = (aqq - app) / (2.0 * apq);
            const double t = (theta >= 0.0 ? 1.0 : -1.0) / (fabs(theta) + sqrt(1.0 + theta * theta));
            c = 1.0 / sqrt(1.0 + t * t);
            s = t * c;
            rotated = 1;
          }
        }
        pc[i] = c; ps[i] = s; pp[i] = p; pq[i] = q;
      }
      __syncthreads();
      for (int idx = tid; idx < (n / 2) * n; idx += bs) {
        const int i = idx / n, j = idx - i * n;
        const double s = ps[i];
        if (s == 0.0) continue;
        const double c = pc[i];
        const int p = pp[i], q = pq[i];
        const double hp = H[p * n + j], hq = H[q * n + j];
        H[p * n + j] = c * hp - s * hq;
        H[q * n + j] = s * hp + c * hq;
      }
      __syncthreads();
      for (int idx = tid; idx < (n / 2) * n; idx += bs) {
        const int i = idx / n, j = idx - i * n;
        const double s = ps[i];
        if (s == 0.0) continue;
        const double c = pc[i];
        const int p = pp[i], q = pq[i];
        const double hp = H[j * n + p], hq = H[j * n + q];
        H[j * n + p] = c * hp - s * hq;
        H[j * n + q] = s * hp + c * hq;
        if (j == p) H[p * n + q] = 0.0;
        if (j == q) H[q * n + p] = 0.0;
        const double vp = V[j * n + p], vq = V[j * n + q];
        V[j * n + p] = c * vp - s * vq;
        V[j * n + q] = s * vp + c * vq;
      }
      __syncthreads();
    }
    if (!rotated) break;
    __syncthreads();
  }

  for (int a = tid; a < l; a += bs) {
    const double la = H[a * n + a];
    int rank = 0;
    for (int b = 0; b < l; ++b) {
      const double lb = H[b * n + b];
      rank += (lb > la || (lb == la && b < a)) ? 1 : 0;
    }
    order[rank] = a;
  }
  __syncthreads();
  for (int idx = tid; idx < l * r; idx += bs) {
    const int row = idx / r, c = idx - row * r;
    const int a = order[c];
    const double sg = sqrt(fmax(H[a * n + a], 0.0));
    const double sq = sqrt(sg);
    SB[row * r + c] = static_cast<float>(V[row * n + a] * sq);
    SA[row * r + c] = sg > 0.0 ? static_cast<float>(V[row * n + a] / sq) : 0.f;
  }
  for (int c = tid; c < r; c += bs) sigma[c] = static_cast<float>(sqrt(fmax(H[order[c] * n + order[c]], 0.0)));
  if (tid == 0) {
    double s2 = 0.0;
    for (int c = 0; c < r; ++c) s2 += fmax(H[order[c] * n + order[c]], 0.0);
    if (stats) stats[0] = s2;
    write_objective(obj, s2);
  }
}

// ---------------------------------------------------------------------------
// Panel times small matrix: out = P S (m x w) or its transpose (w x m), with P
// m x l and S l x w (upper triangular when `upper`).  64 rows of P and all of S
// are staged in LDS; optional fp64 Gram partials of the product.  Serves both
// Q = P R^-1 (orthonormalisation) and the factor products B = Q S_B and
// A = (C S_A)^T.
__global__ __launch_bounds__(256) void panel_small_kernel(const float* __restrict__ P, int64_t m, int l,
                                                          const float* __restrict__ S, int w, int upper,
                                                          float* __restrict__ out, int transpose_out,
                                                          double* __restrict__ gram_parts) {
  __shared__ float Ps[kPanelRows * (kMaxL + 1)];
  __shared__ float Ss[kMaxL * kMaxL];
  __shared__ float Os[kPanelRows * (kMaxL + 1)];
  const int64_t r0 = static_cast<int64_t>(blockIdx.x) * kPanelRows;
  const int ldp = l + 1, ldo = w + 1;
  for (int idx = threadIdx.x; idx < kPanelRows * l; idx += blockDim.x) {
    const int rr = idx / l, a = idx - rr * l;
    const int64_t row = r0 + rr;
    Ps[rr * ldp + a] = row < m ? P[row * l + a] : 0.f;
  }
  for (int idx = threadIdx.x; idx < l * w; idx += blockDim.x) Ss[idx] = S[idx];
  __syncthreads();
  for (int idx = threadIdx.x; idx < kPanelRows * w; idx += blockDim.x) {
    int rr, c;
    if (transpose_out) { rr = idx % kPanelRows; c = idx / kPanelRows; }
    else { rr = idx / w; c = idx - rr * w; }
    const int amax = upper ? (c + 1 < l ? c + 1 : l) : l;
    float acc = 0.f;
    for (int a = 0; a < amax; ++a) acc = fmaf(Ps[rr * ldp + a], Ss[a * w + c], acc);
    const int64_t row = r0 + rr;
    if (row < m) {
      if (transpose_out) out[static_cast<int64_t>(c) * m + row] = acc;
      else out[row * w + c] = acc;
    }
    Os[rr * ldo + c] = row < m ? acc : 0.f;
  }
  if (gram_parts == nullptr) return;
  __syncthreads();
  gram_from_lds(Os, ldo, kPanelRows, w, gram_parts + static_cast<int64_t>(blockIdx.x) * w * w);
}

// ---------------------------------------------------------------------------
// Exact SVD for tiny matrices: one-sided (Hestenes) Jacobi in fp64 on the n =
// min(d, k) vectors of length len = max(d, k) (columns of E when k <= d, rows of
// E otherwise), round-robin pairs, one wave per pair.
__global__ __launch_bounds__(1024) void exact_jacobi_kernel(const float* __restrict__ E, int64_t d, int64_t k, int r,
                                                            double* __restrict__ Xw, float* __restrict__ B,
                                                            float* __restrict__ A, float* __restrict__ sigma,
                                                            double* __restrict__ stats, ObjectiveArgs obj) {
  __shared__ double norm2[kMaxExact];
  __shared__ int order[kMaxExact];
  __shared__ int rotated;
  const bool trans = k > d;
  const int n = static_cast<int>(trans ? d : k);
  const int64_t len = trans ? k : d;
  const int N = n + (n & 1);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, nwaves = blockDim.x >> 6;
  for (int64_t e = tid; e < static_cast<int64_t>(N) * len; e += blockDim.x) {
    const int v = static_cast<int>(e / len);
    const int64_t i = e - static_cast<int64_t>(v) * len;
    double x = 0.0;
    if (v < n) x = trans ? E[static_cast<int64_t>(v) * k + i] : E[i * k + v];
    Xw[e] = x;
  }
  __syncthreads();
  for (int sweep = 0; sweep < 60; ++sweep) {
    if (tid == 0) rotated = 0;
    __syncthreads();
    for (int rnd = 0; rnd < N - 1; ++rnd) {
      for (int i = wave; i < N / 2; i += nwaves) {
        const int pa = rr_player(i, rnd, N), pb = rr_player(N - 1 - i, rnd, N);
        const int p = min(pa, pb), q = max(pa, pb);
        if (q >= n) continue;
        double* xp = Xw + static_cast<int64_t>(p) * len;
        double* xq = Xw + static_cast<int64_t>(q) * len;
        double al = 0.0, be = 0.0, ga = 0.0;
        for (int64_t e = lane; e < len; e += 64) {
          const double u = xp[e], w = xq[e];
          al += u * u; be += w * w; ga += u * w;
        }
        for (int off = 32; off > 0; off >>= 1) {
          al += __shfl_xor(al, off);
          be += __shfl_xor(be, off);
          ga += __shfl_xor(ga, off);
        }
        if (ga == 0.0 || fabs(ga) <= 1e-14 * sqrt(al * be)) continue;
        const double zeta = (be - al) / (2.0 * ga);
        const double t = (zeta >= 0.0 ? 1.0 : -1.0) / (fabs(zeta) + sqrt(1.0 + zeta * zeta));
        const double c = 1.0 / sqrt(1.0 + t * t), s = c * t;
        for (int64_t e = lane; e < len; e += 64) {
          const double u = xp[e], w = xq[e];
          xp[e] = c * u - s * w;
          xq[e] = s * u + c * w;
        }
        if (lane == 0) rotated = 1;
      }
      __syncthreads();
    }
    if (!rotated) break;
    __syncthreads();
  }
  for (int v = wave; v < n; v += nwaves) {
    const double* xv = Xw + static_cast<int64_t>(v) * len;
    double s = 0.0;
    for (int64_t e = lane; e < len; e += 64) s += xv[e] * xv[e];
    for (int off = 32; off > 0; off >>= 1) s += __shfl_xor(s, off);
    if (lane == 0) norm2[v] = s;
  }
  __syncthreads();
  for (int a = tid; a < n; a += blockDim.x) {
    const double la = norm2[a];
    int rank = 0;
    for (int b = 0; b < n; ++b) rank += (norm2[b] > la || (norm2[b] == la && b < a)) ? 1 : 0;
    order[rank] = a;
  }
  __syncthreads();
  // Vector x_j = sigma_j u_j (u_j a unit singular vector on the long side).
  // Long side factor: x_j / sqrt(sigma_j).  Short side: E-product with x_j times sigma_j^(-3/2).
  const int64_t other = trans ? d : k;
  for (int64_t e = tid; e < static_cast<int64_t>(r) * (len + other); e += blockDim.x) {
    const int c = static_cast<int>(e / (len + other));
    const int64_t i = e - static_cast<int64_t>(c) * (len + other);
    const int j = order[c];
    const double sg = sqrt(norm2[j]);
    const double* xj = Xw + static_cast<int64_t>(j) * len;
    if (i < len) {
      const float val = sg > 0.0 ? static_cast<float>(xj[i] / sqrt(sg)) : 0.f;
      if (trans) A[static_cast<int64_t>(c) * k + i] = val;
      else B[i * r + c] = val;
    } else {
      const int64_t o = i - len;
      double s = 0.0;
      if (trans) {
        for (int64_t t2 = 0; t2 < k; ++t2) s += static_cast<double>(E[o * k + t2]) * xj[t2];
      } else {
        for (int64_t t2 = 0; t2 < d; ++t2) s += static_cast<double>(E[t2 * k + o]) * xj[t2];
      }
      const float val = sg > 0.0 ? static_cast<float>(s / (sg * sqrt(sg))) : 0.f;
      if (trans) B[o * r + c] = val;
      else A[static_cast<int64_t>(c) * k + o] = val;
    }
  }
  if (tid < r) sigma[tid] = static_cast<float>(sqrt(norm2[order[tid]]));
  if (tid == 0) {
    double s2 = 0.0;
    for (int c = 0; c < r; ++c) s2 += norm2[order[c]];
    if (stats) stats[0] = s2;
    write_objective(obj, s2);
  }
}

__global__ void objective_kernel(ObjectiveArgs obj) {
  if (threadIdx.x == 0 && blockIdx.x == 0) write_objective(obj, 0.0);
}

__global__ void fill_kernel(float* __restrict__ p, int64_t n, float v) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i < n) p[i] = v;
}

// ---------------------------------------------------------------------------
template <int NT>
void gemm_nn_launch(const float* E, int64_t d, int64_t k, const float* X, int l, const SvdPlan& pl, float* part,
                    hipStream_t s) {
  if (NT <= 2)
    hipLaunchKernelGGL((gemm_nn_kernel<NT, 1>), dim3(pl.nn_row_blocks, pl.nn_splits), dim3(256), 0, s, E, d, k, X, l,
                       pl.nn_kper, part);
  else
    hipLaunchKernelGGL((gemm_nn_kernel<NT, 2>), dim3(pl.nn_row_blocks, pl.nn_splits), dim3(256), 0, s, E, d, k, X, l,
                       pl.nn_kper, part);
}

template <int NT>
struct Ops {
  static void product(bool transposed, const float* E, int64_t d, int64_t k, const float* panel, int l,
                      const SvdPlan& pl, float* part, float* out, double* gram, hipStream_t s) {
    const int64_t m = transposed ? k : d;
    if (transposed) {
      hipLaunchKernelGGL((gemm_tn_kernel<NT>), dim3(pl.tn_col_blocks, pl.tn_splits), dim3(256), 0, s, E, d, k, panel,
                         l, pl.tn_rper, part);
    } else {
      gemm_nn_launch<NT>(E, d, k, panel, l, pl, part, s);
    }
    const int S = transposed ? pl.tn_splits : pl.nn_splits;
    const int blocks = static_cast<int>((m + kGramRows - 1) / kGramRows);
    hipLaunchKernelGGL((reduce_gram_kernel<NT>), dim3(blocks), dim3(256), 0, s, part, S, m, l, out, gram);
  }
};

template <template <int> class F, typename... Args>
void dispatch_nt(int nt, Args... args) {
  switch (nt) {
    case 1: F<1>::run(args...); break;
    case 2: F<2>::run(args...); break;
    case 3: F<3>::run(args...); break;
    case 4: F<4>::run(args...); break;
    case 5: F<5>::run(args...); break;
    default: F<6>::run(args...); break;
  }
}

template <int NT>
struct ProductF {
  static void run(bool tr, const float* E, int64_t d, int64_t k, const float* panel, int l, const SvdPlan* pl,
                  float* part, float* out, double* gram, hipStream_t s) {
    Ops<NT>::product(tr, E, d, k, panel, l, *pl, part, out, gram, s);
  }
};
void panel_small(const float* P, int64_t m, int l, const float* S, int w, bool upper, float* out, bool tr,
                 double* gram, hipStream_t s) {
  const int blocks = static_cast<int>((m + kPanelRows - 1) / kPanelRows);
  hipLaunchKernelGGL(panel_small_kernel, dim3(blocks), dim3(256), 0, s, P, m, l, S, w, upper ? 1 : 0, out,
                     tr ? 1 : 0, gram);
}

int64_t round_up(int64_t x, int64_t m) { return (x + m - 1) / m * m; }
int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

}  // namespace

// ---------------------------------------------------------------------------
SvdPlan make_svd_plan(int64_t d, int64_t k, int r, int oversample, bool exact) {
  SvdPlan p{};
  p.d = d; p.k = k; p.r = r; p.exact = exact;
  if (exact) {
    const int64_t n = d < k ? d : k;
    p.l = static_cast<int>(n);
    p.bytes = 0;
    p.off_x = 0;
    p.bytes = round_up(static_cast<int64_t>(n + 1) * (d > k ? d : k) * 8, 256);
    p.off_stats = p.bytes;
    p.bytes += 256;
    return p;
  }
  const int l = r + oversample;
  p.l = l;
  p.nt = static_cast<int>(cdiv(l, 16));
  const int LP = 16 * p.nt;
  const int rt = p.nt <= 2 ? 1 : 2;
  const int64_t target = 768;
  p.nn_row_blocks = static_cast<int>(cdiv(d, 64 * rt));
  int64_t s_nn = cdiv(target, p.nn_row_blocks);
  int64_t max_s = k / 256 > 1 ? k / 256 : 1;
  if (s_nn > max_s) s_nn = max_s;
  if (s_nn < 1) s_nn = 1;
  p.nn_kper = round_up(cdiv(k, s_nn), kNnKc);
  p.nn_splits = static_cast<int>(cdiv(k, p.nn_kper));
  p.tn_col_blocks = static_cast<int>(cdiv(k, 256));
  int64_t s_tn = cdiv(target, p.tn_col_blocks);
  max_s = d / 128 > 1 ? d / 128 : 1;
  if (s_tn > max_s) s_tn = max_s;
  if (s_tn < 1) s_tn = 1;
  p.tn_rper = round_up(cdiv(d, s_tn), kTnRc);
  p.tn_splits = static_cast<int>(cdiv(d, p.tn_rper));
  p.gram_parts_d = static_cast<int>(cdiv(d, kGramRows));
  p.gram_parts_k = static_cast<int>(cdiv(k, kGramRows));
  p.gram_parts_qy = static_cast<int>(cdiv(d, kPanelRows));
  int64_t gp = p.gram_parts_d > p.gram_parts_k ? p.gram_parts_d : p.gram_parts_k;
  if (p.gram_parts_qy > gp) gp = p.gram_parts_qy;
  int64_t off = 0;
  auto take = [&](int64_t bytes) { const int64_t o = off; off += round_up(bytes, 256); return o; };
  p.off_omega = take(k * l * 4);
  p.off_y = take(d * l * 4);
  p.off_qy = take(d * l * 4);
  p.off_z = take(k * l * 4);
  p.off_qz = take(k * l * 4);
  const int64_t part_rows = (p.nn_splits * d > p.tn_splits * k) ? p.nn_splits * d : p.tn_splits * k;
  p.off_part = take(part_rows * LP * 4);
  p.off_gram1 = take(gp * l * l * 8);
  p.off_gram2 = take(gp * l * l * 8);
  p.off_rinv = take(static_cast<int64_t>(l) * l * 4);
  p.off_sb = take(static_cast<int64_t>(l) * r * 4);
  p.off_sa = take(static_cast<int64_t>(l) * r * 4);
  p.off_stats = take(64);
  p.bytes = off;
  return p;
}

hipError_t run_sketch(uint64_t seed, int t, int64_t k, int l, float* out, hipStream_t s) {
  const int64_t n = k * l;
  hipLaunchKernelGGL(sketch_kernel, dim3(static_cast<unsigned>(cdiv(n, 256))), dim3(256), 0, s, seed, t, k, l, out);
  return hipGetLastError();
}

hipError_t run_fill(float* p, int64_t n, float v, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(fill_kernel, dim3(static_cast<unsigned>(cdiv(n, 256))), dim3(256), 0, s, p, n, v);
  return hipGetLastError();
}

hipError_t run_objective(const ObjectiveArgs& obj, hipStream_t s) {
  hipLaunchKernelGGL(objective_kernel, dim3(1), dim3(64), 0, s, obj);
  return hipGetLastError();
}

hipError_t run_lowrank(const float* E, const SvdPlan& pl, int q, const float* omega, uint64_t seed, int t, float* B,
                       float* A, float* sigma, char* ws, const ObjectiveArgs& obj, hipStream_t s) {
  const int64_t d = pl.d, k = pl.k;
  const int r = pl.r, l = pl.l;
  if (pl.exact) {
    double* Xw = reinterpret_cast<double*>(ws + pl.off_x);
    hipLaunchKernelGGL(exact_jacobi_kernel, dim3(1), dim3(1024), 0, s, E, d, k, r, Xw, B, A, sigma,
                       reinterpret_cast<double*>(ws + pl.off_stats), obj);
    return hipGetLastError();
  }
  float* Om = reinterpret_cast<float*>(ws + pl.off_omega);
  float* Y = reinterpret_cast<float*>(ws + pl.off_y);
  float* Qy = reinterpret_cast<float*>(ws + pl.off_qy);
  float* Z = reinterpret_cast<float*>(ws + pl.off_z);
  float* Qz = reinterpret_cast<float*>(ws + pl.off_qz);
  float* part = reinterpret_cast<float*>(ws + pl.off_part);
  double* g1 = reinterpret_cast<double*>(ws + pl.off_gram1);
  double* g2 = reinterpret_cast<double*>(ws + pl.off_gram2);
  float* Rinv = reinterpret_cast<float*>(ws + pl.off_rinv);
  float* SB = reinterpret_cast<float*>(ws + pl.off_sb);
  float* SA = reinterpret_cast<float*>(ws + pl.off_sa);
  double* stats = reinterpret_cast<double*>(ws + pl.off_stats);
  const int nt = pl.nt;
  const float* X0 = omega;
  if (X0 == nullptr) {
    hipError_t e = run_sketch(seed, t, k, l, Om, s);
    if (e != hipSuccess) return e;
    X0 = Om;
  }
  // Y = E Omega; Q = orth(Y)
  dispatch_nt<ProductF>(nt, false, E, d, k, X0, l, &pl, part, Y, g1, s);
  hipLaunchKernelGGL(chol_inv_kernel, dim3(1), dim3(l <= 32 ? 64 : 256), 0, s, g1, pl.gram_parts_d, l, Rinv);
  for (int it = 0; it < q; ++it) {
    panel_small(Y, d, l, Rinv, l, true, Qy, false, nullptr, s);
    dispatch_nt<ProductF>(nt, true, E, d, k, Qy, l, &pl, part, Z, g1, s);
    hipLaunchKernelGGL(chol_inv_kernel, dim3(1), dim3(l <= 32 ? 64 : 256), 0, s, g1, pl.gram_parts_k, l, Rinv);
    panel_small(Z, k, l, Rinv, l, true, Qz, false, nullptr, s);
    dispatch_nt<ProductF>(nt, false, E, d, k, Qz, l, &pl, part, Y, g1, s);
    hipLaunchKernelGGL(chol_inv_kernel, dim3(1), dim3(l <= 32 ? 64 : 256), 0, s, g1, pl.gram_parts_d, l, Rinv);
  }
  // Q (with its Gram for the orthogonality correction), C = E^T Q with M = C^T C
  panel_small(Y, d, l, Rinv, l, true, Qy, false, g2, s);
  dispatch_nt<ProductF>(nt, true, E, d, k, Qy, l, &pl, part, Z, g1, s);
  hipLaunchKernelGGL(small_svd_kernel, dim3(1), dim3(l <= 32 ? 64 : 256), 0, s, g2, pl.gram_parts_qy, g1,
                     pl.gram_parts_k, l, r, SB, SA, sigma, stats, obj);
  panel_small(Qy, d, l, SB, r, false, B, false, nullptr, s);
  panel_small(Z, k, l, SA, r, false, A, true, nullptr, s);
  return hipGetLastError();
}

}  // namespace loftq
