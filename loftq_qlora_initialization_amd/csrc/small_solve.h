// Small fp64 solves shared by the low-rank kernels and the thin products:
// packed Gram indexing, fp64 reciprocal square root, the one-wave register
// Cholesky (with R^-1), and the workgroup that sums Gram partials and factors
// them while a thin product streams E.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace loftq {
namespace {

// Packed upper triangle, row by row: (a, b) with a <= b.
__device__ __forceinline__ int packed_index(int a, int b, int l) { return a * l - (a * (a - 1)) / 2 + (b - a); }

// 1/x and 1/sqrt(x) in fp64: hardware estimate plus two Newton steps.
__device__ __forceinline__ double rcp_f64(double x) {
  double r = __builtin_amdgcn_rcp(x);
  r = fma(r, fma(-x, r, 1.0), r);
  r = fma(r, fma(-x, r, 1.0), r);
  return r;
}
__device__ __forceinline__ double rsq_f64(double x) {
  double y = __builtin_amdgcn_rsq(x);
  y = y * fma(-0.5 * x * y, y, 1.5);
  y = y * fma(-0.5 * x * y, y, 1.5);
  return y;
}

// Cholesky by one wave (l <= LM <= 32): lane b keeps column b of the Gram
// (rows 0..LM-1) in registers.  Step j takes the pivot from lane j by
// readlane, scales row j (lane b then holds R[j][b]), publishes the row through
// LDS (one write by every lane, broadcast reads by all; a wave's LDS accesses
// are performed in order) and updates the trailing columns.  Entries below the
// diagonal pick up values that are never read back into the upper triangle and
// are dropped at the end.  For INV the same steps carry T = R^-T (lane b holds
// column b of T, starting from the identity): row j of T is divided by R[j][j]
// and rows a > j lose R[j][a] times it; then X = R^-1 = T^T, i.e. lane b holds
// row b of X.  A pivot at or below 1e-13 of the largest diagonal entry drops
// its direction (zero row of R, zero column of X).  rowbuf: LDS, 64 doubles
// per calling wave.
__device__ __forceinline__ double bcast_lane(double v, int lane) {
  const int lo = __builtin_amdgcn_readlane(__double2loint(v), lane);
  const int hi = __builtin_amdgcn_readlane(__double2hiint(v), lane);
  return __hiloint2double(hi, lo);
}

template <int LM, bool INV>
__device__ __forceinline__ void chol_wave(const double* __restrict__ gram, int l, double (&g)[LM], double (&t)[LM],
                                          double* rowbuf) {
  const int b = threadIdx.x & 63;
  // straight-line loads from clamped indices, then selects (no per-entry branches)
#pragma unroll
  for (int a = 0; a < LM; ++a) {
    const bool in = a <= b && b < l;
    const double v = gram[in ? packed_index(a, b, l) : 0];
    g[a] = in ? v : 0.0;
    if (INV) t[a] = (a == b) ? 1.0 : 0.0;
  }
  const double dv = gram[b < l ? packed_index(b, b, l) : 0];
  double dg = b < l ? dv : 0.0;
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) dg = fmax(dg, __shfl_xor(dg, off));
  const double tol = 1e-13 * dg;
#pragma unroll
  for (int j = 0; j < LM; ++j) {
    if (j < l) {
      const double piv = bcast_lane(g[j], j);
      const bool keep = piv > tol && piv > 0.0;
      const double inv = keep ? rsq_f64(piv) : 0.0;   // 1 / R[j][j]
      const double rjj = piv * inv;
      g[j] = b > j ? g[j] * inv : (b == j ? rjj : g[j]);
      if (INV) t[j] *= inv;
      rowbuf[b] = g[j];
      __builtin_amdgcn_wave_barrier();
#pragma unroll
      for (int a = j + 1; a < LM; ++a) {
        const double rja = rowbuf[a];
        g[a] = fma(-rja, g[j], g[a]);
        if (INV) t[a] = fma(-rja, t[j], t[a]);
      }
      __builtin_amdgcn_wave_barrier();
    }
  }
}

// Sum of the P fp64 Gram partials (packed upper triangles of E_ = l (l + 1) / 2
// entries, partial p at parts + p E_) by one workgroup of NW = blockDim / 64
// waves.  Wave w sums partials w, w + NW, w + 2 NW, ... of each entry in that
// order, QB partials' loads in flight at a time; the NW wave sums are then
// added in wave order, so the total is deterministic (and independent of QB).
// lds holds at least (NW + 1) E_ doubles; returns the address of the total
// (lds + NW E_).
template <int LM, int QB = 8>
__device__ __forceinline__ double* gram_sum_block(const double* __restrict__ parts, int P, int l, double* lds) {
  constexpr int EPL = (LM * (LM + 1) / 2 + 63) / 64;
  const int E_ = l * (l + 1) / 2;
  const int NW = static_cast<int>(blockDim.x >> 6);
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63;
  double s[EPL];
#pragma unroll
  for (int i = 0; i < EPL; ++i) s[i] = 0.0;
  for (int p = w; p < P; p += QB * NW) {
    double v[QB][EPL];
#pragma unroll
    for (int q = 0; q < QB; ++q)
#pragma unroll
      for (int i = 0; i < EPL; ++i) {
        const int pp = p + NW * q, e = lane + 64 * i;
        v[q][i] = (pp < P && e < E_) ? parts[static_cast<int64_t>(pp) * E_ + e] : 0.0;
      }
#pragma unroll
    for (int q = 0; q < QB; ++q)
#pragma unroll
      for (int i = 0; i < EPL; ++i) s[i] += v[q][i];
  }
#pragma unroll
  for (int i = 0; i < EPL; ++i) {
    const int e = lane + 64 * i;
    if (e < E_) lds[w * E_ + e] = s[i];
  }
  __syncthreads();
  double* gram = lds + NW * E_;
  for (int e = tid; e < E_; e += blockDim.x) {
    double t = lds[e];
    for (int q = 1; q < NW; ++q) t += lds[q * E_ + e];
    gram[e] = t;
  }
  __syncthreads();
  return gram;
}

template <int LM>
__device__ __forceinline__ void chol_inv_to(const double* gram, int l, float* __restrict__ Xinv, double* rowbuf) {
  double g[LM], t[LM];
  chol_wave<LM, true>(gram, l, g, t, rowbuf);
  const int lane = threadIdx.x & 63;
  if (lane < l) {
#pragma unroll
    for (int a = 0; a < LM; ++a)
      if (a < l) Xinv[lane * l + a] = static_cast<float>(t[a]);
  }
}

}  // namespace
}  // namespace loftq
