// Deterministic block-level reduction helpers.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace loftq {

// Sum of n doubles by the whole workgroup in a fixed order (strided per thread,
// then a fixed tree across lanes and waves); every thread gets the total.
__device__ inline double block_sum_fixed(const double* p, int n) {
  __shared__ double lq_bsum[16];
  const int tid = threadIdx.x, bs = blockDim.x;
  double a0 = 0.0, a1 = 0.0, a2 = 0.0, a3 = 0.0;
  int i = tid;
  for (; i + 3 * bs < n; i += 4 * bs) {
    a0 += p[i];
    a1 += p[i + bs];
    a2 += p[i + 2 * bs];
    a3 += p[i + 3 * bs];
  }
  for (; i < n; i += bs) a0 += p[i];
  double s = (a0 + a1) + (a2 + a3);
  for (int off = 32; off > 0; off >>= 1) s += __shfl_xor(s, off);
  if ((tid & 63) == 0) lq_bsum[tid >> 6] = s;
  __syncthreads();
  double tot = 0.0;
  for (int w = 0; w < (bs + 63) / 64; ++w) tot += lq_bsum[w];
  __syncthreads();
  return tot;
}

}  // namespace loftq
