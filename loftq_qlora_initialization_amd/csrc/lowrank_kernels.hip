// Rank-r SVD of the quantization residual E (d x k, fp32, row-major) on gfx950.
//
// The low-rank step of LoftQ takes the r largest singular triplets of W - Q
// ("LoftQ：协同优化量化与LoRA，实现高效大语言模型微调", §2.3).  Large matrices use
// randomized subspace iteration (Halko, Martinsson and Tropp 2011, Alg. 4.4/5.1):
//   Y = E Omega;  Q = orth(Y);  repeat q: Z = E^T Q, Q = orth(E Z);
//   C = E^T Q;  the SVD of Q^T E = C^T comes from the eigen-decomposition of
//   C^T C (l x l, fp64).
// orth(Y) is CholQR: fp64 Gram Y^T Y = R^T R (fp64 Cholesky), Q = Y R^-1.  Q is
// never formed: E^T Q = (E^T Y) R^-1 is applied to the summed rows of E^T Y in
// the split-K reduction, and B = Q S_B = Y (R^-1 S_B).
// Tiny matrices use an exact one-sided Jacobi SVD of E itself.
//
// Kernels (besides the thin products in gemm_kernels.hip):
//   sketch        counter-based +-1 test matrix (SplitMix64), in fragment order
//                 or straight in the products' split layout
//   reduce_gram   fixed-order sum of the split-K partials, the X = R^-1 product,
//                 fp64 Gram partials and the next product's split operand
//   gram_sum      fixed-order sum of the Gram partials
//   chol_inv      Cholesky of the Gram and X = R^-1 (orthonormalisation); for
//                 l <= 32 it usually rides along with the next E^T Y product
//   core_svd      the l x l core solve: Cholesky, one-sided Jacobi, S_B, S_A
//   panel_small   P S for a row panel P and a small S: B = Q S_B, A = (C S_A)^T
//   exact SVD     block one-sided Jacobi over co-resident workgroups (bj_*), or
//                 one workgroup (exact_jacobi) for vectors too long for its LDS
// Every reduction runs in a fixed order, so results are deterministic.
#include <map>
#include <mutex>
#include <utility>

#include "lowrank.h"
#include "reduce.h"
#include "small_solve.h"
#include "split_bf16.h"

namespace loftq {
namespace {

// ---------------------------------------------------------------------------
// Element (i, j) of the k x l test matrix of alternation t is drawn from
// counter ((t - 1) k + i) l + j; written in fragment order over `rows` rows
// (zero beyond k and l).
__device__ __forceinline__ float rademacher(uint64_t seed, int t, int64_t k, int l, int64_t i, int j) {
  const uint64_t c = (static_cast<uint64_t>(t - 1) * static_cast<uint64_t>(k) + static_cast<uint64_t>(i)) *
                         static_cast<uint64_t>(l) + static_cast<uint64_t>(j);
  uint64_t z = seed + (c + 1) * 0x9E3779B97F4A7C15ull;
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  z ^= z >> 31;
  return (z >> 63) ? -1.f : 1.f;
}

// The same test matrices straight in the split layout of the bf16 products
// (split_index over `rows` rows, a multiple of 32): +-1 is exact in bf16, so
// hi = the value and lo = 0.  One thread per (step, tile, part, lane): 8 values.
__global__ void sketch_split_kernel(uint64_t seed, int t0, int64_t k, int l, int nt, int64_t rows,
                                    uint16_t* __restrict__ out) {
  const int64_t u = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  const int64_t per = (rows >> 5) * nt * 2 * 64;
  if (u >= per) return;
  const int t = t0 + static_cast<int>(blockIdx.y);
  const int L = static_cast<int>(u & 63);
  const int64_t stp = u >> 6;                     // (step * nt + tile) * 2 + part
  const int part = static_cast<int>(stp & 1);
  const int64_t st_tile = stp >> 1;
  const int64_t step = st_tile / nt;
  const int tile = static_cast<int>(st_tile - step * nt);
  const int j = 16 * tile + (L & 15);
  uint32_t h[4] = {0u, 0u, 0u, 0u};
  if (part == 0 && j < l) {
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int64_t i = 32 * step + 8 * (L >> 4) + e;
      if (i < k) {
        const uint32_t b = rademacher(seed, t, k, l, i, j) > 0.f ? 0x3F80u : 0xBF80u;   // bf16(+1), bf16(-1)
        h[e >> 1] |= b << (16 * (e & 1));
      }
    }
  }
  reinterpret_cast<uint4*>(out + static_cast<int64_t>(blockIdx.y) * per * 8)[u] = make_uint4(h[0], h[1], h[2], h[3]);
}

__global__ void sketch_kernel(uint64_t seed, int t0, int64_t k, int l, int nt, int64_t rows, float* __restrict__ out) {
  const int64_t idx = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (idx >= rows * 16 * nt) return;
  const int t = t0 + static_cast<int>(blockIdx.y);   // one sketch per grid row
  out += static_cast<int64_t>(blockIdx.y) * rows * 16 * nt;
  const int64_t blk = idx / (256 * nt);
  const int e = static_cast<int>(idx - blk * 256 * nt);
  const int tile = e >> 8, f = e & 255;
  const int64_t i = blk * 16 + ((f >> 6) << 2) + (f & 3);
  const int j = tile * 16 + ((f >> 2) & 15);
  out[idx] = (i < k && j < l) ? rademacher(seed, t, k, l, i, j) : 0.f;
}

// Warm start of the subspace iteration (a variant the pages do not describe):
// columns j < r of a fragment-order sketch become sqrt(k) V[i][j], V = A^T
// diag(sigma)^-1/2 being the right singular vectors of the previous alternation
// (A = diag(sigma)^1/2 V^T); a column with sigma_j = 0 keeps its +-1 values.
__global__ void warm_columns_kernel(const float* __restrict__ A, const float* __restrict__ sigma, int64_t k, int r,
                                    int nt, float* __restrict__ out) {
  const int64_t idx = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (idx >= k * r) return;
  const int j = static_cast<int>(idx / k);
  const int64_t i = idx - static_cast<int64_t>(j) * k;
  const float sg = sigma[j];
  if (!(sg > 0.f)) return;
  out[frag_index(i, j, nt)] = sqrtf(static_cast<float>(k)) * (A[idx] / sqrtf(sg));
}

// Fragment-order fp32 panel (rows_pad rows, a multiple of 32) to its split copy
// (split_index): one thread per (32-row step, tile, lane) reads the lane's eight
// rows (two float4 of the fragment order) and writes the hi and lo pieces.
__global__ void split_panel_kernel(const float* __restrict__ frag, int64_t rows_pad, int nt,
                                   uint16_t* __restrict__ out) {
  const int64_t u = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (u >= (rows_pad >> 5) * nt * 64) return;
  const int L = static_cast<int>(u & 63);
  const int64_t st_tile = u >> 6;
  const int64_t st = st_tile / nt;
  const int tile = static_cast<int>(st_tile - st * nt);
  // rows 8 g .. 8 g + 7 of the step: quads 2 (g & 1) and 2 (g & 1) + 1 of fragment block 2 st + g / 2
  const int g = L >> 4, li = L & 15;
  const float4* f4 = reinterpret_cast<const float4*>(frag) + ((2 * st + (g >> 1)) * nt + tile) * 64 + li;
  const float4 a = f4[(2 * (g & 1)) * 16];
  const float4 b = f4[(2 * (g & 1) + 1) * 16];
  const float x[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
  uint4 hi, lo;
  split8_u4(x, hi, lo);
  uint4* o = reinterpret_cast<uint4*>(out) + (st_tile * 2) * 64 + L;
  o[0] = hi;
  o[64] = lo;
}

// Row-major n x l panel to fragment order over `rows` rows (zero padding).
__global__ void to_frag_kernel(const float* __restrict__ src, int64_t n, int l, int nt, int64_t rows,
                               float* __restrict__ out) {
  const int64_t idx = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (idx >= rows * 16 * nt) return;
  const int64_t blk = idx / (256 * nt);
  const int e = static_cast<int>(idx - blk * 256 * nt);
  const int tile = e >> 8, f = e & 255;
  const int64_t i = blk * 16 + ((f >> 6) << 2) + (f & 3);
  const int j = tile * 16 + ((f >> 2) & 15);
  out[idx] = (i < n && j < l) ? src[i * l + j] : 0.f;
}

// Round-robin (circle) schedule: position 0 is fixed, the others rotate.
__device__ __forceinline__ int rr_player(int pos, int rnd, int n) {
  return pos == 0 ? 0 : 1 + (pos - 1 + rnd) % (n - 1);
}

// Relative objective sqrt((|E|^2 - sum sigma^2) / |W|^2) from the two sums
// (and sqrt(|E|^2 / |W|^2) into out0); the caller's thread 0 only.
__device__ void objective_from_sums(const ObjectiveArgs& o, double es, double ws, double sig2) {
  const double num = es - sig2;
  *o.out = ws > 0.0 ? sqrt((num > 0.0 ? num : 0.0) / ws) : 0.0;
  if (o.out0 != nullptr) *o.out0 = ws > 0.0 ? sqrt(es / ws) : 0.0;
}

// All threads of the workgroup call this; thread 0 writes the objective.
__device__ void write_objective(const ObjectiveArgs& o, double sig2) {
  if (o.out == nullptr) return;
  const double es = block_sum_fixed(o.e_parts, o.ne);
  const double ws = block_sum_fixed(o.w_parts, o.nw);
  if (threadIdx.x == 0) objective_from_sums(o, es, ws, sig2);
}

// Sum of p[0 .. n) by one wave in a fixed order (lane-strided partial sums,
// four in flight, then a butterfly over the lanes); every lane gets the total.
__device__ double wave_sum_fixed(const double* __restrict__ p, int n) {
  const int lane = threadIdx.x & 63;
  double a0 = 0.0, a1 = 0.0, a2 = 0.0, a3 = 0.0;
  int i = lane;
  for (; i + 192 < n; i += 256) {
    a0 += p[i];
    a1 += p[i + 64];
    a2 += p[i + 128];
    a3 += p[i + 192];
  }
  for (; i < n; i += 64) a0 += p[i];
  double s = (a0 + a1) + (a2 + a3);
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) s += __shfl_xor(s, off);
  return s;
}

// Sum of P Gram partials (packed upper triangles, E = l(l+1)/2 doubles each)
// into one packed total.  Workgroup: 64 entries x 16 part groups; part group g
// sums partials g, g+16, ... (eight loads in flight), then the sixteen group
// sums are added in a fixed order.
__global__ __launch_bounds__(1024) void gram_sum_kernel(const double* __restrict__ parts, int P, int E,
                                                        double* __restrict__ total) {
  __shared__ double acc[16][64];
  const int el = threadIdx.x & 63, pg = threadIdx.x >> 6;
  const int e = blockIdx.x * 64 + el;
  double s = 0.0;
  if (e < E) {
    int p = pg;
    for (; p + 112 < P; p += 128) {
      double v[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) v[u] = parts[static_cast<int64_t>(p + 16 * u) * E + e];
#pragma unroll
      for (int u = 0; u < 8; ++u) s += v[u];
    }
    for (; p < P; p += 16) s += parts[static_cast<int64_t>(p) * E + e];
  }
  acc[pg][el] = s;
  __syncthreads();
  if (pg == 0 && e < E) {
    double t = 0.0;
#pragma unroll
    for (int g = 0; g < 16; ++g) t += acc[g][el];
    total[e] = t;
  }
}

template <int CTRL>
__device__ __forceinline__ float dpp_f32(float v) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), CTRL, 0xF, 0xF, true));
}
// fp32 sum over an aligned group of G = 16, 8 or 4 lanes; every lane of the
// group ends with the same total, bit for bit (each step pairs lanes
// symmetrically, so both lanes of a pair add the same two operands).
template <int G>
__device__ __forceinline__ float group_sumf(float v) {
  static_assert(G == 16 || G == 8 || G == 4, "16-, 8- or 4-lane groups");
  v += dpp_f32<0xB1>(v);                   // quad_perm xor 1
  v += dpp_f32<0x4E>(v);                   // quad_perm xor 2
  if (G >= 8) v += dpp_f32<0x141>(v);      // row_half_mirror: the other quad of the 8
  if (G == 16) v += dpp_f32<0x140>(v);     // row_mirror: the other 8 of the row
  return v;
}

// ---------------------------------------------------------------------------
// The same two solves for l <= 32, on the register Cholesky of chol_wave.
//
// mode 1 for l <= LM: X = R^-1 (fp32, row-major l x l) by one wave.
template <int LM>
__global__ __launch_bounds__(64) void chol_inv_wave_kernel(const double* __restrict__ gram, int l,
                                                           float* __restrict__ Xinv) {
  __shared__ double rowbuf[64];
  double g[LM], t[LM];
  chol_wave<LM, true>(gram, l, g, t, rowbuf);
  const int lane = threadIdx.x;
  if (lane < l) {
#pragma unroll
    for (int a = 0; a < LM; ++a)
      if (a < l) Xinv[lane * l + a] = static_cast<float>(t[a]);
  }
}

// ---------------------------------------------------------------------------
// The core solve.  Q is orthonormal (fp64 Gram and Cholesky; its fp32 rounding
// leaves Q^T Q = I to ~1e-7), so Q^T E = C^T and its singular values are those
// of R, the Cholesky factor of H = C^T C = R^T R.  With R = U_R diag(sigma) V_R^T,
// one-sided Jacobi on the columns of K = R^T (scaled by a power of two, exact)
// converges to K J = V_R diag(sigma) 2^-e: V_R is K's normalised columns, so no
// rotation needs accumulating.  B = Q V_R diag(sigma)^1/2 and
// A = diag(sigma)^1/2 (C R^-1 U_R)^T = (C V_R diag(sigma)^-1/2)^T.

// One-sided Jacobi rotation of a pair held by a 16-lane group (rows sub + 16 i
// of x_p and x_q in xp, xq).  With alpha, beta the squared norms and gamma the
// dot product (already summed over the group), the rotation by theta,
// tan 2 theta = 2 gamma / (beta - alpha), |theta| <= pi / 4, is taken in the
// branch-free form cos 2 theta = |beta - alpha| / h, h = hypot(beta - alpha,
// 2 gamma), c = sqrt((1 + cos 2 theta) / 2), s = sin 2 theta / (2 c).  A pair
// is left alone while gamma^2 <= 1e-14 alpha beta.  alpha and beta are carried
// through the rotation, alpha' = c^2 alpha - 2 c s gamma + s^2 beta and
// beta' = s^2 alpha + 2 c s gamma + c^2 beta.  Returns whether the pair was
// still coupled above the stopping threshold, gamma^2 > 1e-8 alpha beta
// (|cos| > 1e-4): the sweeps stop after one without such a pair.  Convergence
// is quadratic once the couplings are below the relative gaps of the singular
// values; with the nearly flat spectra of quantization residuals (neighbouring
// values ~1% apart) a 1e-3 cut left couplings near 1e-5, visible in the
// orthogonality of A, while 1e-4 leaves them at the fp32 rounding level.
template <int RL>
__device__ __forceinline__ bool jacobi_rotate(float (&xp)[RL], float (&xq)[RL], float& al, float& be, float ga) {
  const float g2 = ga * ga, ab = al * be;
  const bool doit = g2 > 1e-14f * ab;
  const float dd = be - al;
  const float ri = __builtin_amdgcn_rsqf(fmaf(dd, dd, 4.f * g2));
  const float hc = fmaf(0.5f * fabsf(dd), ri, 0.5f);
  const float rh = __builtin_amdgcn_rsqf(hc);
  const float c = doit ? hc * rh : 1.f;
  const float sn = doit ? (dd >= 0.f ? ga : -ga) * ri * rh : 0.f;
#pragma unroll
  for (int i = 0; i < RL; ++i) {
    const float u = xp[i], w = xq[i];
    xp[i] = fmaf(c, u, -(sn * w));
    xq[i] = fmaf(sn, u, c * w);
  }
  const float cc = c * c, ss = sn * sn, cs2 = 2.f * c * sn * ga;
  const float a2 = fmaxf(fmaf(cc, al, fmaf(ss, be, -cs2)), 0.f);
  be = fmaxf(fmaf(ss, al, fmaf(cc, be, cs2)), 0.f);
  al = a2;
  return g2 > 1e-8f * ab;
}

// A value of the lane in the same position of the wave's other 16-lane row of its
// pair (row XOR 1) or half (row XOR 2): v_permlane16_swap / v_permlane32_swap with
// the value as both operands return the even and the odd row's (half's) copy.
__device__ __forceinline__ float rows_xor1(float v) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(((threadIdx.x >> 4) & 1) ? r[0] : r[1]);
}
__device__ __forceinline__ float rows_xor2(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(((threadIdx.x >> 5) & 1) ? r[0] : r[1]);
}

// One-sided Jacobi sweeps on the columns of K (fp32, LDS, column stride
// ld > GL RL with GL = 64 / BW lanes per column; rows GL RL and beyond the
// matrix are zero), a column pair per GL-lane group (lane sub holds rows
// sub + GL i, i < RL), in a block order that needs a workgroup barrier only
// between block rounds.  The columns (n rounded up to nbk blocks of BW, nbk
// even; columns beyond n are zero) form a round-robin of blocks: in block round
// rho wave w holds blocks rr_player(w, rho, nbk) and rr_player(nbk - 1 - w, rho,
// nbk); its lane group g keeps column g of the first block in registers and in
// sub-round j (j < BW) rotates it against column (g + j) mod BW of the second,
// which passes from group to group through LDS within the wave (BW = 4: column
// g ^ j, passed on by lane-row swaps, the groups being the wave's 16-lane rows).  Block round 0
// first runs the pairs inside each of the wave's two blocks (round-robin of BW,
// BW - 1 sub-rounds; its first sub-round meets every column and forms all three
// dot products, later sub-rounds form gamma only).  A sweep is BW - 1 + BW (nbk - 1)
// sub-rounds and meets every pair once.  Row GL RL of each column carries its
// squared norm.  All threads call it (at least nbk / 2 waves); returns the sweeps.
template <int RL, int BW>
__device__ int jacobi_blocks(float* K, int ld, int n, int max_sweeps) {
  static_assert(BW == 4 || BW == 8, "4- or 8-column blocks");
  constexpr int GL = 64 / BW;   // lanes per column pair
  const int wave = threadIdx.x >> 6, g = (threadIdx.x / GL) % BW, sub = threadIdx.x % GL;
  const int nbk0 = (n + BW - 1) / BW, nbk = nbk0 + (nbk0 & 1);
  const bool active = wave < nbk / 2;
  float* Ks = K + sub;
  int sweeps = 0;
  for (int sweep = 0; sweep < max_sweeps; ++sweep) {
    uint64_t big = 0;
    for (int rnd = 0; rnd < nbk - 1; ++rnd) {
      if (active) {
        const int ba = rr_player(wave, rnd, nbk), bb = rr_player(nbk - 1 - wave, rnd, nbk);
        float xa[RL], xb[RL];
        if (rnd == 0) {
          const int blk = g < BW / 2 ? ba : bb, slot = g % (BW / 2);
#pragma unroll
          for (int ir = 0; ir < BW - 1; ++ir) {
            const int x = rr_player(slot, ir, BW), y = rr_player(BW - 1 - slot, ir, BW);
            float* cp = Ks + (blk * BW + min(x, y)) * ld;
            float* cq = Ks + (blk * BW + max(x, y)) * ld;
            float al = cp[GL * RL - sub], be = cq[GL * RL - sub], ga = 0.f;
#pragma unroll
            for (int i = 0; i < RL; ++i) {
              xa[i] = cp[GL * i];
              xb[i] = cq[GL * i];
            }
#pragma unroll
            for (int i = 0; i < RL; ++i) ga = fmaf(xa[i], xb[i], ga);
            ga = group_sumf<GL>(ga);
            if (ir == 0) {
              float a2 = 0.f, b2 = 0.f;
#pragma unroll
              for (int i = 0; i < RL; ++i) {
                a2 = fmaf(xa[i], xa[i], a2);
                b2 = fmaf(xb[i], xb[i], b2);
              }
              al = group_sumf<GL>(a2);
              be = group_sumf<GL>(b2);
            }
            big |= __builtin_amdgcn_ballot_w64(jacobi_rotate<RL>(xa, xb, al, be, ga));
#pragma unroll
            for (int i = 0; i < RL; ++i) {
              cp[GL * i] = xa[i];
              cq[GL * i] = xb[i];
            }
            cp[GL * RL - sub] = al;
            cq[GL * RL - sub] = be;
            __builtin_amdgcn_wave_barrier();
          }
        }
        float* ca = Ks + (ba * BW + g) * ld;
        float al = ca[GL * RL - sub];
#pragma unroll
        for (int i = 0; i < RL; ++i) xa[i] = ca[GL * i];
        const bool a_low = ba < bb;
        if constexpr (BW == 4) {
          // the lane groups are the wave's four 16-lane rows: in sub-round j group g
          // meets column g ^ j of the second block, which the rows pass on between
          // sub-rounds with lane-row swaps (XOR 1, 3, 1) instead of through LDS
          float* cb = Ks + (bb * BW + g) * ld;
          float be = cb[GL * RL - sub];
#pragma unroll
          for (int i = 0; i < RL; ++i) xb[i] = cb[GL * i];
#pragma unroll
          for (int j = 0; j < BW; ++j) {
            if (j > 0) {
#pragma unroll
              for (int i = 0; i < RL; ++i) xb[i] = j == 2 ? rows_xor2(rows_xor1(xb[i])) : rows_xor1(xb[i]);
              be = j == 2 ? rows_xor2(rows_xor1(be)) : rows_xor1(be);
            }
            float ga = 0.f;
#pragma unroll
            for (int i = 0; i < RL; ++i) ga = fmaf(xa[i], xb[i], ga);
            ga = group_sumf<GL>(ga);
            const bool coupled = a_low ? jacobi_rotate<RL>(xa, xb, al, be, ga) : jacobi_rotate<RL>(xb, xa, be, al, ga);
            big |= __builtin_amdgcn_ballot_w64(coupled);
          }
          // after the last sub-round group g holds column g ^ 3
          float* ce = Ks + (bb * BW + (g ^ 3)) * ld;
#pragma unroll
          for (int i = 0; i < RL; ++i) ce[GL * i] = xb[i];
          ce[GL * RL - sub] = be;
        } else {
#pragma unroll
          for (int j = 0; j < BW; ++j) {
            float* cb = Ks + (bb * BW + (g + j) % BW) * ld;
            float be = cb[GL * RL - sub], ga = 0.f;
#pragma unroll
            for (int i = 0; i < RL; ++i) xb[i] = cb[GL * i];
#pragma unroll
            for (int i = 0; i < RL; ++i) ga = fmaf(xa[i], xb[i], ga);
            ga = group_sumf<GL>(ga);
            const bool coupled = a_low ? jacobi_rotate<RL>(xa, xb, al, be, ga) : jacobi_rotate<RL>(xb, xa, be, al, ga);
            big |= __builtin_amdgcn_ballot_w64(coupled);
#pragma unroll
            for (int i = 0; i < RL; ++i) cb[GL * i] = xb[i];
            cb[GL * RL - sub] = be;
            __builtin_amdgcn_wave_barrier();
          }
        }
#pragma unroll
        for (int i = 0; i < RL; ++i) ca[GL * i] = xa[i];
        ca[GL * RL - sub] = al;
      }
      __syncthreads();
    }
    sweeps = sweep + 1;
    if (!__syncthreads_or(big != 0)) break;
  }
  return sweeps;
}

// Outputs of the core from the swept K (column a: 2^-e sigma_a V_R[:, a], column
// stride ld, n rows): columns ranked by sigma (ties by index); for rank c < r,
// column a, S_B[row][c] = (X V_R)[row][a] sigma_a^1/2 and S_A[row][c] =
// V_R[row][a] sigma_a^-1/2 (X = R_Y^-1, l x l row-major upper triangular, so
// that B = Y S_B), sigma, the stats (sum of the r sigma^2, sweeps) and the
// objective.  All threads call it.
__device__ void core_finish(const float* K, int ld, int l, int n, double ksc, const float* X, int r, float* SB,
                            float* SA, float* sigma, double* stats, const ObjectiveArgs& obj, int sweeps,
                            double* norm2, int* order, const double* objsums = nullptr) {
  const int tid = threadIdx.x, nt = blockDim.x;
  for (int a = tid; a < l; a += nt) {
    double s = 0.0;
    for (int row = 0; row < n; ++row) s += static_cast<double>(K[a * ld + row]) * static_cast<double>(K[a * ld + row]);
    norm2[a] = s / (ksc * ksc);
  }
  __syncthreads();
  for (int a = tid; a < l; a += nt) {
    const double la = norm2[a];
    int rank = 0;
    for (int b = 0; b < l; ++b) rank += (norm2[b] > la || (norm2[b] == la && b < a)) ? 1 : 0;
    order[rank] = a;
  }
  __syncthreads();
  for (int idx = tid; idx < l * r; idx += nt) {
    const int row = idx / r, c = idx - row * r;
    const int a = order[c];
    const double sg = sqrt(norm2[a]);
    const double sq = sqrt(sg);
    const double kn = sg * ksc;   // |K_a|
    double acc = 0.0;
    for (int j = row; j < l; ++j) acc = fma(static_cast<double>(X[row * l + j]), static_cast<double>(K[a * ld + j]), acc);
    SB[row * r + c] = kn > 0.0 ? static_cast<float>(acc * sq / kn) : 0.f;
    SA[row * r + c] = kn > 0.0 ? static_cast<float>(static_cast<double>(K[a * ld + row]) / (kn * sq)) : 0.f;
  }
  for (int c = tid; c < r; c += nt) sigma[c] = static_cast<float>(sqrt(norm2[order[c]]));
  double s2 = 0.0;
  for (int c = 0; c < r; ++c) s2 += norm2[order[c]];
  if (tid == 0 && stats) {
    stats[0] = s2;
    stats[1] = static_cast<double>(sweeps);
  }
  if (objsums == nullptr) write_objective(obj, s2);
  else if (tid == 0 && obj.out != nullptr) objective_from_sums(obj, objsums[0], objsums[1], s2);
}

// mode 2 for l <= LM (LM <= 32), 16 lanes per pair, by 256 threads: the four
// waves sum the P Gram partials of C (gram_sum_block, 16 partials in flight per
// wave), wave 0 factors H in fp64 and writes K = 2^-e R^T while wave 1 sums the
// |E|^2 and |W|^2 partials of the objective; the sweeps use the first
// ceil(l / 8) waves.
template <int LM>
__global__ __launch_bounds__(256) void core_small_kernel(const double* __restrict__ gparts, int P, int l,
                                                         const float* __restrict__ Xinv, int r, float* __restrict__ SB,
                                                         float* __restrict__ SA, float* __restrict__ sigma,
                                                         double* __restrict__ stats, ObjectiveArgs obj) {
  constexpr int LD = 33;
  __shared__ double gsum[5 * (LM * (LM + 1) / 2)];   // (waves + 1) E_ doubles, at most 4 waves
  __shared__ double rowbuf[64];
  __shared__ float K[32 * LD];
  __shared__ float Xs[32 * 32];
  __shared__ double norm2[32];
  __shared__ int order[32];
  __shared__ double kscale;
  __shared__ double objsums[2];
  const int tid = threadIdx.x;
  const int n = l + (l & 1);
  for (int e = tid; e < l * l; e += blockDim.x) Xs[e] = Xinv[e];
  const double* gram = gram_sum_block<LM, 16>(gparts, P, l, gsum);
  const int sum_wave = blockDim.x > 64 ? 1 : 0;
  if (obj.out != nullptr && sum_wave == 1 && (tid >> 6) == 1) {
    const double es = wave_sum_fixed(obj.e_parts, obj.ne), ws = wave_sum_fixed(obj.w_parts, obj.nw);
    if (tid == 64) {
      objsums[0] = es;
      objsums[1] = ws;
    }
  }
  if (tid < 64) {
    double g[LM], t[LM];
    chol_wave<LM, false>(gram, l, g, t, rowbuf);
    // 2^-e with 2^e at the scale of R's largest entry, so the fp32 sweeps
    // neither overflow nor underflow whatever the magnitude of E
    double m = 0.0;
#pragma unroll
    for (int a = 0; a < LM; ++a) m = fmax(m, (a <= tid && tid < l) ? fabs(g[a]) : 0.0);
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) m = fmax(m, __shfl_xor(m, off));
    const double sc = m > 0.0 ? ldexp(1.0, -ilogb(m)) : 1.0;
    if (tid == 0) kscale = sc;
    // lane b holds column b of R: K[a][b] = R[a][b] (column a of K = row a of R)
    if (tid < LD) {
#pragma unroll
      for (int a = 0; a < 32; ++a)
        K[a * LD + tid] = (a < LM && a <= tid && tid < l) ? static_cast<float>(g[a < LM ? a : 0] * sc) : 0.f;
    }
    if (obj.out != nullptr && sum_wave == 0) {
      const double es = wave_sum_fixed(obj.e_parts, obj.ne), ws = wave_sum_fixed(obj.w_parts, obj.nw);
      if (tid == 0) {
        objsums[0] = es;
        objsums[1] = ws;
      }
    }
  }
  __syncthreads();
  const int sweeps = jacobi_blocks<2, 4>(K, LD, n, 30);
  core_finish(K, LD, l, n, kscale, Xs, r, SB, SA, sigma, stats, obj, sweeps, norm2, order, objsums);
}

// ---------------------------------------------------------------------------
// The two solves for 32 < l <= kMaxL, by one workgroup of 640 threads.
//
// chol_blocked: right-looking Cholesky H = R^T R of the fp64 Gram in 16 x 16
// blocks, the matrix in LDS (A, stride kWideLd, zero beyond l).  Block step p:
// wave 0 factors the diagonal block with the register recurrence of chol_wave
// (lanes 0..15, lane b holding column b), giving R_pp and T_pp = R_pp^-T; the
// waves then form the block row R[p, q] = T_pp A[p, q] (q > p) and subtract
// R[p, q]^T R[p, s] from the trailing blocks (p < q <= s), one 16 x 16 block
// per wave at a time, each lane four entries (rows ra + 4 i, column cb).  A
// pivot at or below 1e-13 of the largest diagonal entry of H drops its
// direction (zero row of R, zero row of T_pp).  Three barriers per block step
// instead of one per row.
constexpr int kWideLd = kMaxL + 1;
constexpr int kCB = 16;                          // block of the blocked Cholesky
constexpr int kCNB = (kMaxL + kCB - 1) / kCB;    // block rows at most
// measured on MI355X at l = 80: more lanes per pair and more waves win (4-lane
// pairs on 3 waves: 2.5x slower core)
constexpr int kWideCholWaves = 10;   // waves of the l > 32 Cholesky workgroup
constexpr int kWideGroup = 8;        // lanes per Jacobi pair of the l > 32 core (8: blocks of 8 columns)

// Diagonal block (LDS, stride ld) by one wave: lane (ra, cb) = (lane / 16,
// lane % 16) keeps entries (ra + 4 i, cb), i < 4, of the block and of T (the
// identity at first).  Step j: the lanes holding row j scale it by 1 / R[j][j]
// (R's row j, T's row j) and publish both rows through LDS (rowbuf: 2 x 16
// doubles); rows a > j then lose R[j][a] times them.  Writes R_pp over the
// block's upper triangle and T_pp (row-major 16 x 16) to T.
__device__ __forceinline__ void chol_diag16(double* D, int ld, double tol, double* T, double* rowbuf) {
  const int lane = threadIdx.x & 63, ra = lane >> 4, cb = lane & 15;
  double g[4], t[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int a = ra + 4 * i;
    const double v = D[a * ld + cb];
    g[i] = a <= cb ? v : 0.0;
    t[i] = a == cb ? 1.0 : 0.0;
  }
#pragma unroll
  for (int j = 0; j < kCB; ++j) {
    const int jr = j & 3, ji = j >> 2;
    const double piv = bcast_lane(g[ji], jr * 16 + j);
    const bool keep = piv > tol && piv > 0.0;
    const double inv = keep ? rsq_f64(piv) : 0.0;   // 1 / R[j][j]
    const double rjj = piv * inv;
    if (ra == jr) {
      const double v = g[ji];
      g[ji] = cb > j ? v * inv : (cb == j ? rjj : v);
      t[ji] *= inv;
      rowbuf[cb] = g[ji];
      rowbuf[kCB + cb] = t[ji];
    }
    __builtin_amdgcn_wave_barrier();
    const double rjb = rowbuf[cb], tjb = rowbuf[kCB + cb];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int a = ra + 4 * i;
      const double rja = rowbuf[a];
      const bool upd = a > j;
      g[i] = upd ? fma(-rja, rjb, g[i]) : g[i];
      t[i] = upd ? fma(-rja, tjb, t[i]) : t[i];
    }
    __builtin_amdgcn_wave_barrier();
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int a = ra + 4 * i;
    if (a <= cb) D[a * ld + cb] = g[i];
    T[a * kCB + cb] = t[i];
  }
}

// All threads call it.  Td: kCNB blocks of 16 x 16 doubles (the T_pp).
__device__ __forceinline__ void chol_blocked(const double* __restrict__ gram, int l, double* A, double* Td, double* rowbuf,
                             double* scratch) {
  const int tid = threadIdx.x, nt = blockDim.x, w = tid >> 6, lane = tid & 63, nw = nt >> 6;
  const int nb = (l + kCB - 1) / kCB, lp = nb * kCB;
  for (int e = tid; e < lp * lp; e += nt) {
    const int a = e / lp, b = e - a * lp;
    const bool in = a <= b && b < l;
    A[a * kWideLd + b] = in ? gram[packed_index(a, b, l)] : 0.0;
  }
  if (tid < 64) {
    double m = 0.0;
    for (int a = tid; a < l; a += 64) m = fmax(m, gram[packed_index(a, a, l)]);
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) m = fmax(m, __shfl_xor(m, off));
    if (tid == 0) scratch[0] = m;
  }
  __syncthreads();
  const double tol = 1e-13 * scratch[0];
  const int ra = lane >> 4, cb = lane & 15;
  for (int p = 0; p < nb; ++p) {
    const int p0 = p * kCB;
    if (w == 0) chol_diag16(A + p0 * kWideLd + p0, kWideLd, tol, Td + p * kCB * kCB, rowbuf);
    __syncthreads();
    const double* T = Td + p * kCB * kCB;
    for (int q = p + 1 + w; q < nb; q += nw) {   // R[p, q] = T_pp A[p, q]
      double* Apq = A + p0 * kWideLd + q * kCB;
      double acc[4] = {0.0, 0.0, 0.0, 0.0};
#pragma unroll 2
      for (int c = 0; c < kCB; ++c) {
        const double x = Apq[c * kWideLd + cb];
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[i] = fma(T[(ra + 4 * i) * kCB + c], x, acc[i]);
      }
      __builtin_amdgcn_wave_barrier();   // the wave's reads of the block precede its writes
#pragma unroll
      for (int i = 0; i < 4; ++i) Apq[(ra + 4 * i) * kWideLd + cb] = acc[i];
    }
    __syncthreads();
    const int m = nb - p - 1, nblk = m * (m + 1) / 2;
    for (int bi = w; bi < nblk; bi += nw) {   // A[q, s] -= R[p, q]^T R[p, s]
      int q = 0, rem = bi;
      while (rem >= m - q) {
        rem -= m - q;
        ++q;
      }
      const int Q = p + 1 + q, S = Q + rem;
      const double* Rq = A + p0 * kWideLd + Q * kCB;
      const double* Rs = A + p0 * kWideLd + S * kCB;
      double* Aqs = A + Q * kCB * kWideLd + S * kCB;
      double acc[4] = {0.0, 0.0, 0.0, 0.0};
#pragma unroll 2
      for (int c = 0; c < kCB; ++c) {
        const double y = Rs[c * kWideLd + cb];
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[i] = fma(Rq[c * kWideLd + ra + 4 * i], y, acc[i]);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) Aqs[(ra + 4 * i) * kWideLd + cb] -= acc[i];
    }
    __syncthreads();
  }
}

// X = R^-1 = T^T from the factored A (upper blocks R) and Td: T = R^-T by block
// forward substitution, T[p, p] = T_pp and, for block rows q in order,
// T[q, p] = -T_qq sum_{s=p}^{q-1} R[s, q]^T T[s, p] (p < q; one block per wave,
// the partial sum parked in the block's own place in Tm).  Writes X (l x l fp32,
// row-major upper triangular, zero below).
__device__ __forceinline__ void chol_inverse(const double* A, const double* Td, int l, double* Tm, float* __restrict__ X) {
  const int tid = threadIdx.x, nt = blockDim.x, w = tid >> 6, lane = tid & 63, nw = nt >> 6;
  const int nb = (l + kCB - 1) / kCB;
  const int ra = lane >> 4, cb = lane & 15;
  for (int e = tid; e < nb * kCB * kCB; e += nt) {
    const int p = e / (kCB * kCB), a = (e / kCB) % kCB, b = e % kCB;
    Tm[(p * kCB + a) * kWideLd + p * kCB + b] = Td[e];
  }
  __syncthreads();
  for (int q = 1; q < nb; ++q) {
    const double* Tq = Td + q * kCB * kCB;
    for (int p = w; p < q; p += nw) {
      double acc[4] = {0.0, 0.0, 0.0, 0.0};
      for (int s = p; s < q; ++s) {
        const double* Rsq = A + s * kCB * kWideLd + q * kCB;
        const double* Tsp = Tm + s * kCB * kWideLd + p * kCB;
#pragma unroll 2
        for (int c = 0; c < kCB; ++c) {
          const double y = Tsp[c * kWideLd + cb];
#pragma unroll
          for (int i = 0; i < 4; ++i) acc[i] = fma(Rsq[c * kWideLd + ra + 4 * i], y, acc[i]);
        }
      }
      double* Tqp = Tm + q * kCB * kWideLd + p * kCB;
#pragma unroll
      for (int i = 0; i < 4; ++i) Tqp[(ra + 4 * i) * kWideLd + cb] = acc[i];
      __builtin_amdgcn_wave_barrier();
      double out[4] = {0.0, 0.0, 0.0, 0.0};
#pragma unroll 2
      for (int c = 0; c < kCB; ++c) {
        const double y = Tqp[c * kWideLd + cb];
#pragma unroll
        for (int i = 0; i < 4; ++i) out[i] = fma(Tq[(ra + 4 * i) * kCB + c], y, out[i]);
      }
      __builtin_amdgcn_wave_barrier();
#pragma unroll
      for (int i = 0; i < 4; ++i) Tqp[(ra + 4 * i) * kWideLd + cb] = -out[i];
    }
    __syncthreads();
  }
  for (int e = tid; e < l * l; e += nt) {
    const int a = e / l, b = e - a * l;
    X[e] = a <= b ? static_cast<float>(Tm[b * kWideLd + a]) : 0.f;
  }
}

// MODE 1: Cholesky and X = R^-1 on NW waves; MODE 2: the core on 10 waves, the
// Jacobi pairs on GW-lane groups (jacobi_blocks with blocks of 64 / GW columns).
template <int MODE, int NW, int GW>
__global__ __launch_bounds__(64 * NW) void solve_wide_kernel(const double* __restrict__ gram, int l,
                                                                  float* __restrict__ Xinv, int r,
                                                                  float* __restrict__ SB, float* __restrict__ SA,
                                                                  float* __restrict__ sigma, double* __restrict__ stats,
                                                                  ObjectiveArgs obj) {
  constexpr int NB = kMaxL * kWideLd;
  static_assert(MODE == 1 || ((GW == 16 || GW == 8) && NW == 10), "the wide core: 10 waves, 16- or 8-lane pairs");
  __shared__ double Rm[NB];
  __shared__ double Tm[MODE == 1 ? NB : 1];
  __shared__ double Td[kCNB * kCB * kCB];
  __shared__ float Kf[MODE == 2 ? NB : 1];
  __shared__ double rowbuf[2 * kCB];
  __shared__ double norm2[kMaxL];
  __shared__ int order[kMaxL];
  __shared__ double scratch[2];
  const int tid = threadIdx.x, nt = blockDim.x;
  chol_blocked(gram, l, Rm, Td, rowbuf, scratch);
  if (MODE == 1) {
    chol_inverse(Rm, Td, l, Tm, Xinv);
    return;
  }
  const int n = l + (l & 1);
  // K = 2^-e R^T (column c of K = row c of R), fp32, with 2^e at the scale of R's largest entry
  if (tid < 64) {
    double m = 0.0;
    for (int a = tid; a < l; a += 64) m = fmax(m, fabs(Rm[a * kWideLd + a]));
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) m = fmax(m, __shfl_xor(m, off));
    if (tid == 0) scratch[1] = m > 0.0 ? ldexp(1.0, -ilogb(m)) : 1.0;
  }
  __syncthreads();
  const double ksc = scratch[1];
  for (int e = tid; e < NB; e += nt) {
    const int c = e / kWideLd, j = e - c * kWideLd;
    Kf[e] = (c < l && j >= c && j < l) ? static_cast<float>(Rm[c * kWideLd + j] * ksc) : 0.f;
  }
  __syncthreads();
  constexpr int RL = (kMaxL + GW - 1) / GW;
  const int sweeps = jacobi_blocks<RL, 64 / GW>(Kf, kWideLd, n, 40);
  core_finish(Kf, kWideLd, l, n, ksc, Xinv, r, SB, SA, sigma, stats, obj, sweeps, norm2, order);
}

// Sum of the split-K partials, sum_s part[s], in fixed order for a tile of
// kGramRows rows, optionally right-multiplied by X (l x l fp32, upper
// triangular; entries below the diagonal are ignored), written in fragment
// order (zero-padded to m_pad rows), plus the fp64 Gram partial (packed upper
// triangle) of the tile when gram_parts is given.  The two small contractions
// run on the matrix cores, one 16 x 16 output tile per wave at a time: the X
// product with fp32 MFMA (16x16x4), the Gram with fp64 MFMA (16x16x4) over the
// tile's rows; each accumulates its K steps in ascending order, so results are
// deterministic.
typedef float mfma_f4 __attribute__((ext_vector_type(4)));
typedef double mfma_d4 __attribute__((ext_vector_type(4)));

template <int NT>
__global__ __launch_bounds__(kReduceThreads) void reduce_gram_kernel(const float* __restrict__ part, int S, int64_t m,
                                                          int64_t m_pad, int l, const float* __restrict__ X,
                                                          float* __restrict__ out, uint16_t* __restrict__ out_split,
                                                          double* __restrict__ gram_parts, int paired) {
  constexpr int LP = 16 * NT, PER = (kGramRows * LP + kReduceThreads - 1) / kReduceThreads, LDR = LP + 1;
  constexpr int NW = kReduceThreads / 64;
  static_assert(kGramRows % 64 == 0, "whole pairs of 32-row steps of the split copy (and 16-row MFMA tiles)");
  // wide panels (NT >= 3) keep fewer loads in flight, so the per-thread state
  // fits the register file of a 512-thread workgroup
  constexpr int QB = NT <= 2 ? 8 : 2;
  __shared__ float rows[kGramRows * LDR];
  __shared__ float rowsx[kGramRows * LDR];
  __shared__ float Xs[LP * LP];
  const int64_t r0 = static_cast<int64_t>(blockIdx.x) * kGramRows;
  const int64_t stride = m * LP;
  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63, li = lane & 15, lk = lane >> 4;
  if (X) {
    for (int e = threadIdx.x; e < LP * LP; e += blockDim.x) {
      const int a = e / LP, b = e - a * LP;
      Xs[e] = (a <= b && b < l) ? X[a * l + b] : 0.f;
    }
  }
  // every thread sums its PER elements over the S partials, QB partials of all
  // its elements in flight at a time, each element in ascending s order
  float acc[PER];
  int off[PER];   // row offset within the tile times LP plus column; -1: nothing to load
#pragma unroll
  for (int u = 0; u < PER; ++u) {
    const int idx = threadIdx.x + kReduceThreads * u;
    const int rr = idx / LP, n = idx - rr * LP;
    const bool ok = idx < kGramRows * LP && r0 + rr < m && n < l;
    off[u] = ok ? idx : -1;
    acc[u] = 0.f;
  }
  const float* base = part + r0 * LP;
  int p = 0;
  for (; p + QB <= S; p += QB) {
    float v[QB][PER];
#pragma unroll
    for (int q = 0; q < QB; ++q)
#pragma unroll
      for (int u = 0; u < PER; ++u) v[q][u] = off[u] >= 0 ? base[(p + q) * stride + off[u]] : 0.f;
#pragma unroll
    for (int q = 0; q < QB; ++q)
#pragma unroll
      for (int u = 0; u < PER; ++u) acc[u] += v[q][u];
  }
  for (; p < S; ++p)
#pragma unroll
    for (int u = 0; u < PER; ++u) acc[u] += off[u] >= 0 ? base[p * stride + off[u]] : 0.f;
#pragma unroll
  for (int u = 0; u < PER; ++u) {
    const int idx = threadIdx.x + kReduceThreads * u;
    if (idx < kGramRows * LP) rows[(idx / LP) * LDR + idx % LP] = acc[u];
  }
  __syncthreads();
  const float* R = rows;
  if (X) {
    // tile (rt, ct) of rows x X: lane (li, lk) supplies A[li][lk] = rows[16 rt + li][4 ks + lk] and
    // B[lk][li] = X[4 ks + lk][16 ct + li]; D[4 lk + v][li] comes back in element v
    for (int t = w; t < (kGramRows / 16) * NT; t += NW) {
      const int rt = t / NT, ct = t - rt * NT;
      mfma_f4 dacc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < LP / 4; ++ks)
        dacc = __builtin_amdgcn_mfma_f32_16x16x4f32(rows[(16 * rt + li) * LDR + 4 * ks + lk],
                                                    Xs[(4 * ks + lk) * LP + 16 * ct + li], dacc, 0, 0, 0);
#pragma unroll
      for (int v = 0; v < 4; ++v) rowsx[(16 * rt + 4 * lk + v) * LDR + 16 * ct + li] = dacc[v];
    }
    __syncthreads();
    R = rowsx;
  }
  // fragment-order output: a thread writes rows 4 q .. 4 q + 3 of one column as one float4
  for (int qd = threadIdx.x; qd < (kGramRows / 4) * LP; qd += blockDim.x) {
    const int n = qd % LP, q = qd / LP;
    const int64_t row = r0 + 4 * q;
    if (row < m_pad)
      *reinterpret_cast<float4*>(out + frag_index(row, n, NT)) =
          make_float4(R[(4 * q) * LDR + n], R[(4 * q + 1) * LDR + n], R[(4 * q + 2) * LDR + n],
                      R[(4 * q + 3) * LDR + n]);
  }
  // the split copy for the bf16 products: per 32-row step, tile and lane, the lane's
  // eight rows of its column as hi and lo pieces
  if (out_split != nullptr) {
    uint4* os = reinterpret_cast<uint4*>(out_split);
    for (int ui = threadIdx.x; ui < (kGramRows / 32) * NT * 64; ui += blockDim.x) {
      const int L = ui & 63, tn = (ui >> 6) % NT, st = (ui >> 6) / NT;
      const int64_t rs = r0 + 32 * st;
      if (rs >= m_pad) continue;
      const int gg = L >> 4, n = 16 * tn + (L & 15);
      float x[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) x[e] = R[split_row(st, gg, e, paired != 0) * LDR + n];
      uint4 hi, lo;
      split8_u4(x, hi, lo);
      const int64_t b = (((rs >> 5) * NT + tn) * 2) * 64 + L;
      os[b] = hi;
      os[b + 64] = lo;
    }
  }
  if (gram_parts == nullptr || r0 >= m) return;
  // Gram partial, tiles (ta, tb), ta <= tb: A[li][lk] = R[4 ks + lk][16 ta + li],
  // B[lk][li] = R[4 ks + lk][16 tb + li]; the fp64 MFMA returns D[lk + 4 v][li] in
  // element v.  Rows beyond m and columns beyond l are zero in R.
  double* gp = gram_parts + static_cast<int64_t>(blockIdx.x) * (l * (l + 1) / 2);
  for (int t = w; t < NT * (NT + 1) / 2; t += NW) {
    int ta = 0, rem = t;
    while (rem >= NT - ta) {
      rem -= NT - ta;
      ++ta;
    }
    const int tb = ta + rem;
    mfma_d4 dacc = {0.0, 0.0, 0.0, 0.0};
#pragma unroll
    for (int ks = 0; ks < kGramRows / 4; ++ks)
      dacc = __builtin_amdgcn_mfma_f64_16x16x4f64(static_cast<double>(R[(4 * ks + lk) * LDR + 16 * ta + li]),
                                                  static_cast<double>(R[(4 * ks + lk) * LDR + 16 * tb + li]), dacc,
                                                  0, 0, 0);
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int a = 16 * ta + lk + 4 * v, b = 16 * tb + li;
      if (a <= b && b < l) gp[packed_index(a, b, l)] = dacc[v];
    }
  }
}

// ---------------------------------------------------------------------------
// Panel times small matrix: out = P S (m x w) or its transpose (w x m), with P
// an m x l panel in fragment order (nt tiles) and S l x w.  64 rows of P and all
// of S are staged in LDS.  One launch serves both factor products: workgroups
// [0, nb0) take job 0 (B = Q S_B) and the rest job 1 (A = (C S_A)^T).
struct PanelJob {
  const float* P;
  int64_t m;
  const float* S;
  float* out;
  int transpose_out;
};

__global__ __launch_bounds__(256) void panel_small_kernel(PanelJob j0, PanelJob j1, int nb0, int l, int nt, int w) {
  __shared__ float Ps[kPanelRows * (kMaxL + 1)];
  __shared__ float Ss[kMaxL * kMaxL];
  const bool second = static_cast<int>(blockIdx.x) >= nb0;
  const PanelJob& jb = second ? j1 : j0;
  const float* __restrict__ P = jb.P;
  const float* __restrict__ S = jb.S;
  float* __restrict__ out = jb.out;
  const int64_t m = jb.m;
  const int transpose_out = jb.transpose_out;
  const int64_t r0 = static_cast<int64_t>(second ? blockIdx.x - nb0 : blockIdx.x) * kPanelRows;
  const int ldp = l + 1;
  for (int idx = threadIdx.x; idx < kPanelRows * l; idx += blockDim.x) {
    const int rr = idx / l, a = idx - rr * l;
    const int64_t row = r0 + rr;
    Ps[rr * ldp + a] = row < m ? P[frag_index(row, a, nt)] : 0.f;
  }
  for (int idx = threadIdx.x; idx < l * w; idx += blockDim.x) Ss[idx] = S[idx];
  __syncthreads();
  // wave wv: rows 16 wv .. 16 wv + 15 of the panel times S on fp32 MFMA (16x16x4:
  // lane L supplies A[L%16][L/16] and B[L/16][L%16], receives D[4(L/16)+v][L%16]),
  // K steps of 4 over a < l (zero beyond), one 16-column tile of S per accumulator
  static_assert(kPanelRows == 64, "four waves of 16 rows");
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6, li = lane & 15, g = lane >> 4;
  const int nct = (w + 15) >> 4;
  mfma_f4 acc[kMaxR / 16];
#pragma unroll
  for (int ct = 0; ct < kMaxR / 16; ++ct) acc[ct] = mfma_f4{0.f, 0.f, 0.f, 0.f};
  for (int kk = 0; kk < (l + 3) >> 2; ++kk) {
    const int a = 4 * kk + g;
    const float pa = a < l ? Ps[(16 * wv + li) * ldp + a] : 0.f;
#pragma unroll
    for (int ct = 0; ct < kMaxR / 16; ++ct) {
      if (ct < nct) {
        const int c = 16 * ct + li;
        const float sb = (a < l && c < w) ? Ss[a * w + c] : 0.f;
        acc[ct] = __builtin_amdgcn_mfma_f32_16x16x4f32(pa, sb, acc[ct], 0, 0, 0);
      }
    }
  }
#pragma unroll
  for (int ct = 0; ct < kMaxR / 16; ++ct) {
    if (ct >= nct) continue;
    const int c = 16 * ct + li;
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int64_t row = r0 + 16 * wv + 4 * g + v;
      if (row < m && c < w) {
        if (transpose_out) out[static_cast<int64_t>(c) * m + row] = acc[ct][v];
        else out[row * w + c] = acc[ct][v];
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Final stage of both exact paths: the n converged vectors x_j = sigma_j u_j
// (stride ldx) give sigma_j = |x_j|; the r largest (ties: lower index first)
// give the long-side factor x_j / sqrt(sigma_j) and the short-side factor
// (E-product with x_j) * sigma_j^(-3/2).  Every thread of the workgroup calls it.
template <typename T>
__device__ void exact_finish(const float* __restrict__ E, int64_t d, int64_t k, int r, const T* __restrict__ Xw,
                             int64_t ldx, int sweeps, float* __restrict__ B, float* __restrict__ A,
                             float* __restrict__ sigma, double* __restrict__ stats, const ObjectiveArgs& obj,
                             double* norm2, int* order) {
  const bool trans = k > d;
  const int n = static_cast<int>(trans ? d : k);
  const int64_t len = trans ? k : d;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, nwaves = blockDim.x >> 6;
  for (int v = wave; v < n; v += nwaves) {
    const T* xv = Xw + static_cast<int64_t>(v) * ldx;
    double s = 0.0;
    for (int64_t e = lane; e < len; e += 64) s += static_cast<double>(xv[e]) * static_cast<double>(xv[e]);
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
  const int64_t other = trans ? d : k;
  for (int64_t e = tid; e < static_cast<int64_t>(r) * (len + other); e += blockDim.x) {
    const int c = static_cast<int>(e / (len + other));
    const int64_t i = e - static_cast<int64_t>(c) * (len + other);
    const int j = order[c];
    const double sg = sqrt(norm2[j]);
    const T* xj = Xw + static_cast<int64_t>(j) * ldx;
    if (i < len) {
      const float val = sg > 0.0 ? static_cast<float>(static_cast<double>(xj[i]) / sqrt(sg)) : 0.f;
      if (trans) A[static_cast<int64_t>(c) * k + i] = val;
      else B[i * r + c] = val;
    } else {
      const int64_t o = i - len;
      double s = 0.0;
      if (trans) {
        for (int64_t t2 = 0; t2 < k; ++t2) s += static_cast<double>(E[o * k + t2]) * static_cast<double>(xj[t2]);
      } else {
        for (int64_t t2 = 0; t2 < d; ++t2) s += static_cast<double>(E[t2 * k + o]) * static_cast<double>(xj[t2]);
      }
      const float val = sg > 0.0 ? static_cast<float>(s / (sg * sqrt(sg))) : 0.f;
      if (trans) B[o * r + c] = val;
      else A[static_cast<int64_t>(c) * k + o] = val;
    }
  }
  if (tid < r) sigma[tid] = static_cast<float>(sqrt(norm2[order[tid]]));
  double s2 = 0.0;
  for (int c = 0; c < r; ++c) s2 += norm2[order[c]];
  if (tid == 0 && stats) {
    stats[0] = s2;
    stats[1] = sweeps;
  }
  write_objective(obj, s2);
}

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
  int sweeps = 0;
  for (int sweep = 0; sweep < 60; ++sweep) {
    if (tid == 0) rotated = 0;
    __syncthreads();
    sweeps = sweep + 1;
    for (int rnd = 0; rnd < N - 1; ++rnd) {
      if (len <= 256) {
        // Vectors of <= 256: a wave takes its pairs four at a time with every load of
        // the batch issued before the first reduction, and rotates in registers
        // (lane holds elements lane + 64 j, j < 4): the same arithmetic and order as
        // the loop below, with one memory round trip per batch instead of per pair.
        constexpr int kPB = 4;
        for (int i0 = wave; i0 < N / 2; i0 += nwaves * kPB) {
          double u[kPB][4], w[kPB][4];
          int pp[kPB], qq[kPB];
#pragma unroll
          for (int b = 0; b < kPB; ++b) {
            const int i = i0 + b * nwaves;
            int p = 0, q = 0;
            if (i < N / 2) {
              const int pa = rr_player(i, rnd, N), pb = rr_player(N - 1 - i, rnd, N);
              p = min(pa, pb);
              q = max(pa, pb);
            }
            pp[b] = p;
            qq[b] = (i < N / 2 && q < n) ? q : -1;
            const double* xp = Xw + static_cast<int64_t>(p) * len;
            const double* xq = Xw + static_cast<int64_t>(qq[b] < 0 ? p : q) * len;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
              const int64_t e = lane + 64 * j;
              u[b][j] = e < len ? xp[e] : 0.0;
              w[b][j] = e < len ? xq[e] : 0.0;
            }
          }
#pragma unroll
          for (int b = 0; b < kPB; ++b) {
            if (qq[b] < 0) continue;   // wave-uniform
            double al = 0.0, be = 0.0, ga = 0.0;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
              al += u[b][j] * u[b][j];
              be += w[b][j] * w[b][j];
              ga += u[b][j] * w[b][j];
            }
            for (int off = 32; off > 0; off >>= 1) {
              al += __shfl_xor(al, off);
              be += __shfl_xor(be, off);
              ga += __shfl_xor(ga, off);
            }
            if (ga == 0.0 || fabs(ga) <= 1e-14 * sqrt(al * be)) continue;
            const double zeta = (be - al) / (2.0 * ga);
            const double t = (zeta >= 0.0 ? 1.0 : -1.0) / (fabs(zeta) + sqrt(1.0 + zeta * zeta));
            const double c = 1.0 / sqrt(1.0 + t * t), sn = c * t;
            double* xp = Xw + static_cast<int64_t>(pp[b]) * len;
            double* xq = Xw + static_cast<int64_t>(qq[b]) * len;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
              const int64_t e = lane + 64 * j;
              if (e < len) {
                xp[e] = c * u[b][j] - sn * w[b][j];
                xq[e] = sn * u[b][j] + c * w[b][j];
              }
            }
            if (lane == 0) rotated = 1;
          }
        }
        __syncthreads();
        continue;
      }
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
    const int rot = rotated;
    __syncthreads();
    if (!rot) break;
  }
  exact_finish(E, d, k, r, Xw, len, sweeps, B, A, sigma, stats, obj, norm2, order);
}

// ---------------------------------------------------------------------------
// Exact SVD, block one-sided Jacobi.  The n vectors (padded with zero vectors
// to nb blocks of kBjW, nb even) live in fp64 in global memory, rows padded
// with zeros to ldx = 64 * NQ.  nb / 2 workgroups run concurrently (one
// cooperative launch); in block round rho workgroup g holds the block pair
// (rr_player(g, rho, nb), rr_player(nb - 1 - g, rho, nb)) in LDS and rotates
// every cross pair of the two blocks: in round j the 16-lane group c rotates
// column c of the first block (kept in its registers for all kBjW rounds)
// against column (c + j) mod kBjW of the second.  In block round 0 it first
// rotates the pairs inside each of its two blocks (round-robin, kBjW - 1
// rounds).  nb - 1 block rounds make one sweep, in which every pair of
// vectors meets once.  Between block rounds the workgroups write their blocks
// back and meet at a grid barrier.  A pair is rotated when
// |x_p . x_q| > kBjTol * |x_p| |x_q|.  The sweeps stop after the first sweep
// without a rotation (at most kBjMaxSweeps).
constexpr int kBjW = 16;
constexpr int kBjThreads = 16 * kBjW;   // one 16-lane group per pair
constexpr int kBjMaxNq = 9;             // vectors of up to 64 * kBjMaxNq = 576 elements
constexpr int kBjMaxSweeps = 60;
constexpr double kBjTol = 1e-7;
constexpr unsigned kBjSpinLimit = 1u << 20;

struct BjSync {
  unsigned bar;      // grid-barrier arrivals, monotone over the launch
  unsigned err;      // set when a barrier wait gave up
  unsigned sweeps;   // sweeps run
  unsigned pad;
  unsigned rot[kBjMaxSweeps];   // per sweep: workgroups that rotated
};
static_assert(sizeof(BjSync) <= 512, "BjSync");

// LDS of one workgroup: two blocks of (64 * NQ + 2)-double columns.
inline int64_t bj_nq(int64_t len) { return (len + 63) / 64; }
inline int64_t bj_lds_bytes(int64_t len) { return 2 * kBjW * (64 * bj_nq(len) + 2) * 8; }
constexpr int64_t kBjMaxLds = 159 * 1024;
inline bool bj_fits(int64_t len) { return bj_nq(len) <= kBjMaxNq && bj_lds_bytes(len) <= kBjMaxLds; }
inline int64_t bj_blocks(int64_t n) {
  const int64_t nb = (n + kBjW - 1) / kBjW;
  return nb + (nb & 1);
}

// Sum over the 16 lanes of a DPP row; every lane of the row ends with the
// same value (the pairings are symmetric, so each lane adds the same operands).
template <int CTRL>
__device__ __forceinline__ double bj_dpp(double v) {
  const int lo = __builtin_amdgcn_mov_dpp(__double2loint(v), CTRL, 0xF, 0xF, false);
  const int hi = __builtin_amdgcn_mov_dpp(__double2hiint(v), CTRL, 0xF, 0xF, false);
  return __hiloint2double(hi, lo);
}
__device__ __forceinline__ double bj_sum16(double v) {
  v += bj_dpp<0xB1>(v);    // quad_perm [1,0,3,2]
  v += bj_dpp<0x4E>(v);    // quad_perm [2,3,0,1]
  v += bj_dpp<0x141>(v);   // row_half_mirror
  v += bj_dpp<0x140>(v);   // row_mirror
  return v;
}

// Lane l16 of a 16-lane group holds elements 64 j + 4 l16 + e (e < 4) of a column.
template <int NQ>
__device__ __forceinline__ void bj_get(const double* col, int l16, double (&v)[NQ][4]) {
#pragma unroll
  for (int j = 0; j < NQ; ++j) {
    const double2* p = reinterpret_cast<const double2*>(col + 64 * j + 4 * l16);
    const double2 x = p[0], y = p[1];
    v[j][0] = x.x; v[j][1] = x.y; v[j][2] = y.x; v[j][3] = y.y;
  }
}
template <int NQ>
__device__ __forceinline__ void bj_put(double* col, int l16, const double (&v)[NQ][4]) {
#pragma unroll
  for (int j = 0; j < NQ; ++j) {
    double2* p = reinterpret_cast<double2*>(col + 64 * j + 4 * l16);
    p[0] = make_double2(v[j][0], v[j][1]);
    p[1] = make_double2(v[j][2], v[j][3]);
  }
}

// One Jacobi rotation of the pair (x_p, x_q) held by a 16-lane group; returns
// true if it rotated.
template <int NQ>
__device__ __forceinline__ bool bj_rot(double (&xp)[NQ][4], double (&xq)[NQ][4]) {
  double al = 0.0, be = 0.0, ga = 0.0;
#pragma unroll
  for (int j = 0; j < NQ; ++j)
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      al = fma(xp[j][e], xp[j][e], al);
      be = fma(xq[j][e], xq[j][e], be);
      ga = fma(xp[j][e], xq[j][e], ga);
    }
  al = bj_sum16(al);
  be = bj_sum16(be);
  ga = bj_sum16(ga);
  if (ga == 0.0 || ga * ga <= (kBjTol * kBjTol) * (al * be)) return false;
  // zeta = (be - al) / (2 ga) and t = sign(zeta) / (|zeta| + sqrt(1 + zeta^2)) only
  // pick the angle, so t is formed in fp32 (an angle off by ~1e-7 of itself still
  // shrinks the pair's dot by that factor); c = 1 / sqrt(1 + t^2) and s = c t are
  // formed in fp64 from that t, so the rotation stays orthogonal to fp64 rounding.
  const double g2 = 2.0 * ga;
  double rg = __builtin_amdgcn_rcp(g2);
  rg = fma(rg, fma(-g2, rg, 1.0), rg);
  const float zf = static_cast<float>((be - al) * rg);
  const float az = fabsf(zf);
  float tf = az > 1e18f ? 0.5f * __builtin_amdgcn_rcpf(az)
                        : __builtin_amdgcn_rcpf(az + __builtin_amdgcn_sqrtf(fmaf(az, az, 1.f)));
  const double t = zf >= 0.f ? tf : -tf;
  const double x = fma(t, t, 1.0);
  double c = __builtin_amdgcn_rsq(x);
  c = c * fma(-0.5 * x * c, c, 1.5);
  c = c * fma(-0.5 * x * c, c, 1.5);
  const double sn = c * t;
#pragma unroll
  for (int j = 0; j < NQ; ++j)
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const double u = xp[j][e], w = xq[j][e];
      xp[j][e] = fma(c, u, -(sn * w));
      xq[j][e] = fma(sn, u, c * w);
    }
  return true;
}

// Block pair (bp, bq) between X (stride 64 NQ doubles) and LDS (stride
// 64 NQ + 2): each thread issues all of its loads before its first store.
template <int NQ>
__device__ __forceinline__ void bj_move(double* X, int bp, int bq, bool load, double* lds) {
  constexpr int per_col = 32 * NQ;   // double2 per column
  constexpr int ldl = 64 * NQ + 2;
  constexpr int kPer = 2 * kBjW * per_col / kBjThreads;
  static_assert(kPer * kBjThreads == 2 * kBjW * per_col, "block pair split");
  double2 v[kPer];
  double2* gp[kPer];
  double2* lp[kPer];
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    const int idx = static_cast<int>(threadIdx.x) + i * kBjThreads;
    const int col = idx / per_col, q = idx - col * per_col;
    const int64_t gc = col < kBjW ? static_cast<int64_t>(bp) * kBjW + col : static_cast<int64_t>(bq) * kBjW + col - kBjW;
    gp[i] = reinterpret_cast<double2*>(X + gc * (64 * NQ)) + q;
    lp[i] = reinterpret_cast<double2*>(lds + col * ldl) + q;
  }
  if (load) {
#pragma unroll
    for (int i = 0; i < kPer; ++i) v[i] = *gp[i];
#pragma unroll
    for (int i = 0; i < kPer; ++i) *lp[i] = v[i];
  } else {
#pragma unroll
    for (int i = 0; i < kPer; ++i) v[i] = *lp[i];
#pragma unroll
    for (int i = 0; i < kPer; ++i) *gp[i] = v[i];
  }
}

// Grid barrier for the co-resident workgroups of a cooperative launch: thread 0
// publishes the workgroup's stores (device-scope release), arrives, waits until
// `target` arrivals and acquires the others' stores; the wait is bounded, and a
// wait that gives up (or sees that another workgroup gave up) sets err and makes
// every workgroup leave.
__device__ bool bj_grid_barrier(BjSync* sy, unsigned target) {
  __shared__ int ok;
  __syncthreads();
  if (threadIdx.x == 0) {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
    atomicAdd(&sy->bar, 1u);
    int good = 1;
    unsigned spins = 0;
    while (__hip_atomic_load(&sy->bar, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) < target) {
      if (__hip_atomic_load(&sy->err, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != 0u || ++spins > kBjSpinLimit) {
        atomicOr(&sy->err, 1u);
        good = 0;
        break;
      }
      __builtin_amdgcn_s_sleep(2);
    }
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
    ok = good;
  }
  __syncthreads();
  return ok != 0;
}

__global__ void bj_load_kernel(const float* __restrict__ E, int64_t d, int64_t k, int n, int64_t ncols, int64_t ldx,
                               double* __restrict__ X) {
  const int64_t e = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (e >= ncols * ldx) return;
  const bool trans = k > d;
  const int64_t len = trans ? k : d;
  const int64_t c = e / ldx, i = e - c * ldx;
  double v = 0.0;
  if (c < n && i < len) v = trans ? E[c * k + i] : E[i * k + c];
  X[e] = v;
}

template <int NQ>
__global__ __launch_bounds__(kBjThreads) void bj_sweep_kernel(double* __restrict__ X, BjSync* __restrict__ sy) {
  extern __shared__ double2 bj_lds2[];
  double* lds = reinterpret_cast<double*>(bj_lds2);
  constexpr int ldl = 64 * NQ + 2;
  __shared__ int any_rot;
  const int G = gridDim.x, nb = 2 * G, g = blockIdx.x;
  const int tid = threadIdx.x, grp = tid >> 4, l16 = tid & 15;
  unsigned nbar = 0;
  int sweep = 0;
  for (; sweep < kBjMaxSweeps; ++sweep) {
    if (tid == 0) any_rot = 0;
    for (int rnd = 0; rnd < nb - 1; ++rnd) {
      const int bp = rr_player(g, rnd, nb), bq = rr_player(nb - 1 - g, rnd, nb);
      bj_move<NQ>(X, bp, bq, true, lds);
      __syncthreads();
      bool rot = false;
      double xa[NQ][4], xb[NQ][4];
      if (rnd == 0) {
        const int blk = grp / (kBjW / 2), i = grp % (kBjW / 2);
        for (int ir = 0; ir < kBjW - 1; ++ir) {
          const int x = rr_player(i, ir, kBjW), y = rr_player(kBjW - 1 - i, ir, kBjW);
          double* cp = lds + (blk * kBjW + min(x, y)) * ldl;
          double* cq = lds + (blk * kBjW + max(x, y)) * ldl;
          bj_get<NQ>(cp, l16, xa);
          bj_get<NQ>(cq, l16, xb);
          if (bj_rot<NQ>(xa, xb)) {
            rot = true;
            bj_put<NQ>(cp, l16, xa);
            bj_put<NQ>(cq, l16, xb);
          }
          __syncthreads();
        }
      }
      // cross pairs: column grp of the first block stays in xa
      double* ca = lds + grp * ldl;
      bj_get<NQ>(ca, l16, xa);
      for (int j = 0; j < kBjW; ++j) {
        double* cb = lds + (kBjW + (grp + j) % kBjW) * ldl;
        bj_get<NQ>(cb, l16, xb);
        if (bp < bq ? bj_rot<NQ>(xa, xb) : bj_rot<NQ>(xb, xa)) {
          rot = true;
          bj_put<NQ>(cb, l16, xb);
        }
        __syncthreads();
      }
      bj_put<NQ>(ca, l16, xa);
      if (rot && l16 == 0) any_rot = 1;
      __syncthreads();
      bj_move<NQ>(X, bp, bq, false, lds);
      if (rnd == nb - 2) {
        __syncthreads();
        if (tid == 0 && any_rot) atomicAdd(&sy->rot[sweep], 1u);
      }
      if (!bj_grid_barrier(sy, static_cast<unsigned>(G) * ++nbar)) return;
    }
    // every workgroup's count for this sweep arrived before the last barrier
    if (__hip_atomic_load(&sy->rot[sweep], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == 0u) break;
  }
  if (g == 0 && tid == 0) sy->sweeps = static_cast<unsigned>(sweep < kBjMaxSweeps ? sweep + 1 : kBjMaxSweeps);
}

using BjSweepFn = void (*)(double*, BjSync*);
constexpr BjSweepFn kBjSweep[kBjMaxNq] = {bj_sweep_kernel<1>, bj_sweep_kernel<2>, bj_sweep_kernel<3>,
                                          bj_sweep_kernel<4>, bj_sweep_kernel<5>, bj_sweep_kernel<6>,
                                          bj_sweep_kernel<7>, bj_sweep_kernel<8>, bj_sweep_kernel<9>};

__global__ __launch_bounds__(1024) void bj_finish_kernel(const float* __restrict__ E, int64_t d, int64_t k, int r,
                                                        const double* __restrict__ X, int64_t ldx,
                                                        const BjSync* __restrict__ sy, float* __restrict__ B,
                                                        float* __restrict__ A, float* __restrict__ sigma,
                                                        double* __restrict__ stats, ObjectiveArgs obj) {
  __shared__ double norm2[kMaxExact];
  __shared__ int order[kMaxExact];
  exact_finish(E, d, k, r, X, ldx, static_cast<int>(sy->sweeps), B, A, sigma, stats, obj, norm2, order);
  if (sy->err != 0u) {   // a barrier wait gave up: no valid result
    if (threadIdx.x < r) sigma[threadIdx.x] = __builtin_nanf("");
    if (threadIdx.x == 0 && stats) stats[2] = 1.0;
  }
}

__global__ __launch_bounds__(256) void objective_kernel(ObjectiveArgs obj) { write_objective(obj, 0.0); }

__global__ void fill_kernel(float* __restrict__ p, int64_t n, float v) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i < n) p[i] = v;
}

__global__ void zero_u32_kernel(unsigned* __restrict__ p, int n) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = 0u;
}

// ---------------------------------------------------------------------------
int64_t round_up(int64_t x, int64_t m) { return (x + m - 1) / m * m; }
int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

template <int NT>
void reduce_typed(const float* part, int S, int64_t m, int64_t m_pad, int l, const float* X, float* out,
                  uint16_t* out_split, double* gram_parts, bool paired, hipStream_t s) {
  const int blocks = static_cast<int>(cdiv(m_pad, kGramRows));
  LQ_LAUNCH("reduce_gram", (reduce_gram_kernel<NT>), dim3(blocks), dim3(kReduceThreads), 0, s, part, S, m, m_pad, l, X, out,
            out_split, gram_parts, paired ? 1 : 0);
}

void launch_reduce(int nt, const float* part, int S, int64_t m, int64_t m_pad, int l, const float* X, float* out,
                   uint16_t* out_split, double* gram_parts, bool paired, hipStream_t s) {
  switch (nt) {
    case 1: reduce_typed<1>(part, S, m, m_pad, l, X, out, out_split, gram_parts, paired, s); break;
    case 2: reduce_typed<2>(part, S, m, m_pad, l, X, out, out_split, gram_parts, paired, s); break;
    case 3: reduce_typed<3>(part, S, m, m_pad, l, X, out, out_split, gram_parts, paired, s); break;
    case 4: reduce_typed<4>(part, S, m, m_pad, l, X, out, out_split, gram_parts, paired, s); break;
    default: reduce_typed<5>(part, S, m, m_pad, l, X, out, out_split, gram_parts, paired, s); break;
  }
}

// mode 1 factors the summed Gram `gram`; mode 2 sums the P partials `gparts` itself.
template <int LM>
void small_wave_typed(int mode, const double* gram, const double* gparts, int P, int l, float* Xinv, int r, float* SB,
                      float* SA, float* sigma, double* stats, const ObjectiveArgs& obj, hipStream_t s) {
  if (mode == 1)
    LQ_LAUNCH("chol_inv", chol_inv_wave_kernel<LM>, dim3(1), dim3(64), 0, s, gram, l, Xinv);
  else
    LQ_LAUNCH("core_svd", core_small_kernel<LM>, dim3(1), dim3(256), 0,
              s, gparts, P, l, Xinv, r, SB, SA, sigma, stats, obj);
}

// l <= 32: the register Cholesky is unrolled for the smallest of 8/16/24/32 rows that holds l.
void launch_small_wave(int mode, const double* gram, const double* gparts, int P, int l, float* Xinv, int r, float* SB,
                       float* SA, float* sigma, double* stats, const ObjectiveArgs& obj, hipStream_t s) {
  if (l <= 8) small_wave_typed<8>(mode, gram, gparts, P, l, Xinv, r, SB, SA, sigma, stats, obj, s);
  else if (l <= 16) small_wave_typed<16>(mode, gram, gparts, P, l, Xinv, r, SB, SA, sigma, stats, obj, s);
  else if (l <= 24) small_wave_typed<24>(mode, gram, gparts, P, l, Xinv, r, SB, SA, sigma, stats, obj, s);
  else small_wave_typed<32>(mode, gram, gparts, P, l, Xinv, r, SB, SA, sigma, stats, obj, s);
}

void panels(const PanelJob& j0, const PanelJob& j1, int l, int nt, int w, hipStream_t s) {
  const int nb0 = static_cast<int>(cdiv(j0.m, kPanelRows)), nb1 = static_cast<int>(cdiv(j1.m, kPanelRows));
  LQ_LAUNCH("panel_small", panel_small_kernel, dim3(nb0 + nb1), dim3(256), 0, s, j0, j1, nb0, l, nt, w);
}

}  // namespace

// ---------------------------------------------------------------------------
SvdPlan make_svd_plan(int64_t d, int64_t k, int r, int oversample, bool exact) {
  SvdPlan p{};
  p.d = d; p.k = k; p.r = r; p.exact = exact;
  int64_t off = 0;
  auto take = [&](int64_t bytes) { const int64_t o = off; off += round_up(bytes, 256); return o; };
  if (exact) {
    const int64_t n = d < k ? d : k;
    const int64_t len = d > k ? d : k;
    p.l = static_cast<int>(n);
    p.bj = bj_fits(len);
    int64_t xbytes = (n + 1) * len * 8;   // fp64 vectors of the single-workgroup Jacobi
    if (p.bj) {
      const int64_t nb = bj_blocks(n);
      const int64_t bj_bytes = nb * kBjW * bj_nq(len) * 64 * 8;
      if (bj_bytes > xbytes) xbytes = bj_bytes;
    }
    p.off_x = take(xbytes);
    p.off_sync = take(sizeof(BjSync));
    p.off_stats = take(64);
    p.bytes = off;
    return p;
  }
  const int l = r + oversample;
  p.l = l;
  p.nt = static_cast<int>(cdiv(l, 16));
  const int LP = 16 * p.nt;
  // Split of the contraction (split-K count S): among the counts that keep the
  // split-K partials under ~8% of E's bytes (S * LP / len) and give every split
  // at least one unit of the kernel's K granularity, the smallest S whose grid
  // best fills the 256 CUs of the chip -- score = (occupancy of the last wave
  // of workgroups) x min(1, workgroups / 512).
  constexpr int64_t kCUs = 256;
  // max_wgs > 0 only admits counts whose grid stays within max_wgs workgroups;
  // returns 0 if none does.
  auto choose = [&](int64_t tiles, int64_t len, int unit, int64_t max_wgs, int64_t& per) {
    int64_t cap = (len * 8) / (100 * LP);
    if (cap < 1) cap = 1;
    if (cap > cdiv(len, unit)) cap = cdiv(len, unit);
    int64_t best_s = 0;
    double best = -1.0;
    for (int64_t sp = 1; sp <= cap; ++sp) {
      const int64_t ps = round_up(cdiv(len, sp), unit);
      if (cdiv(len, ps) != sp) continue;   // rounding merges this count into another
      const int64_t wgs = tiles * sp;
      if (max_wgs > 0 && wgs > max_wgs) continue;
      const double fill = static_cast<double>(wgs) / static_cast<double>(kCUs * cdiv(wgs, kCUs));
      const double busy = wgs >= 2 * kCUs ? 1.0 : static_cast<double>(wgs) / static_cast<double>(2 * kCUs);
      if (fill * busy > best + 1e-9) {
        best = fill * busy;
        best_s = sp;
      }
    }
    if (best_s == 0) return 0;
    per = round_up(cdiv(len, best_s), unit);
    return static_cast<int>(cdiv(len, per));
  };
  const GemmShape nn = gemm_shape(false, p.nt, d, k), tn = gemm_shape(true, p.nt, d, k);
  p.nn_row_blocks = static_cast<int>(cdiv(d, nn.tile));
  p.nn_splits = choose(p.nn_row_blocks, k, nn.unit, 0, p.nn_kper);
  p.tn_col_blocks = static_cast<int>(cdiv(k, tn.tile));
  p.tn_splits = choose(p.tn_col_blocks, d, tn.unit, 0, p.tn_rper);
  // Mid-size E with a wide panel takes its orthonormalisation solves on the side
  // lane (run_lowrank); E^T Y then leaves a CU free for them, as for the ride-along
  // Cholesky below (measured on MI355X: 11008 x 4096 at l = 80, 4.14 -> 4.04 ms
  // per init; the larger E of 8192 x 28672 keeps its full grid, its E^T Y outlasts
  // the solves anyway).
  if (l > 32 && d * k >= kSideMinElems && d * k < kSideFullGridElems) {
    int64_t rper = 0;
    const int sc = choose(p.tn_col_blocks, d, tn.unit, kCUs - 1, rper);
    if (sc > 0) {
      p.tn_splits = sc;
      p.tn_rper = rper;
    }
  }
  // The Cholesky that rides along with E^T Y (l <= 32) is a serial chain that
  // slows several-fold when a streaming workgroup shares its CU, so it rides
  // only where a split leaves a CU free while still covering at least three
  // quarters of the chip; otherwise it keeps launches of its own.
  p.ride = false;
  if (l <= 32) {
    int64_t rper = 0;
    const int sr = choose(p.tn_col_blocks, d, tn.unit, kCUs - 1, rper);
    if (sr > 0 && p.tn_col_blocks * sr * 4 >= 3 * kCUs) {
      p.ride = true;
      p.tn_splits = sr;
      p.tn_rper = rper;
    }
  }
  p.k_pad = p.nn_splits * p.nn_kper;
  p.d_pad = p.tn_splits * p.tn_rper;
  // the products step K by 32 (E^T Y by pairs of steps), so k_pad and d_pad are multiples of 64
  p.gram_parts_d = static_cast<int>(cdiv(d, kGramRows));
  p.gram_parts_k = static_cast<int>(cdiv(k, kGramRows));
  const int64_t gp = p.gram_parts_d > p.gram_parts_k ? p.gram_parts_d : p.gram_parts_k;
  const int64_t E = static_cast<int64_t>(l) * (l + 1) / 2;
  p.off_omega = take(p.k_pad * LP * 4);
  p.off_y = take(p.d_pad * LP * 4);
  p.off_z = take(p.k_pad * LP * 4);
  const int64_t part_rows = (p.nn_splits * d > p.tn_splits * k) ? p.nn_splits * d : p.tn_splits * k;
  p.off_part = take(part_rows * LP * 4);
  p.off_gram_parts = take(gp * E * 8);
  p.off_gram_total = take(E * 8);
  p.off_rinv = take(static_cast<int64_t>(l) * l * 4);
  p.off_sb = take(static_cast<int64_t>(l) * r * 4);
  p.off_sa = take(static_cast<int64_t>(l) * r * 4);
  p.off_stats = take(64);
  p.off_omega_s = take(p.k_pad * LP * 4);
  p.off_z_s = take(p.k_pad * LP * 4);
  p.off_y_s = take(p.d_pad * LP * 4);
  p.bytes = off;
  return p;
}

hipError_t run_sketch(uint64_t seed, int t, int count, int64_t k, int l, int nt, int64_t rows, float* out,
                      hipStream_t s) {
  const int64_t n = rows * 16 * nt;
  LQ_LAUNCH("sketch", sketch_kernel, dim3(static_cast<unsigned>(cdiv(n, 256)), static_cast<unsigned>(count)), dim3(256),
            0, s, seed, t, k, l, nt, rows, out);
  return hipGetLastError();
}

hipError_t run_sketch_split(uint64_t seed, int t, int count, int64_t k, int l, int nt, int64_t rows, uint16_t* out,
                            hipStream_t s) {
  const int64_t n = (rows / 32) * nt * 2 * 64;
  LQ_LAUNCH("sketch", sketch_split_kernel, dim3(static_cast<unsigned>(cdiv(n, 256)), static_cast<unsigned>(count)),
            dim3(256), 0, s, seed, t, k, l, nt, rows, out);
  return hipGetLastError();
}

hipError_t run_warm_columns(const float* A, const float* sigma, int64_t k, int r, int nt, float* out, hipStream_t s) {
  const int64_t n = k * r;
  if (n <= 0) return hipSuccess;
  LQ_LAUNCH("warm_sketch", warm_columns_kernel, dim3(static_cast<unsigned>(cdiv(n, 256))), dim3(256), 0, s, A, sigma, k,
            r, nt, out);
  return hipGetLastError();
}

hipError_t run_fill(float* p, int64_t n, float v, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  LQ_LAUNCH("fill", fill_kernel, dim3(static_cast<unsigned>(cdiv(n, 256))), dim3(256), 0, s, p, n, v);
  return hipGetLastError();
}

hipError_t run_objective(const ObjectiveArgs& obj, hipStream_t s) {
  LQ_LAUNCH("objective", objective_kernel, dim3(1), dim3(256), 0, s, obj);
  return hipGetLastError();
}

hipError_t run_lowrank(const float* E, const SvdPlan& pl, int q, const float* omega, const float* omega_frag,
                       uint64_t seed, int t, float* B, float* A, float* sigma, char* ws, const ObjectiveArgs& obj,
                       hipStream_t s, SideLane* side, const VirtualE* ve, const uint16_t* omega_split,
                       double* norm_parts) {
  const int64_t d = pl.d, k = pl.k;
  const int r = pl.r, l = pl.l;
  if (pl.exact && pl.bj) {
    const int64_t n = d < k ? d : k, len = d > k ? d : k;
    const int nq = static_cast<int>(bj_nq(len));
    const int nb = static_cast<int>(bj_blocks(n));
    const int64_t ldx = 64 * static_cast<int64_t>(nq);
    const int64_t ncols = static_cast<int64_t>(nb) * kBjW;
    double* X = reinterpret_cast<double*>(ws + pl.off_x);
    BjSync* sy = reinterpret_cast<BjSync*>(ws + pl.off_sync);
    double* stats = reinterpret_cast<double*>(ws + pl.off_stats);
    LQ_LAUNCH("zero_u32", zero_u32_kernel, dim3(1), dim3(256), 0, s, reinterpret_cast<unsigned*>(sy),
              static_cast<int>(sizeof(BjSync) / 4));
    LQ_LAUNCH("exact_load", bj_load_kernel, dim3(static_cast<unsigned>(cdiv(ncols * ldx, 256))), dim3(256), 0, s, E, d,
              k, static_cast<int>(n), ncols, ldx, X);
    {
      ProfScope ps("exact_sweeps");
      if (ps.start()) (void)hipEventRecord(ps.start(), s);
      void* args[] = {&X, &sy};
      const hipError_t e = hipLaunchCooperativeKernel(reinterpret_cast<const void*>(kBjSweep[nq - 1]), dim3(nb / 2),
                                                      dim3(kBjThreads), args, static_cast<unsigned>(bj_lds_bytes(len)), s);
      if (ps.stop()) (void)hipEventRecord(ps.stop(), s);
      if (e != hipSuccess) return e;
    }
    LQ_LAUNCH("exact_finish", bj_finish_kernel, dim3(1), dim3(1024), 0, s, E, d, k, r, X, ldx, sy, B, A, sigma, stats,
              obj);
    return hipGetLastError();
  }
  if (pl.exact) {
    double* Xw = reinterpret_cast<double*>(ws + pl.off_x);
    LQ_LAUNCH("exact_jacobi", exact_jacobi_kernel, dim3(1), dim3(1024), 0, s, E, d, k, r, Xw, B, A, sigma,
              reinterpret_cast<double*>(ws + pl.off_stats), obj);
    return hipGetLastError();
  }
  const float* Om = omega_frag != nullptr ? omega_frag : reinterpret_cast<float*>(ws + pl.off_omega);
  float* Om_ws = reinterpret_cast<float*>(ws + pl.off_omega);
  float* Y = reinterpret_cast<float*>(ws + pl.off_y);
  float* Z = reinterpret_cast<float*>(ws + pl.off_z);
  float* part = reinterpret_cast<float*>(ws + pl.off_part);
  double* gparts = reinterpret_cast<double*>(ws + pl.off_gram_parts);
  float* Xinv = reinterpret_cast<float*>(ws + pl.off_rinv);
  float* SB = reinterpret_cast<float*>(ws + pl.off_sb);
  float* SA = reinterpret_cast<float*>(ws + pl.off_sa);
  double* stats = reinterpret_cast<double*>(ws + pl.off_stats);
  const ObjectiveArgs none{nullptr, 0, nullptr, 0, nullptr, nullptr};
  const int64_t nfrag = pl.k_pad * 16 * pl.nt;
  if (omega != nullptr && omega_split == nullptr) {
    LQ_LAUNCH("to_frag", to_frag_kernel, dim3(static_cast<unsigned>(cdiv(nfrag, 256))), dim3(256), 0, s, omega, k, l,
              pl.nt, pl.k_pad, Om_ws);
    Om = Om_ws;
  } else if (omega_frag == nullptr && omega_split == nullptr) {
    hipError_t e = run_sketch(seed, t, 1, k, l, pl.nt, pl.k_pad, Om_ws, s);
    if (e != hipSuccess) return e;
  }
  // split copies of the panels for the bf16 products (a sketch may come split already)
  const uint16_t* Om_s = omega_split;
  uint16_t* Y_s = reinterpret_cast<uint16_t*>(ws + pl.off_y_s);
  uint16_t* Z_s = reinterpret_cast<uint16_t*>(ws + pl.off_z_s);
  if (Om_s == nullptr) {
    uint16_t* os = reinterpret_cast<uint16_t*>(ws + pl.off_omega_s);
    const int64_t units = (pl.k_pad / 32) * pl.nt * 64;
    LQ_LAUNCH("split_panel", split_panel_kernel, dim3(static_cast<unsigned>(cdiv(units, 256))), dim3(256), 0, s, Om,
              pl.k_pad, pl.nt, os);
    Om_s = os;
  }
  double* gtotal = reinterpret_cast<double*>(ws + pl.off_gram_total);
  const int E_ = l * (l + 1) / 2;
  // product and split-K reduction; mode 1 then orthonormalises (Gram, Cholesky,
  // X = R^-1), mode 2 runs the core solve, mode 0 keeps the product.  E P goes
  // to Y (fragment order, d_pad rows, not orthonormalised: Q = Y X); E^T Y goes
  // through X to Z = E^T Q (fragment order, k_pad rows).
  // For l <= 32 the Cholesky of Y's Gram (mode 1) needs no launch of its own:
  // it rides along with the E^T Y product that always follows, whose split-K
  // reduction is the first consumer of X.
  // The fork and join between the streams cost several microseconds, and the
  // solves slow down several-fold on a CU shared with the product's waves: the
  // side lane is taken only for E of at least kSideMinElems elements, whose E^T Y
  // leaves a CU free (make_svd_plan) or runs long enough to cover the solves.
  if (d * k < kSideMinElems) side = nullptr;
  const bool ride = pl.ride;
  bool pending = false, joining = false;
  hipError_t serr = hipSuccess;
  auto product = [&](bool transposed, const uint16_t* panel_s, int mode, double* nparts = nullptr) {
    const CholJob job{pending ? gparts : nullptr, pl.gram_parts_d, l, Xinv};
    launch_gemm(transposed, E, d, k, panel_s, pl, part, job, s, ve, nparts);
    if (transposed) pending = false;
    if (transposed && joining) {   // X = R^-1 from the side lane
      if (serr == hipSuccess) serr = hipStreamWaitEvent(s, side->join, 0);
      joining = false;
    }
    if (transposed)
      launch_reduce(pl.nt, part, pl.tn_splits, k, pl.k_pad, l, Xinv, Z, mode == 2 ? nullptr : Z_s,
                    mode ? gparts : nullptr, false, s);
    else
      launch_reduce(pl.nt, part, pl.nn_splits, d, pl.d_pad, l, nullptr, Y, Y_s, mode ? gparts : nullptr, true, s);
    if (mode == 0) return;
    if (mode == 1 && ride) {
      pending = true;
      return;
    }
    const int P = transposed ? pl.gram_parts_k : pl.gram_parts_d;
    if (l <= 32 && mode == 2) {
      launch_small_wave(2, nullptr, gparts, P, l, Xinv, r, SB, SA, sigma, stats, obj, s);
      return;
    }
    // mode 1 (always followed by an E^T Y product): on the side lane when there is one
    hipStream_t ss = s;
    if (mode == 1 && side != nullptr) {
      if (serr == hipSuccess) serr = hipEventRecord(side->fork, s);
      if (serr == hipSuccess) serr = hipStreamWaitEvent(side->stream, side->fork, 0);
      ss = side->stream;
    }
    LQ_LAUNCH("gram_sum", gram_sum_kernel, dim3((E_ + 63) / 64), dim3(1024), 0, ss, gparts, P, E_, gtotal);
    if (l <= 32)
      launch_small_wave(1, gtotal, nullptr, 0, l, Xinv, r, SB, SA, sigma, stats, none, ss);
    else if (mode == 1)
      LQ_LAUNCH("chol_inv", (solve_wide_kernel<1, kWideCholWaves, 16>), dim3(1), dim3(64 * kWideCholWaves), 0, ss,
                gtotal, l, Xinv, r, SB, SA, sigma, stats, none);
    else
      LQ_LAUNCH("core_svd", (solve_wide_kernel<2, 10, kWideGroup>), dim3(1), dim3(640), 0, s, gtotal, l, Xinv, r, SB,
                SA, sigma, stats, obj);
    if (ss != s) {
      if (serr == hipSuccess) serr = hipEventRecord(side->join, ss);
      joining = true;
    }
  };
  // Y = E Omega; X = R^-1 of its Gram.  Each power iteration multiplies by E^T
  // and E and re-orthonormalises Y only: span(E Z) does not depend on Z's basis,
  // so orthonormalising Z as well would not change the subspace.
  product(false, Om_s, 1, norm_parts);
  for (int it = 0; it < q; ++it) {
    product(true, Y_s, 0);
    product(false, Z_s, 1);
  }
  // C = E^T Q = (E^T Y) X, then the core solve on C^T C
  product(true, Y_s, 2);
  panels(PanelJob{Y, d, SB, B, 0}, PanelJob{Z, k, SA, A, 1}, l, pl.nt, r, s);
  if (serr != hipSuccess) return serr;
  return hipGetLastError();
}

SideLane* side_lane_for(hipStream_t s) {
  static std::mutex mu;
  static std::map<std::pair<int, hipStream_t>, SideLane> lanes;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return nullptr;
  std::lock_guard<std::mutex> lk(mu);
  const auto key = std::make_pair(dev, s);
  auto it = lanes.find(key);
  if (it != lanes.end()) return &it->second;
  SideLane lane{};
  if (hipStreamCreateWithFlags(&lane.stream, hipStreamNonBlocking) != hipSuccess) return nullptr;
  lane.mu = new std::mutex;
  if (hipEventCreateWithFlags(&lane.fork, hipEventDisableTiming) != hipSuccess ||
      hipEventCreateWithFlags(&lane.join, hipEventDisableTiming) != hipSuccess)
    return nullptr;
  return &lanes.emplace(key, lane).first->second;
}

}  // namespace loftq
