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
//   sketch        counter-based +-1 test matrix (SplitMix64)
//   reduce_gram   fixed-order sum of the split-K partials (+ fp64 Gram partials)
//   gram_sum      fixed-order sum of the Gram partials
//   chol_inv      Cholesky of the Gram and X = R^-1 (orthonormalisation); for
//                 l <= 32 it usually rides along with the next E^T Y product
//   core_svd      the l x l core solve: Cholesky, one-sided Jacobi, S_B, S_A
//   panel_small   P S for a row panel P and a small S: B = Q S_B, A = (C S_A)^T
//   exact_jacobi  single-workgroup one-sided Jacobi SVD for tiny matrices
// Every reduction runs in a fixed order, so results are deterministic.
#include "lowrank.h"
#include "reduce.h"
#include "small_solve.h"

namespace loftq {
namespace {

// ---------------------------------------------------------------------------
// Element (i, j) of the k x l test matrix of alternation t is drawn from
// counter ((t - 1) k + i) l + j; written in fragment order over `rows` rows
// (zero beyond k and l).
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
  float v = 0.f;
  if (i < k && j < l) {
    const uint64_t c = (static_cast<uint64_t>(t - 1) * static_cast<uint64_t>(k) + static_cast<uint64_t>(i)) *
                           static_cast<uint64_t>(l) + static_cast<uint64_t>(j);
    uint64_t z = seed + (c + 1) * 0x9E3779B97F4A7C15ull;
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    z ^= z >> 31;
    v = (z >> 63) ? -1.f : 1.f;
  }
  out[idx] = v;
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
// group ends with the same total.
template <int G>
__device__ __forceinline__ float group_sumf(float v) {
  static_assert(G == 16 || G == 8 || G == 4, "16-, 8- or 4-lane groups");
  if (G == 16) {
    v += dpp_f32<0x128>(v);   // row_ror:8
    v += dpp_f32<0x124>(v);   // row_ror:4
    v += dpp_f32<0x122>(v);   // row_ror:2
    v += dpp_f32<0x121>(v);   // row_ror:1
  } else {
    v += dpp_f32<0xB1>(v);    // quad_perm xor 1
    v += dpp_f32<0x4E>(v);    // quad_perm xor 2
    if (G == 8) v += dpp_f32<0x141>(v);   // row_half_mirror: the other quad of the 8
  }
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

// Round-robin (circle) pairing of the n columns: in round rnd, slot i < n / 2
// pairs the players at positions i and n - 1 - i.  sched[rnd * np + i] holds the
// byte offsets (column times ld floats) of the slot's lower and higher column in
// its low and high 16 bits.  Slots n / 2 .. np - 1 (lanes that pad the last
// wave) get columns 2 np - 2 and 2 np - 1, which the caller keeps zero.
__device__ void build_schedule(uint32_t* sched, int n, int np, int ld) {
  for (int e = threadIdx.x; e < (n - 1) * np; e += blockDim.x) {
    const int rnd = e / np, i = e - rnd * np;
    int p = 2 * np - 2, q = 2 * np - 1;
    if (i < n / 2) {
      const int x = rr_player(i, rnd, n), y = rr_player(n - 1 - i, rnd, n);
      p = x < y ? x : y;
      q = x < y ? y : x;
    }
    sched[e] = static_cast<uint32_t>(p * ld * 4) | (static_cast<uint32_t>(q * ld * 4) << 16);
  }
}

// One-sided Jacobi sweeps on the columns of K (fp32, LDS; rows GW * RL and
// beyond the matrix are zero), GW lanes per column pair: lane `sub` holds rows
// sub + GW i (i < RL) of both columns for the round.  With alpha, beta the
// squared norms and gamma the dot product, the rotation by theta,
// tan 2 theta = 2 gamma / (beta - alpha), |theta| <= pi / 4, is taken in the
// branch-free form cos 2 theta = |beta - alpha| / h, h = hypot(beta - alpha,
// 2 gamma), c = sqrt((1 + cos 2 theta) / 2), s = sin 2 theta / (2 c).  A pair
// is left alone while gamma^2 <= 1e-14 alpha beta.  The sweeps stop after one in
// which every pair had gamma^2 <= 1e-8 alpha beta (|cos| <= 1e-4).  Convergence is
// quadratic once the couplings are below the relative gaps of the singular
// values; with the nearly flat spectra of quantization residuals (neighbouring
// values ~1% apart) a 1e-3 cut left couplings near 1e-5, visible in the
// orthogonality of A, while 1e-4 leaves them at the fp32 rounding level.  All
// threads call it; returns the sweeps.
template <int GW, int RL>
__device__ int jacobi_columns(float* K, const uint32_t* sched, int n, int max_sweeps) {
  const int np = __builtin_amdgcn_readfirstlane(blockDim.x / GW);   // uniform: next row's offset is scalar
  const int pair = threadIdx.x / GW, sub = threadIdx.x - pair * GW;
  char* base = reinterpret_cast<char*>(K + sub);
  const int rounds = n - 1;
  uint32_t pq = sched[pair];
  int sweeps = 0;
  for (int sweep = 0; sweep < max_sweeps; ++sweep) {
    uint64_t big = 0;
    for (int rnd = 0; rnd < rounds; ++rnd) {
      const uint32_t pq_next = sched[(rnd + 1 < rounds ? rnd + 1 : 0) * np + pair];
      float* kp = reinterpret_cast<float*>(base + (pq & 0xFFFFu));
      float* kq = reinterpret_cast<float*>(base + (pq >> 16));
      float xp[RL], xq[RL];
      float al = 0.f, be = 0.f, ga = 0.f;
#pragma unroll
      for (int i = 0; i < RL; ++i) {
        xp[i] = kp[GW * i];
        xq[i] = kq[GW * i];
      }
#pragma unroll
      for (int i = 0; i < RL; ++i) {
        al = fmaf(xp[i], xp[i], al);
        be = fmaf(xq[i], xq[i], be);
        ga = fmaf(xp[i], xq[i], ga);
      }
      al = group_sumf<GW>(al);
      be = group_sumf<GW>(be);
      ga = group_sumf<GW>(ga);
      const float g2 = ga * ga, ab = al * be;
      // g2 > 0 here also keeps dd^2 + 4 g2 > 0 (alpha beta >= 0)
      const bool doit = g2 > 1e-14f * ab;
      const float dd = be - al;
      const float ri = __builtin_amdgcn_rsqf(fmaf(dd, dd, 4.f * g2));
      const float hc = fmaf(0.5f * fabsf(dd), ri, 0.5f);
      const float rh = __builtin_amdgcn_rsqf(hc);
      const float c = doit ? hc * rh : 1.f;
      const float sn = doit ? (dd >= 0.f ? ga : -ga) * ri * rh : 0.f;
#pragma unroll
      for (int i = 0; i < RL; ++i) {
        kp[GW * i] = c * xp[i] - sn * xq[i];
        kq[GW * i] = sn * xp[i] + c * xq[i];
      }
      big |= __builtin_amdgcn_ballot_w64(g2 > 1e-8f * ab);   // wave-uniform, kept in scalar registers
      pq = pq_next;
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

// mode 2 for l <= LM (LM <= 32), 16 lanes per pair: 16 ceil(l / 2) threads
// rounded up to whole waves.  The workgroup sums the P Gram partials of C
// (gram_sum_block), wave 0 factors H in fp64 and writes K = 2^-e R^T while
// wave 1 (wave 0 afterwards when it is alone) sums the |E|^2 and |W|^2
// partials of the objective.
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
  __shared__ uint32_t sched[31 * 16];
  __shared__ double norm2[32];
  __shared__ int order[32];
  __shared__ double kscale;
  __shared__ double objsums[2];
  const int tid = threadIdx.x;
  const int n = l + (l & 1);
  for (int e = tid; e < l * l; e += blockDim.x) Xs[e] = Xinv[e];
  build_schedule(sched, n, blockDim.x / 16, LD);
  const double* gram = gram_sum_block<LM>(gparts, P, l, gsum);
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
  const int sweeps = jacobi_columns<16, 2>(K, sched, n, 30);
  core_finish(K, LD, l, n, kscale, Xs, r, SB, SA, sigma, stats, obj, sweeps, norm2, order, objsums);
}

// ---------------------------------------------------------------------------
// The two solves for 32 < l <= kMaxL, by one workgroup of 640
// threads (pair i of a Jacobi round on lanes 16 i .. 16 i + 15).
//
// chol_wide: right-looking Cholesky of the fp64 Gram with the matrix in
// registers: wave w owns rows w, w + 10, ..., lane c owns columns c and c + 64,
// 16 entries per thread.  Step j: the owner of row j publishes it (and row j of
// T) through a double-buffered LDS row, one barrier, then every thread takes the
// pivot and updates its own entries with the outer product of row j.  Updates
// are unconditional: entries of finished rows and columns pick up values that
// are never read again.  R's rows go to Rm when given; with INV the same steps
// build X = R^-1 the way chol_wave does (T = R^-T, lane c holding its columns
// of T's rows), each finished row of T written straight into X's column.
constexpr int kWideLd = kMaxL + 1;
// measured on MI355X at l = 80: more lanes per pair and more waves win (4-lane
// pairs on 3 waves: 2.5x slower core; 4 Cholesky waves: 1.35x slower)
constexpr int kWideCholWaves = 10;   // waves of the l > 32 Cholesky workgroup
constexpr int kWideGroup = 16;       // lanes per Jacobi pair of the l > 32 core

template <bool INV, int NW>
__device__ void chol_wide(const double* __restrict__ gram, int l, double* Rm, float* __restrict__ X, double* rowbuf,
                          double* scratch) {
  constexpr int kWideWaves = NW, kWideRows = (kMaxL + NW - 1) / NW;
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63;
  double g[kWideRows][2], t[kWideRows][2];
#pragma unroll
  for (int i = 0; i < kWideRows; ++i)
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      const int a = w + kWideWaves * i, b = lane + 64 * c;
      const bool in = a < l && b < l;
      const int pi = !in ? 0 : (a <= b ? packed_index(a, b, l) : packed_index(b, a, l));
      const double v = gram[pi];
      g[i][c] = in ? v : 0.0;
      if (INV) t[i][c] = (a == b) ? 1.0 : 0.0;
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
  for (int j = 0; j < l; ++j) {
    double* rb = rowbuf + (j & 1) * 2 * kWideLd;   // [G row j | T row j]
    if (w == j % kWideWaves) {
      const int ij = j / kWideWaves;
#pragma unroll
      for (int i = 0; i < kWideRows; ++i)
        if (i == ij) {
#pragma unroll
          for (int c = 0; c < 2; ++c) {
            const int b = lane + 64 * c;
            if (b < kWideLd) {
              rb[b] = g[i][c];
              if (INV) rb[kWideLd + b] = t[i][c];
            }
          }
        }
    }
    __syncthreads();
    const double piv = rb[j];
    const bool keep = piv > tol && piv > 0.0;
    const double inv = keep ? rsq_f64(piv) : 0.0;   // 1 / R[j][j]
    double rjb[2], tjb[2];
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      const int b = lane + 64 * c;
      const int bb = b < kWideLd ? b : 0;
      rjb[c] = rb[bb] * inv;                        // R[j][b] (b > j)
      if (INV) tjb[c] = rb[kWideLd + bb] * inv;     // final T[j][b]
    }
    if (Rm != nullptr && w == 0) {
#pragma unroll
      for (int c = 0; c < 2; ++c) {
        const int b = lane + 64 * c;
        if (b >= j && b < l) Rm[j * kWideLd + b] = (b == j) ? piv * inv : rjb[c];
      }
    }
    if (INV && w == 0) {
#pragma unroll
      for (int c = 0; c < 2; ++c) {
        const int b = lane + 64 * c;
        if (b <= j) X[b * l + j] = static_cast<float>(tjb[c]);   // X = T^T
      }
    }
#pragma unroll
    for (int i = 0; i < kWideRows; ++i) {
      const int a = w + kWideWaves * i;
      const double rja = rb[a < kWideLd ? a : 0] * inv;   // R[j][a]
#pragma unroll
      for (int c = 0; c < 2; ++c) {
        g[i][c] = fma(-rja, rjb[c], g[i][c]);
        if (INV) t[i][c] = fma(-rja, tjb[c], t[i][c]);
      }
    }
  }
  __syncthreads();
}

// MODE 1: Cholesky and X = R^-1 on NW waves; MODE 2: the core, Jacobi pairs on
// GW-lane groups (NW = 40 GW / 64 rounded up).
template <int MODE, int NW, int GW>
__global__ __launch_bounds__(64 * NW) void solve_wide_kernel(const double* __restrict__ gram, int l,
                                                                  float* __restrict__ Xinv, int r,
                                                                  float* __restrict__ SB, float* __restrict__ SA,
                                                                  float* __restrict__ sigma, double* __restrict__ stats,
                                                                  ObjectiveArgs obj) {
  constexpr int NB = kMaxL * kWideLd;
  constexpr int NP = 64 * NW / GW;   // pair slots
  static_assert(2 * NP <= kMaxL, "the padding slots' zero columns lie inside K");
  __shared__ double Rm[MODE == 2 ? NB : 1];
  __shared__ float Kf[MODE == 2 ? NB : 1];
  __shared__ uint32_t sched[MODE == 2 ? (kMaxL - 1) * NP : 1];
  __shared__ double rowbuf[4 * kWideLd];
  __shared__ double norm2[kMaxL];
  __shared__ int order[kMaxL];
  __shared__ double scratch[2];
  const int tid = threadIdx.x, nt = blockDim.x;
  if (MODE == 1) {
    for (int e = tid; e < l * l; e += nt) Xinv[e] = 0.f;
    chol_wide<true, NW>(gram, l, nullptr, Xinv, rowbuf, scratch);
    return;
  }
  const int n = l + (l & 1);
  build_schedule(sched, n, NP, kWideLd);
  chol_wide<false, NW>(gram, l, Rm, nullptr, rowbuf, scratch);
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
  const int sweeps = jacobi_columns<GW, RL>(Kf, sched, n, 40);
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
                                                          float* __restrict__ out, double* __restrict__ gram_parts) {
  constexpr int LP = 16 * NT, PER = (kGramRows * LP + kReduceThreads - 1) / kReduceThreads, LDR = LP + 1;
  constexpr int NW = kReduceThreads / 64;
  static_assert(kGramRows % 16 == 0, "whole 16-row MFMA tiles");
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
  for (int idx = threadIdx.x; idx < kPanelRows * w; idx += blockDim.x) {
    int rr, c;
    if (transpose_out) { rr = idx % kPanelRows; c = idx / kPanelRows; }
    else { rr = idx / w; c = idx - rr * w; }
    float acc = 0.f;
    for (int a = 0; a < l; ++a) acc = fmaf(Ps[rr * ldp + a], Ss[a * w + c], acc);
    const int64_t row = r0 + rr;
    if (row < m) {
      if (transpose_out) out[static_cast<int64_t>(c) * m + row] = acc;
      else out[row * w + c] = acc;
    }
  }
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
  // Long-side factor: x_j / sqrt(sigma_j).  Short side: E-product with x_j times sigma_j^(-3/2).
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
  double s2 = 0.0;
  for (int c = 0; c < r; ++c) s2 += norm2[order[c]];
  if (tid == 0 && stats) {
    stats[0] = s2;
    stats[1] = sweeps;
  }
  write_objective(obj, s2);
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
                  double* gram_parts, hipStream_t s) {
  const int blocks = static_cast<int>(cdiv(m_pad, kGramRows));
  LQ_LAUNCH("reduce_gram", (reduce_gram_kernel<NT>), dim3(blocks), dim3(kReduceThreads), 0, s, part, S, m, m_pad, l, X, out,
            gram_parts);
}

void launch_reduce(int nt, const float* part, int S, int64_t m, int64_t m_pad, int l, const float* X, float* out,
                   double* gram_parts, hipStream_t s) {
  switch (nt) {
    case 1: reduce_typed<1>(part, S, m, m_pad, l, X, out, gram_parts, s); break;
    case 2: reduce_typed<2>(part, S, m, m_pad, l, X, out, gram_parts, s); break;
    case 3: reduce_typed<3>(part, S, m, m_pad, l, X, out, gram_parts, s); break;
    case 4: reduce_typed<4>(part, S, m, m_pad, l, X, out, gram_parts, s); break;
    default: reduce_typed<5>(part, S, m, m_pad, l, X, out, gram_parts, s); break;
  }
}

// mode 1 factors the summed Gram `gram`; mode 2 sums the P partials `gparts` itself.
template <int LM>
void small_wave_typed(int mode, const double* gram, const double* gparts, int P, int l, float* Xinv, int r, float* SB,
                      float* SA, float* sigma, double* stats, const ObjectiveArgs& obj, hipStream_t s) {
  if (mode == 1)
    LQ_LAUNCH("chol_inv", chol_inv_wave_kernel<LM>, dim3(1), dim3(64), 0, s, gram, l, Xinv);
  else
    LQ_LAUNCH("core_svd", core_small_kernel<LM>, dim3(1), dim3(static_cast<unsigned>(round_up(16 * ((l + 1) / 2), 64))), 0,
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
    p.l = static_cast<int>(n);
    p.off_x = take((n + 1) * (d > k ? d : k) * 8);
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
  const GemmShape nn = gemm_shape(false, p.nt), tn = gemm_shape(true, p.nt);
  p.nn_row_blocks = static_cast<int>(cdiv(d, nn.tile));
  p.nn_splits = choose(p.nn_row_blocks, k, nn.unit, 0, p.nn_kper);
  p.tn_col_blocks = static_cast<int>(cdiv(k, tn.tile));
  p.tn_splits = choose(p.tn_col_blocks, d, tn.unit, 0, p.tn_rper);
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
                       hipStream_t s) {
  const int64_t d = pl.d, k = pl.k;
  const int r = pl.r, l = pl.l;
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
  if (omega != nullptr) {
    LQ_LAUNCH("to_frag", to_frag_kernel, dim3(static_cast<unsigned>(cdiv(nfrag, 256))), dim3(256), 0, s, omega, k, l,
              pl.nt, pl.k_pad, Om_ws);
    Om = Om_ws;
  } else if (omega_frag == nullptr) {
    hipError_t e = run_sketch(seed, t, 1, k, l, pl.nt, pl.k_pad, Om_ws, s);
    if (e != hipSuccess) return e;
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
  const bool ride = pl.ride;
  bool pending = false;
  auto product = [&](bool transposed, const float* panel, int mode) {
    const CholJob job{pending ? gparts : nullptr, pl.gram_parts_d, l, Xinv};
    launch_gemm(transposed, E, d, k, panel, pl, part, job, s);
    if (transposed) pending = false;
    if (transposed)
      launch_reduce(pl.nt, part, pl.tn_splits, k, pl.k_pad, l, Xinv, Z, mode ? gparts : nullptr, s);
    else
      launch_reduce(pl.nt, part, pl.nn_splits, d, pl.d_pad, l, nullptr, Y, mode ? gparts : nullptr, s);
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
    LQ_LAUNCH("gram_sum", gram_sum_kernel, dim3((E_ + 63) / 64), dim3(1024), 0, s, gparts, P, E_, gtotal);
    if (l <= 32)
      launch_small_wave(1, gtotal, nullptr, 0, l, Xinv, r, SB, SA, sigma, stats, none, s);
    else if (mode == 1)
      LQ_LAUNCH("chol_inv", (solve_wide_kernel<1, kWideCholWaves, 16>), dim3(1), dim3(64 * kWideCholWaves), 0, s, gtotal,
                l, Xinv, r, SB, SA, sigma, stats, none);
    else
      LQ_LAUNCH("core_svd", (solve_wide_kernel<2, (40 * kWideGroup + 63) / 64, kWideGroup>), dim3(1),
                dim3(64 * ((40 * kWideGroup + 63) / 64)), 0, s, gtotal, l, Xinv, r, SB, SA, sigma, stats, obj);
  };
  // Y = E Omega; X = R^-1 of its Gram.  Each power iteration multiplies by E^T
  // and E and re-orthonormalises Y only: span(E Z) does not depend on Z's basis,
  // so orthonormalising Z as well would not change the subspace.
  product(false, Om, 1);
  for (int it = 0; it < q; ++it) {
    product(true, Y, 0);
    product(false, Z, 1);
  }
  // C = E^T Q = (E^T Y) X, then the core solve on C^T C
  product(true, Y, 2);
  panels(PanelJob{Y, d, SB, B, 0}, PanelJob{Z, k, SA, A, 1}, l, pl.nt, r, s);
  return hipGetLastError();
}

}  // namespace loftq
