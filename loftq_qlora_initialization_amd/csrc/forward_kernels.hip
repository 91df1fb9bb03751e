// QLoRA forward of one adapted layer on gfx950, the consumer of LoftQ's Q, B, A:
//   Y = X bf16(deq(Q))^T + alpha (X bf16(A)^T) bf16(B)^T
// ("参数高效微调：LoRA、Adapter 与 QLoRA" §2.2: the LoRA output adds to the frozen
// weight's, h = W x + B A x; §4.3: the 4-bit base computes in bfloat16).
// Tokens are rows: X n x cols (bf16), Y n x rows (fp32), W = deq(Q) rows x cols.
//
// lora_down_kernel   T = X bf16(A)^T (n x r, fp32) on bf16 MFMA (16x16x32) as up
//                    to 8 partial products over K ranges (16 tokens and one range
//                    per workgroup, the range split over its 16 waves); the GEMM
//                    kernels sum the partials of their tokens once, into LDS.
// nf4_gemm_kernel    more than 64 tokens: Y = X bf16(W)^T + alpha T bf16(B)^T, a
//                    256 or 128 (tokens) x 128 output tile per workgroup of 8 or 4
//                    waves (64 x 64 each, 4 x 4 MFMA tiles), K in steps of 64.  Each step the workgroup
//                    stages X (bf16) and the weight decoded from its codes (deq =
//                    fl32(c[code] a') exactly as in the dequantization, then rounded
//                    to bf16) in LDS, double buffered with one barrier per step,
//                    while the global loads of two steps ahead are in flight.  The
//                    epilogue adds the LoRA term in fp32.
// nf4_skinny_kernel  up to 64 tokens: bound by reading Q; decodes codes straight
//                    into matrix-core operands, K split over the workgroup's waves.
//
// v_mfma_f32_16x16x32_bf16: lane L supplies A[L%16][8(L/16) + j] and
// B[8(L/16) + j][L%16] (j = 0..7) and receives D[4(L/16) + v][L%16] in element v.
#include "internal.h"

namespace loftq {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float mfma_f4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kBN = 128, kBK = 64;   // tiled kernel: output features and K per step
// X A^T is formed as up to kMaxSplits partial products over K ranges.
constexpr int kMaxSplits = 8;

// The sum of the ks (1 <= ks <= kMaxSplits) partials p[0], p[stride], ... added in the
// order q = 0, 1, ..., with every load issued before the first add (a load-add chain
// would wait a full memory latency per partial): the loads are unconditional, those
// past ks repeating partial ks - 1, and their values are dropped.
__device__ __forceinline__ float sum_partials(const float* __restrict__ p, int64_t stride, int ks) {
  float v[kMaxSplits];
#pragma unroll
  for (int q = 0; q < kMaxSplits; ++q) v[q] = p[(q < ks ? q : ks - 1) * stride];
  float t = 0.f;
#pragma unroll
  for (int q = 0; q < kMaxSplits; ++q)
    if (q < ks) t += v[q];
  return t;
}

typedef float f32x2 __attribute__((ext_vector_type(2)));

// Byte-pair decode: a byte holds two codes (element 2j in the high nibble), and all
// codes a thread decodes in one go share one block scale, so a 256-entry LDS table
// of level pairs (c[b >> 4], c[b & 15]) serves two elements per lookup.  Each value
// is still fl32(c[code] a') rounded to bf16 (nearest even), as the dequantization.
__device__ __forceinline__ void fill_level_pairs(f32x2* lvl2, const Nf4Tables& tab, int tid, int nthreads) {
  for (int i = tid; i < 256; i += nthreads) lvl2[i] = f32x2{tab.level[i >> 4], tab.level[i & 15]};
}
__device__ __forceinline__ bf16x8 decode8(const f32x2* lvl2, uint32_t word, float sc) {
  bf16x8 o;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const f32x2 c = lvl2[(word >> (8 * j)) & 0xFFu];
    o[2 * j] = static_cast<__bf16>(c.x * sc);
    o[2 * j + 1] = static_cast<__bf16>(c.y * sc);
  }
  return o;
}

// Workgroups are dealt to the 8 XCDs round-robin by id.  Tile t = xcd * per + slot
// gives each XCD a contiguous run of tiles (token tile outer, feature tile inner),
// so the activations of its token tiles stay in that XCD's L2; ids past the last
// full round keep their own index.
__device__ __forceinline__ int64_t xcd_tile(int64_t wg, int64_t total) {
  const int64_t per = total / 8;
  return wg < per * 8 ? (wg % 8) * per + wg / 8 : wg;
}

// Epilogue of the tiled kernels (kBM token rows, kThreads threads, waves of 64 x 64).
// Element v of tile (mt, nt) is token m = .. + 4 lg + v, feature n = .. + li.  The
// LoRA operands go to LDS over the idle tile buffers, rows padded to r + 1 floats:
// the tile's rows of X A^T (Ts, the sum of the ks K-split partials in split order)
// and bf16(B) of its kBN features (Bs), with the loads of eight elements per thread
// in flight at once.  The LoRA term T bf16(B)^T of a 16 x 16 tile is one fp32 MFMA
// (16x16x4) per 4 of r: lane L supplies T[m0 + L%16][p0 + L/16] and
// bf16(B)[n0 + L%16][p0 + L/16].
template <int kBM, int kThreads>
__device__ __forceinline__ void tile_epilogue(float* Ts, mfma_f4 (&acc)[4][4], int tid, int wm, int wn, int li,
                                              int lg, int64_t m0, int64_t n0, int64_t M, int64_t N,
                                              const float* __restrict__ T, int ks, const float* __restrict__ B,
                                              int r, float alpha, float* __restrict__ Y) {
  const int rp = r + 1;
  float* Bs = Ts + kBM * rp;
  if (T != nullptr) {
    __syncthreads();
    for (int base = 0; base < kBM * r; base += 8 * kThreads) {
      float v[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int idx = base + e * kThreads + tid, i = idx / r, p = idx - i * r;
        const bool ok = idx < kBM * r && m0 + i < M;
        const float t = sum_partials(T + (ok ? (m0 + i) * r + p : 0), M * r, ks);
        v[e] = ok ? t : 0.f;
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int idx = base + e * kThreads + tid, i = idx / r, p = idx - i * r;
        if (idx < kBM * r) Ts[i * rp + p] = v[e];
      }
    }
    for (int base = 0; base < kBN * r; base += 8 * kThreads) {
      float v[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int idx = base + e * kThreads + tid, i = idx / r, p = idx - i * r;
        const bool ok = idx < kBN * r && n0 + i < N;
        const float b = B[ok ? (n0 + i) * r + p : 0];
        v[e] = ok ? static_cast<float>(static_cast<__bf16>(b)) : 0.f;
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int idx = base + e * kThreads + tid, i = idx / r, p = idx - i * r;
        if (idx < kBN * r) Bs[i * rp + p] = v[e];
      }
    }
    __syncthreads();
  }
  const int64_t mw = m0 + wm * 64, nw = n0 + wn * 64;
#pragma unroll
  for (int mt = 0; mt < 4; ++mt) {
    mfma_f4 lora[4];
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) lora[nt] = mfma_f4{0.f, 0.f, 0.f, 0.f};
    if (T != nullptr) {
      const int tl = wm * 64 + mt * 16 + li;
      for (int p0 = 0; p0 < r; p0 += 4) {
        const int p = p0 + lg;
        const float tv = p < r ? Ts[tl * rp + p] : 0.f;
#pragma unroll
        for (int nt = 0; nt < 4; ++nt) {
          const float bv = p < r ? Bs[(wn * 64 + nt * 16 + li) * rp + p] : 0.f;
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

template <bool kDQ, int kBM>
__global__ __launch_bounds__(2 * kBM, kBM == 128 ? 2 : 1) void nf4_gemm_kernel(const __bf16* __restrict__ X, int64_t M, int64_t N,
                                                       int64_t K, const uint8_t* __restrict__ packed,
                                                       const float* __restrict__ absmax,
                                                       const int8_t* __restrict__ qa,
                                                       const float* __restrict__ dqs,
                                                       const float* __restrict__ T, int ks,
                                                       const float* __restrict__ B, int r, float alpha,
                                                       float* __restrict__ Y, Nf4Tables tab) {
  constexpr int kThreads = 2 * kBM;      // kBM / 64 x 2 waves, 64 x 64 outputs each
  constexpr int kWM = kBM / 64;
  // padded rows against bank conflicts: +16 bf16 (40-dword rows) measured fewer conflicts than +8 for
  // 256-token tiles; 128-token tiles keep +8 so that two workgroups fit a CU's LDS
  constexpr int kLdsRow = kBK + (kBM == 256 ? 16 : 8);
  constexpr int XPT = kBM * kBK / kThreads;   // X elements per thread and step (32)
  constexpr int WPT = kBN * kBK / kThreads;   // weight codes per thread and step (32 or 16)
  typedef uint32_t WcT __attribute__((ext_vector_type(WPT / 8)));
  // double-buffered X and W tiles in one array (the epilogue reuses all of it)
  __shared__ __align__(16) __bf16 lds[2 * (kBM + kBN) * kLdsRow];
  __bf16(*Xs)[kBM][kLdsRow] = reinterpret_cast<__bf16(*)[kBM][kLdsRow]>(lds);
  __bf16(*Ws)[kBN][kLdsRow] = reinterpret_cast<__bf16(*)[kBN][kLdsRow]>(lds + 2 * kBM * kLdsRow);
  __shared__ f32x2 lvl2[256];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, wm = w % kWM, wn = w / kWM;
  const int li = lane & 15, lg = lane >> 4;
  fill_level_pairs(lvl2, tab, tid, kThreads);
  const int64_t ntn = (N + kBN - 1) / kBN, ntm = (M + kBM - 1) / kBM;
  const int64_t tile = xcd_tile(blockIdx.x, ntn * ntm);
  const int64_t m0 = (tile / ntn) * kBM, n0 = (tile % ntn) * kBN;
  // this thread's share of one step: XPT elements of X row xrow and WPT codes of weight
  // row wrow (inside one 64-element scale block, since K % 64 = 0)
  const int xrow = tid / (kBK / XPT), xcol = (tid % (kBK / XPT)) * XPT;
  const int wrow = tid / (kBK / WPT), wcol = (tid % (kBK / WPT)) * WPT;
  const int64_t xr = (m0 + xrow < M) ? m0 + xrow : M - 1;   // clamped rows: loaded, never stored
  const int64_t wr = (n0 + wrow < N) ? n0 + wrow : N - 1;
  const u32x4* xsrc = reinterpret_cast<const u32x4*>(X + xr * K + xcol);
  const int64_t we0 = wr * K + wcol;                        // element index of this thread's codes
  // one step's global data in registers; two of them keep the loads of step kt + 2
  // in flight while step kt computes and step kt + 1 goes from registers to LDS
  struct Stage {
    u32x4 x[XPT / 8];
    WcT wc;
    float sc;
  };
  auto load = [&](Stage& st, int kt) __attribute__((always_inline)) {
    const int64_t k0 = static_cast<int64_t>(kt) * kBK;
#pragma unroll
    for (int q = 0; q < XPT / 8; ++q) st.x[q] = xsrc[k0 / 8 + q];
    const int64_t e = we0 + k0;
    st.wc = *reinterpret_cast<const WcT*>(packed + (e >> 1));
    const int64_t b = e >> 6;
    st.sc = kDQ ? static_cast<float>(qa[b]) * dqs[b >> 8] : absmax[b];
  };
  auto store = [&](const Stage& st, int buf) __attribute__((always_inline)) {
    u32x4* xd = reinterpret_cast<u32x4*>(&Xs[buf][xrow][xcol]);
#pragma unroll
    for (int q = 0; q < XPT / 8; ++q) xd[q] = st.x[q];
    bf16x8* wd = reinterpret_cast<bf16x8*>(&Ws[buf][wrow][wcol]);
#pragma unroll
    for (int q = 0; q < WPT / 8; ++q) wd[q] = decode8(lvl2, st.wc[q], st.sc);
  };
  mfma_f4 acc[4][4];
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int b = 0; b < 4; ++b) acc[a][b] = mfma_f4{0.f, 0.f, 0.f, 0.f};
  auto compute = [&](int buf) __attribute__((always_inline)) {
#pragma unroll
    for (int kk = 0; kk < kBK; kk += 32) {
      bf16x8 af[4], bfr[4];
#pragma unroll
      for (int mt = 0; mt < 4; ++mt)
        af[mt] = *reinterpret_cast<const bf16x8*>(&Xs[buf][wm * 64 + mt * 16 + li][kk + 8 * lg]);
#pragma unroll
      for (int nt = 0; nt < 4; ++nt)
        bfr[nt] = *reinterpret_cast<const bf16x8*>(&Ws[buf][wn * 64 + nt * 16 + li][kk + 8 * lg]);
#pragma unroll
      for (int mt = 0; mt < 4; ++mt)
#pragma unroll
        for (int nt = 0; nt < 4; ++nt)
          acc[mt][nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[mt], bfr[nt], acc[mt][nt], 0, 0, 0);
    }
  };
  const int KT = static_cast<int>(K / kBK);
  Stage s0, s1;
  __syncthreads();   // level pairs
  load(s0, 0);
  load(s1, KT > 1 ? 1 : 0);
  store(s0, 0);
  __syncthreads();
  // Even steps read LDS buffer 0, odd steps buffer 1.  Each half of the loop is one
  // basic block (loads of two steps ahead, this step's products, the decode and
  // store of the next step), so the decode can issue between the matrix ops; past
  // the last step the loads repeat step KT - 1 and the store fills the idle buffer.
  int kt = 0;
  for (; kt + 1 < KT; kt += 2) {
    load(s0, kt + 2 < KT ? kt + 2 : KT - 1);
    compute(0);
    store(s1, 1);
    __syncthreads();
    load(s1, kt + 3 < KT ? kt + 3 : KT - 1);
    compute(1);
    store(s0, 0);
    __syncthreads();
  }
  if (kt < KT) compute(0);   // odd step count: the last step sits in buffer 0
  static_assert(sizeof(lds) >= (kBM + kBN) * 65 * sizeof(float), "the LoRA operands (r <= 64) reuse the tile buffers");
  tile_epilogue<kBM, kThreads>(reinterpret_cast<float*>(lds), acc, tid, wm, wn, li, lg, m0, n0, M, N, T, ks, B, r,
                               alpha, Y);
}

// Partial products P_q = X bf16(A)^T over the q-th of ks K ranges, for TT 16-token
// tiles per workgroup (workgroup = group * ks + q); P_q lands at T + q n r.  The 16
// waves split the range (wave w takes its 32-wide steps w, w + 16, ...); each step's
// A operand serves all TT tiles.  The waves' partial products are summed through LDS
// in a fixed order.  Consumers add the ks partials in order q = 0, 1, ...
template <int NT, int U, int TT>
__global__ __launch_bounds__(1024) void lora_down_kernel(const __bf16* __restrict__ X, int64_t M, int64_t K,
                                                         const float* __restrict__ A, int r, int ks,
                                                         float* __restrict__ T) {
  constexpr int kOut = TT * NT * 256;   // accumulator floats per wave
  __shared__ float part[8][kOut];
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, li = lane & 15, lg = lane >> 4;
  const int64_t group = blockIdx.x / ks;
  const int q = static_cast<int>(blockIdx.x - group * ks);
  const int64_t m0 = group * 16 * TT;
  int64_t xr[TT];
#pragma unroll
  for (int tt = 0; tt < TT; ++tt) xr[tt] = (m0 + 16 * tt + li < M) ? m0 + 16 * tt + li : M - 1;
  mfma_f4 acc[TT][NT];
#pragma unroll
  for (int tt = 0; tt < TT; ++tt)
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) acc[tt][nt] = mfma_f4{0.f, 0.f, 0.f, 0.f};
  // wave w takes the steps w, w + 16, ... of the range, U of them per round (U covers
  // a wave's share of the range when registers allow) with all their loads issued
  // before the first product (rows p >= r load row r - 1 and are zeroed)
  const int KT = static_cast<int>(K / 32);
  const int per = (KT + ks - 1) / ks;
  const int k_begin = q * per, k_end = k_begin + per < KT ? k_begin + per : KT;
  for (int base = k_begin + w; base < k_end; base += 16 * U) {
    bf16x8 a[U][TT];
    float4 ua[U][NT], ub[U][NT];
#pragma unroll
    for (int i = 0; i < U; ++i) {
      const int kt = base + 16 * i < KT ? base + 16 * i : KT - 1;
      const int64_t k0 = static_cast<int64_t>(kt) * 32 + 8 * lg;
#pragma unroll
      for (int tt = 0; tt < TT; ++tt) a[i][tt] = *reinterpret_cast<const bf16x8*>(X + xr[tt] * K + k0);
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        const int p = nt * 16 + li < r ? nt * 16 + li : r - 1;
        const float4* src = reinterpret_cast<const float4*>(A + static_cast<int64_t>(p) * K + k0);
        ua[i][nt] = src[0];
        ub[i][nt] = src[1];
      }
    }
    __builtin_amdgcn_sched_barrier(0);   // every load of the round is in flight before the first wait
#pragma unroll
    for (int i = 0; i < U; ++i) {
      // steps past the range (clamped loads) and rows p >= r contribute exact zeros
      const bool live = base + 16 * i < k_end;
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        const float z = (live && nt * 16 + li < r) ? 1.f : 0.f;
        const float4 u = ua[i][nt], v4 = ub[i][nt];
        bf16x8 b;
        b[0] = static_cast<__bf16>(u.x * z); b[1] = static_cast<__bf16>(u.y * z);
        b[2] = static_cast<__bf16>(u.z * z); b[3] = static_cast<__bf16>(u.w * z);
        b[4] = static_cast<__bf16>(v4.x * z); b[5] = static_cast<__bf16>(v4.y * z);
        b[6] = static_cast<__bf16>(v4.z * z); b[7] = static_cast<__bf16>(v4.w * z);
#pragma unroll
        for (int tt = 0; tt < TT; ++tt) {
          const bf16x8 ai = live ? a[i][tt] : bf16x8{};
          acc[tt][nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ai, b, acc[tt][nt], 0, 0, 0);
        }
      }
    }
  }
  // waves 8..15 park their partials, waves 0..7 add theirs, then one thread per
  // element sums the 8 pair sums in wave order; element ((tt NT + nt) 4 + v) 64 + lane
  if (w >= 8) {
#pragma unroll
    for (int tt = 0; tt < TT; ++tt)
#pragma unroll
      for (int nt = 0; nt < NT; ++nt)
#pragma unroll
        for (int v = 0; v < 4; ++v) part[w - 8][((tt * NT + nt) * 4 + v) * 64 + lane] = acc[tt][nt][v];
  }
  __syncthreads();
  if (w < 8) {
#pragma unroll
    for (int tt = 0; tt < TT; ++tt)
#pragma unroll
      for (int nt = 0; nt < NT; ++nt)
#pragma unroll
        for (int v = 0; v < 4; ++v) part[w][((tt * NT + nt) * 4 + v) * 64 + lane] += acc[tt][nt][v];
  }
  __syncthreads();
  for (int e = threadIdx.x; e < kOut; e += 1024) {
    float sum = 0.f;
#pragma unroll
    for (int qq = 0; qq < 8; ++qq) sum += part[qq][e];
    const int ln = e & 63, v = (e >> 6) & 3, tn = e >> 8, tt = tn / NT, nt = tn - tt * NT;
    const int64_t m = m0 + 16 * tt + 4 * (ln >> 4) + v;
    const int p = nt * 16 + (ln & 15);
    if (m < M && p < r) T[(q * M + m) * r + p] = sum;
  }
}

// Few tokens (<= 64): the product is bound by reading Q, so each workgroup owns 16
// output features and every token, and its NW waves split K in 128-wide chunks
// (wave w takes chunks w, w + NW, ...; NW = 16, or 8 for 3-4 token tiles, whose
// operands need more registers).  Lane L decodes the 32 codes of feature
// n0 + L%16 at k = 128 c + 32 (L/16) .. + 31 (one 16-byte load, one block scale)
// straight into matrix-core operands: MFMA s (0..3) of a chunk contracts the k
// 128 c + 32 g + 8 s + j of lane group g, and the token operand is loaded at the
// same k, so each chunk covers its 128 k exactly once.  Partial sums meet in LDS in
// a fixed order, then the LoRA term is added in fp32.
template <int NTT, int NW, int U, bool kDQ>
__global__ __launch_bounds__(NW * 64) void nf4_skinny_kernel(const __bf16* __restrict__ X, int64_t M, int64_t N,
                                                          int64_t K, const uint8_t* __restrict__ packed,
                                                          const float* __restrict__ absmax,
                                                          const int8_t* __restrict__ qa,
                                                          const float* __restrict__ dqs,
                                                          const float* __restrict__ T, int ks,
                                                          const float* __restrict__ B, int r, float alpha,
                                                          float* __restrict__ Y, Nf4Tables tab) {
  __shared__ float part[NW / 2][NTT * 256];
  __shared__ float Ts[NTT * 16 * 64];   // the tokens' rows of X A^T, r <= 64
  __shared__ float Bs[16 * 64];         // bf16(B) of the workgroup's 16 features
  __shared__ f32x2 lvl2[256];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, li = lane & 15, lg = lane >> 4;
  const int64_t n0 = static_cast<int64_t>(blockIdx.x) * 16;
  fill_level_pairs(lvl2, tab, tid, NW * 64);
  // the epilogue's LoRA operands, staged first so their loads overlap the main loop:
  // X A^T of every token (the ks K-split partials summed in order) and bf16(B)
  if (T != nullptr) {
    for (int idx = tid; idx < M * r; idx += NW * 64) Ts[idx] = sum_partials(T + idx, M * r, ks);
    for (int idx = tid; idx < 16 * r; idx += NW * 64) {
      const int64_t n = n0 + idx / r < N ? n0 + idx / r : N - 1;
      Bs[idx] = static_cast<float>(static_cast<__bf16>(B[n * r + idx % r]));
    }
  }
  __syncthreads();
  const int64_t wr = (n0 + li < N) ? n0 + li : N - 1;
  int64_t xr[NTT];
#pragma unroll
  for (int t = 0; t < NTT; ++t) xr[t] = (t * 16 + li < M) ? t * 16 + li : M - 1;
  mfma_f4 acc[NTT];
#pragma unroll
  for (int t = 0; t < NTT; ++t) acc[t] = mfma_f4{0.f, 0.f, 0.f, 0.f};
  // U chunks per round (w + NW i, i < U) with every load issued before the first
  // product; chunks past the end and lane groups past K (a 64-wide tail chunk) load
  // a valid address and are zeroed: scale 0 for the weight, a select for the tokens
  const int KC = static_cast<int>((K + 127) / 128);
  for (int c0 = w; c0 < KC; c0 += NW * U) {
    u32x4 code[U];
    float sc[U];
    u32x4 xv[U][NTT][4];
#pragma unroll
    for (int i = 0; i < U; ++i) {
      const int c = c0 + NW * i < KC ? c0 + NW * i : KC - 1;
      int64_t k = static_cast<int64_t>(c) * 128 + 32 * lg;
      const bool live = c0 + NW * i < KC && k < K;
      if (!live) k = K - 32;
      const int64_t e = wr * K + k;
      code[i] = *reinterpret_cast<const u32x4*>(packed + (e >> 1));
      const int64_t b = e >> 6;
      const float a = kDQ ? static_cast<float>(qa[b]) * dqs[b >> 8] : absmax[b];
      sc[i] = live ? a : 0.f;
#pragma unroll
      for (int t = 0; t < NTT; ++t)
#pragma unroll
        for (int s4 = 0; s4 < 4; ++s4) {
          const u32x4 v = *reinterpret_cast<const u32x4*>(X + xr[t] * K + k + 8 * s4);
          xv[i][t][s4] = live ? v : u32x4{0u, 0u, 0u, 0u};
        }
    }
    __builtin_amdgcn_sched_barrier(0);   // every load of the round is in flight before the first wait
#pragma unroll
    for (int i = 0; i < U; ++i) {
      bf16x8 wf[4];
#pragma unroll
      for (int s4 = 0; s4 < 4; ++s4) wf[s4] = decode8(lvl2, code[i][s4], sc[i]);
#pragma unroll
      for (int s4 = 0; s4 < 4; ++s4)
#pragma unroll
        for (int t = 0; t < NTT; ++t)
          acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, xv[i][t][s4]), wf[s4], acc[t],
                                                           0, 0, 0);
    }
  }
  if (w >= NW / 2) {
#pragma unroll
    for (int t = 0; t < NTT; ++t)
#pragma unroll
      for (int v = 0; v < 4; ++v) part[w - NW / 2][(t * 4 + v) * 64 + lane] = acc[t][v];
  }
  __syncthreads();
  if (w < NW / 2) {
#pragma unroll
    for (int t = 0; t < NTT; ++t)
#pragma unroll
      for (int v = 0; v < 4; ++v) part[w][(t * 4 + v) * 64 + lane] += acc[t][v];
  }
  __syncthreads();
  // element (t, v, lane): token t*16 + 4 (lane/16) + v, feature n0 + lane%16
  for (int e = tid; e < NTT * 256; e += NW * 64) {
    const int ln = e & 63, v = (e >> 6) & 3, t = e >> 8;
    const int64_t m = t * 16 + 4 * (ln >> 4) + v, n = n0 + (ln & 15);
    if (m >= M || n >= N) continue;
    float y = 0.f;
#pragma unroll
    for (int q = 0; q < NW / 2; ++q) y += part[q][e];
    if (T != nullptr) {
      float lora = 0.f;
      for (int p = 0; p < r; ++p)
        lora = fmaf(Ts[m * r + p], Bs[(ln & 15) * r + p], lora);
      y = fmaf(alpha, lora, y);
    }
    Y[m * N + n] = y;
  }
}

}  // namespace

// Token rows per tiled-kernel workgroup: 256 (8 waves) halves the weight decode per
// product and measured 12 % faster at 2048 x 4096 outputs; it is taken while its
// tiles still give every CU a workgroup, else 128 (4 waves).
constexpr int kCUs = 256;

size_t qlora_forward_workspace_bytes(int64_t n_tok, int r) {
  return static_cast<size_t>((kMaxSplits * n_tok * r * 4 + 255) / 256 * 256);
}

// Launch shapes of one forward call (shared by the launcher and the argument check).
struct ForwardPlan {
  int64_t tiles;     // 16-token tiles
  int tt;            // LoRA down: tiles per workgroup (4 for r <= 16 and many tokens: A is read once per 4)
  int ks;            // LoRA down: K ranges
  bool skinny;       // <= 64 tokens: few-token kernel
  int ntt;           // its 16-token tiles
  int bm;            // tiled kernel: tokens per workgroup
  int64_t grid_down, grid_gemm;
  int block_gemm;
};

ForwardPlan plan_forward(int64_t n_tok, int64_t rows, int64_t cols, int r) {
  ForwardPlan p{};
  p.tiles = (n_tok + 15) / 16;
  p.tt = (r <= 16 && p.tiles >= 64) ? 4 : 1;
  const int64_t groups = (p.tiles + p.tt - 1) / p.tt;
  // enough workgroups to spread the reads of A and X (about 512, or 256 with four
  // tiles each), each with at least 16 of the 32-wide K steps
  const int64_t target = p.tt == 4 ? 256 : 512;
  const int64_t kt = cols / 32;
  int64_t ks = (target + groups - 1) / groups;
  if (ks > kt / 16) ks = kt / 16;
  if (ks > kMaxSplits) ks = kMaxSplits;
  p.ks = ks < 1 ? 1 : static_cast<int>(ks);
  p.grid_down = groups * p.ks;
  p.skinny = n_tok <= 64;
  p.ntt = static_cast<int>((n_tok + 15) / 16);
  if (p.skinny) {
    p.grid_gemm = (rows + 15) / 16;
    p.block_gemm = p.ntt <= 2 ? 1024 : 512;
  } else {
    const int64_t ntn = (rows + kBN - 1) / kBN;
    p.bm = ntn * ((n_tok + 255) / 256) >= kCUs ? 256 : 128;
    p.grid_gemm = ntn * ((n_tok + p.bm - 1) / p.bm);
    p.block_gemm = 2 * p.bm;
  }
  return p;
}

bool qlora_forward_shape_ok(int64_t n_tok, int64_t rows, int64_t cols, int r) {
  if (n_tok <= 0 || rows <= 0) return true;   // nothing is launched
  const ForwardPlan p = plan_forward(n_tok, rows, cols, r);
  const int64_t limit = int64_t(1) << 32;        // work-items of one launch
  return p.grid_down * 1024 < limit && p.grid_gemm * p.block_gemm < limit;
}

hipError_t launch_qlora_forward(const void* X, int64_t n_tok, int64_t rows, int64_t cols, const uint8_t* packed,
                                const float* absmax, const int8_t* qa, const float* dqs, int bits, const float* B,
                                const float* A, int r, float alpha, float* Y, float* Tws, hipStream_t s) {
  if (n_tok == 0 || rows == 0) return hipSuccess;
  if (cols % 64 != 0 || cols == 0 || !qlora_forward_shape_ok(n_tok, rows, cols, r)) return hipErrorInvalidValue;
  const __bf16* Xb = static_cast<const __bf16*>(X);
  const ForwardPlan pl = plan_forward(n_tok, rows, cols, r);
  const int ks = pl.ks;
  if (B != nullptr) {
    const dim3 grid(static_cast<unsigned>(pl.grid_down));
    // steps per wave in one K range, rounded up to a power of two, capped by registers
    // (1024-thread workgroups: at most 128 VGPRs)
    const int64_t per = ((cols / 32) + ks - 1) / ks;
    const int64_t spw = (per + 15) / 16;
    const int nt = (r + 15) / 16;
    const int umax = pl.tt == 4 ? 2 : (nt == 1 ? 8 : (nt == 2 ? 4 : 2));
    int u = spw <= 1 ? 1 : spw <= 2 ? 2 : spw <= 4 ? 4 : 8;
    if (u > umax) u = umax;
#define LQ_DOWN(NT, U, TT)                                                                                 \
  LQ_LAUNCH("lora_down", (lora_down_kernel<NT, U, TT>), grid, dim3(1024), 0, s, Xb, n_tok, cols, A, r, ks, \
            Tws)
    if (pl.tt == 4) {
      if (u == 1) LQ_DOWN(1, 1, 4);
      else LQ_DOWN(1, 2, 4);
    } else {
      switch (nt * 16 + u) {
        case 16 + 1: LQ_DOWN(1, 1, 1); break;
        case 16 + 2: LQ_DOWN(1, 2, 1); break;
        case 16 + 4: LQ_DOWN(1, 4, 1); break;
        case 16 + 8: LQ_DOWN(1, 8, 1); break;
        case 32 + 1: LQ_DOWN(2, 1, 1); break;
        case 32 + 2: LQ_DOWN(2, 2, 1); break;
        case 32 + 4: LQ_DOWN(2, 4, 1); break;
        case 48 + 1: LQ_DOWN(3, 1, 1); break;
        case 48 + 2: LQ_DOWN(3, 2, 1); break;
        case 64 + 1: LQ_DOWN(4, 1, 1); break;
        default: LQ_DOWN(4, 2, 1); break;
      }
    }
#undef LQ_DOWN
  }
  const Nf4Tables& tab = nf_tables(bits);
  const float* T = B != nullptr ? Tws : nullptr;
  const dim3 grid(static_cast<unsigned>(pl.grid_gemm));
  const bool dq = qa != nullptr;
  if (pl.skinny) {
// 16 waves with two chunks each per round (1-2 token tiles; 8 waves x 4 chunks and 4 x 4
// measured slower), 8 waves with one chunk for 3-4 token tiles (registers)
#define LQ_SKINNY(NTT, DQ)                                                                                    \
  LQ_LAUNCH("nf4_gemm_skinny", (nf4_skinny_kernel<NTT, (NTT <= 2 ? 16 : 8), (NTT <= 2 ? 2 : 1), DQ>), grid,      \
            dim3(NTT <= 2 ? 1024 : 512), 0, s, Xb, n_tok, rows, cols, packed, absmax, qa, dqs, T, ks, B, r, alpha, Y, \
            tab)
    switch (pl.ntt * 2 + (dq ? 1 : 0)) {
      case 2: LQ_SKINNY(1, false); break;
      case 3: LQ_SKINNY(1, true); break;
      case 4: LQ_SKINNY(2, false); break;
      case 5: LQ_SKINNY(2, true); break;
      case 6: LQ_SKINNY(3, false); break;
      case 7: LQ_SKINNY(3, true); break;
      case 8: LQ_SKINNY(4, false); break;
      default: LQ_SKINNY(4, true); break;
    }
#undef LQ_SKINNY
    return hipGetLastError();
  }
#define LQ_TILED(BM, DQ)                                                                                        \
  LQ_LAUNCH("nf4_gemm", (nf4_gemm_kernel<DQ, BM>), grid, dim3(2 * BM), 0, s, Xb, n_tok, rows, cols, packed, absmax, \
            qa, dqs, T, ks, B, r, alpha, Y, tab)
  if (dq) {
    if (pl.bm == 256) LQ_TILED(256, true);
    else LQ_TILED(128, true);
  } else {
    if (pl.bm == 256) LQ_TILED(256, false);
    else LQ_TILED(128, false);
  }
#undef LQ_TILED
  return hipGetLastError();
}

}  // namespace loftq
