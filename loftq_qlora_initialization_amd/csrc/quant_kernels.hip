// NF4 quantize (optionally fused with the residual W - B A), double quant and
// dequant(-subtract) kernels for gfx950.
//
// Work unit: a "group" of 16 consecutive elements of the row-major flattening,
// four groups per 64-element absmax block.  The four lanes of a DPP quad hold one
// block, so the block absmax takes two quad_perm exchanges and no LDS.  A group
// is two 16-byte loads for bf16 (four for fp32) and one 8-byte store of packed
// nibbles, so every wave moves contiguous 2 KB (bf16) in and 512 B out.
//
// Encoding: y = fma(R, 16 rcp(a), 16), cell g = int(y) of a 33-cell grid held
// in LDS, code = base[g] + (y > thr16[g]) with thr16 = fl32(16 thr + 16).  y can
// differ from 16 fl32(R / a) + 16 by far less than the 2^-16 window, so any
// element whose y lies within the window of its cell's threshold is redone
// with an IEEE division and a full threshold count.  Codes are therefore
// bit-identical to fl32(R / a) rounding.
#include <float.h>

#include "internal.h"
#include "reduce.h"
#include "split_bf16.h"

namespace loftq {
namespace {

constexpr int kThreads = 256;

__device__ __forceinline__ float quad_xor1(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0xB1, 0xF, 0xF, false));
}
__device__ __forceinline__ float quad_xor2(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x4E, 0xF, 0xF, false));
}
__device__ __forceinline__ float quad_max(float v) {
  v = fmaxf(v, quad_xor1(v));
  return fmaxf(v, quad_xor2(v));
}

__device__ __forceinline__ void load16(const uint16_t* __restrict__ p, float v[16]) {
  const uint4 a = *reinterpret_cast<const uint4*>(p);
  const uint4 b = *reinterpret_cast<const uint4*>(p + 8);
  const uint32_t w[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    v[2 * i] = __uint_as_float(w[i] << 16);
    v[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
  }
}
__device__ __forceinline__ void load16(const float* __restrict__ p, float v[16]) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float4 q = reinterpret_cast<const float4*>(p)[i];
    v[4 * i] = q.x; v[4 * i + 1] = q.y; v[4 * i + 2] = q.z; v[4 * i + 3] = q.w;
  }
}
__device__ __forceinline__ float load1(const uint16_t* p, int64_t i) {
  return __uint_as_float(static_cast<uint32_t>(p[i]) << 16);
}
__device__ __forceinline__ float load1(const float* p, int64_t i) { return p[i]; }

struct EncodeLds {
  float2 cell[33];  // (fl32(16 threshold + origin), base code as int bits); +inf where the cell has none
  float thr[15];
  float level[16];
  float origin;     // y = 16 x + origin picks the cell (16 for NF4)
};

__device__ __forceinline__ void fill_lds(EncodeLds& s, const Nf4Tables& t) {
  const int tid = threadIdx.x;
  if (tid < 33) s.cell[tid] = make_float2(t.cell_thr16[tid], __int_as_float(t.cell_base[tid]));
  if (tid < 15) s.thr[tid] = t.thr[tid];
  if (tid < 16) s.level[tid] = t.level[tid];
  if (tid == 0) s.origin = t.cell_origin;
}

// Exact reference decision for one value: count of thresholds strictly below x.
__device__ __forceinline__ uint32_t exact_code(float r, float a, const EncodeLds& s) {
  const float x = (a > 0.f) ? r / a : 0.f;
  uint32_t c = 0;
#pragma unroll
  for (int j = 0; j < 15; ++j) c += (x > s.thr[j]) ? 1u : 0u;
  return c;
}

__device__ __forceinline__ int nib_shift(int e) { return 8 * ((e >> 1) & 3) + ((e & 1) ? 0 : 4); }

// A byte of packed codes holds two elements (element 2i in the high nibble), so the
// decoders look up level pairs (c[b >> 4], c[b & 15]) by whole bytes: one LDS read
// per two elements, each then multiplied by the block scale as before.
typedef float lvpair __attribute__((ext_vector_type(2)));
__device__ __forceinline__ void fill_level_pairs(lvpair* lvl2, const Nf4Tables& tab, int tid, int nthreads) {
  for (int i = tid; i < 256; i += nthreads) lvl2[i] = lvpair{tab.level[i >> 4], tab.level[i & 15]};
}

// Encode 16 residual values sharing absmax a into two packed 32-bit words.
// y = 16 x + o (o = the grid origin, 16 for NF4) is formed straight from the
// value, y = fma(v, 16 rcp(a), o), and lands in cell int(y) of the grid
// (unsigned conversion saturates below 0, and x <= 1 + 2^-22 keeps y below 33);
// the cell stores (fl32(16 thr + o), base) and code = base + (y > thr16).  y
// differs from 16 fl32(v / a) + o by less than 2^-18 and thr16 from 16 thr + o
// by at most 2^-19, so outside the window |y - thr16| < 2^-16 the comparison
// decides exactly as fl32(v / a) > thr; elements inside it are redone with an
// IEEE division and a full threshold count.
// The reciprocal bound needs a normal rcp(a) whose 16-fold product stays finite,
// so a block with a outside [2^-120, 2^120] (tiny normals and subnormals, where
// 16 rcp(a) would overflow, and huge values, whose reciprocal is subnormal)
// skips the fast path: inv16 = 0 keeps every y at the origin cell, in range,
// and all 16 elements take the exact division.  With inv16 finite and
// |v| <= a, 0 <= y < 33 for every finite v, so the cell index is in range.
__device__ __forceinline__ uint2 encode16(const float v[16], float a, const EncodeLds& s) {
  const bool fast = a >= 0x1p-120f && a <= 0x1p+120f;
  const float inv16 = fast ? 16.f * __builtin_amdgcn_rcpf(a) : 0.f;
  const float origin = s.origin;
  uint32_t danger = (!fast && a > 0.f) ? 0xFFFFu : 0u;
  uint32_t w0 = 0, w1 = 0;
#pragma unroll
  for (int e = 0; e < 16; ++e) {
    const float y = fmaf(v[e], inv16, origin);
    const float2 c = s.cell[static_cast<uint32_t>(y)];
    const float d = y - c.x;
    const uint32_t code = static_cast<uint32_t>(__float_as_int(c.y)) + ((d > 0.f) ? 1u : 0u);
    if (fabsf(d) < kDangerWindow16) danger |= 1u << e;
    if (e < 8) w0 |= code << nib_shift(e);
    else w1 |= code << nib_shift(e);
  }
  if (danger) {
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      if (danger & (1u << e)) {
        const uint32_t code = exact_code(v[e], a, s);
        const int sh = nib_shift(e);
        if (e < 8) w0 = (w0 & ~(0xFu << sh)) | (code << sh);
        else w1 = (w1 & ~(0xFu << sh)) | (code << sh);
      }
    }
  }
  return make_uint2(w0, w1);
}

// ---------------------------------------------------------------------------
// Quantize full 64-blocks of R = W (no adapter).  One thread per group; the
// grid-stride loop advances whole quads, so a quad is always uniformly active.
template <typename T>
__global__ __launch_bounds__(kThreads) void quantize_plain_kernel(const T* __restrict__ W, int64_t ngroups,
                                                                  uint8_t* __restrict__ packed,
                                                                  float* __restrict__ absmax, Nf4Tables tab) {
  __shared__ EncodeLds s;
  fill_lds(s, tab);
  __syncthreads();
  const int64_t stride = static_cast<int64_t>(gridDim.x) * kThreads;
  for (int64_t g = static_cast<int64_t>(blockIdx.x) * kThreads + threadIdx.x; g < ngroups; g += stride) {
    float v[16];
    load16(W + g * 16, v);
    float m = 0.f;  // (one group per thread at the launch size below)
#pragma unroll
    for (int e = 0; e < 16; ++e) m = fmaxf(m, fabsf(v[e]));
    const float a = quad_max(m);
    const uint2 w = encode16(v, a, s);
    reinterpret_cast<uint2*>(packed)[g] = w;
    if ((threadIdx.x & 3) == 0) absmax[g >> 2] = a;
  }
}

// Any shape, any tail, optional adapter: one quad per 64-block with per-element
// bounds and per-element (row, col) indexing.  Used for ragged tails and for
// adapters on matrices whose column count is not a multiple of 64.
template <typename T>
__global__ __launch_bounds__(kThreads) void quantize_generic_kernel(const T* __restrict__ W, int64_t n,
                                                                    int64_t cols, const float* __restrict__ B,
                                                                    const float* __restrict__ A, int r,
                                                                    int64_t block_begin, int64_t block_end,
                                                                    uint8_t* __restrict__ packed,
                                                                    float* __restrict__ absmax, Nf4Tables tab) {
  __shared__ EncodeLds s;
  fill_lds(s, tab);
  __syncthreads();
  const int64_t quads = static_cast<int64_t>(gridDim.x) * (kThreads / 4);
  const int sub = threadIdx.x & 3;
  for (int64_t blk = block_begin + static_cast<int64_t>(blockIdx.x) * (kThreads / 4) + (threadIdx.x >> 2);
       blk < block_end; blk += quads) {
    const int64_t base = blk * 64 + sub * 16;
    float v[16];
    float m = 0.f;
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const int64_t i = base + e;
      float x = 0.f;
      if (i < n) {
        x = load1(W, i);
        if (B != nullptr) {
          const int64_t row = i / cols, col = i - row * cols;
          float acc = 0.f;
          for (int p = 0; p < r; ++p) acc = fmaf(B[row * r + p], A[static_cast<int64_t>(p) * cols + col], acc);
          x = x - acc;
        }
      }
      v[e] = x;
      m = fmaxf(m, fabsf(x));
    }
    const float a = quad_max(m);
    const uint2 w = encode16(v, a, s);
    uint32_t word[2] = {w.x, w.y};
#pragma unroll
    for (int e = 0; e < 16; ++e)  // elements past the end leave a zero nibble
      if (base + e >= n) word[e >> 3] &= ~(0xFu << nib_shift(e));
#pragma unroll
    for (int b = 0; b < 8; ++b) {
      const int64_t i = base + 2 * b;
      if (i < n) packed[i >> 1] = static_cast<uint8_t>((word[b >> 2] >> (8 * (b & 3))) & 0xFFu);
    }
    if (sub == 0) absmax[blk] = a;
  }
}

template <typename T>
__device__ __forceinline__ void load16_raw(const T* __restrict__ p, uint4 (&raw)[4]) {
  if (sizeof(T) == 2) {
    raw[0] = reinterpret_cast<const uint4*>(p)[0];
    raw[1] = reinterpret_cast<const uint4*>(p)[1];
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i) raw[i] = reinterpret_cast<const uint4*>(p)[i];
  }
}
template <typename T>
__device__ __forceinline__ void raw_to_f32(const uint4 (&raw)[4], float v[16]) {
  if (sizeof(T) == 2) {
    const uint32_t w[8] = {raw[0].x, raw[0].y, raw[0].z, raw[0].w, raw[1].x, raw[1].y, raw[1].z, raw[1].w};
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      v[2 * i] = __uint_as_float(w[i] << 16);
      v[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
    }
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[4 * i] = __uint_as_float(raw[i].x);
      v[4 * i + 1] = __uint_as_float(raw[i].y);
      v[4 * i + 2] = __uint_as_float(raw[i].z);
      v[4 * i + 3] = __uint_as_float(raw[i].w);
    }
  }
}

// Where the fused kernel takes the base of its residual from.  load() fetches
// the 16 elements e0 .. e0 + 15 of one lane (raw words), to_f32() turns them
// into fp32 values; lvl2 is the level-pair table in LDS (kCodes sources only).
// kScaleB: the B operand is multiplied by the kernel's bscale when loaded.
template <typename T>
struct WeightSource {   // the weight W itself (bf16 or fp32): R = W - B A
  const T* W;
  static constexpr bool kScaleB = false, kCodes = false;
  __device__ __forceinline__ void load(int64_t e0, uint4 (&raw)[4]) const { load16_raw(W + e0, raw); }
  __device__ __forceinline__ void to_f32(const uint4 (&raw)[4], float v[16], const lvpair*) const {
    raw_to_f32<T>(raw, v);
  }
};
template <bool kDQ>
struct Nf4Source {      // deq(Q) of existing codes: R = deq(Q) - bscale B A
  const uint8_t* packed;
  const float* absmax;  // per-block scale (no double quant)
  const int8_t* qa;     // or qabsmax and dq_scale per dq group
  const float* dqs;
  int dqbs;
  static constexpr bool kScaleB = true, kCodes = true;
  // 16 codes (8 bytes) and the block's dequant scale a', as in the dequant kernel
  __device__ __forceinline__ void load(int64_t e0, uint4 (&raw)[4]) const {
    const uint2 c = *reinterpret_cast<const uint2*>(packed + (e0 >> 1));
    const int64_t b = e0 >> 6;
    const float a = kDQ ? static_cast<float>(qa[b]) * dqs[b / dqbs] : absmax[b];
    raw[0] = make_uint4(c.x, c.y, __float_as_uint(a), 0u);
  }
  __device__ __forceinline__ void to_f32(const uint4 (&raw)[4], float v[16], const lvpair* lvl2) const {
    const float a = __uint_as_float(raw[0].z);
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const lvpair c = lvl2[((j < 4 ? raw[0].x : raw[0].y) >> (8 * (j & 3))) & 0xFFu];
      v[2 * j] = c.x * a;       // deq = fl32(c[code] a'), one rounding
      v[2 * j + 1] = c.y * a;
    }
  }
};

// Fused residual R = W - B A (cols % 64 == 0, r <= 64).  Each wave owns one
// 64-column block column and walks a run of 16-row tiles of it; waves share
// nothing, so there is no LDS tile and no barrier after the table fill.
//
// B A of a tile comes from the bf16 matrix cores (v_mfma_f32_16x16x32_bf16:
// lane L supplies A_op[L%16][8(L/16)+e] and B_op[8(L/16)+e][L%16], e = 0..7, and
// receives D[4(L/16)+v][L%16]) with M = 16 columns, N = 16 rows and K = 32 rank
// indices p = 32 s + 8 (L/16) + e (K step s; zero past r); for r <= 16 the
// 16x16x16 form, K = 16 rank indices p = 4 (L/16) + e, e = 0..3.  Both operands are
// split into bf16 pieces, hi = bf16(x) and lo = bf16(x - hi), and B A is
// accumulated in fp32 as A_hi B_hi + A_hi B_lo + A_lo B_hi (the dropped lo lo
// term is below 2^-16 of each product).  MFMA tile t maps its M index m to block
// column 16 (m >> 2) + 4 t + (m & 3), so lane (li, g) ends up holding row li,
// columns 16 g .. 16 g + 15 of the block: exactly the 16-element group it loaded
// from W, with the block's four groups in lanes li, li + 16, li + 32, li + 48.
// A's split operands (4 tiles per K step) stay in registers for the whole run;
// the next tile's W and B values are loaded before the current tile is
// computed, and B is split when its tile is.
constexpr int kFusedThreads = 256, kFusedMaxR = 64;

typedef float floatx4 __attribute__((ext_vector_type(4)));

template <typename Src, int R16, bool kFullR>
__global__ __launch_bounds__(kFusedThreads) __attribute__((amdgpu_waves_per_eu(R16 <= 16 ? 4 : 2))) void quantize_fused_kernel(Src src, int64_t rows,
                                                                       int64_t cols, const float* __restrict__ B,
                                                                       const float* __restrict__ A, int r, float bscale,
                                                                       int tpw, uint8_t* __restrict__ packed,
                                                                       float* __restrict__ absmax, Nf4Tables tab) {
  constexpr bool K16 = R16 == 16;            // one K step of 16 rank indices (16x16x16 MFMA)
  constexpr int KS = K16 ? 1 : (R16 + 31) / 32;   // else K steps of 32
  constexpr int KW = K16 ? 4 : 8;            // rank indices per lane and K step
  __shared__ EncodeLds s;
  __shared__ lvpair lvl2[Src::kCodes ? 256 : 1];
  fill_lds(s, tab);
  if constexpr (Src::kCodes) fill_level_pairs(lvl2, tab, threadIdx.x, kFusedThreads);
  __syncthreads();
  const int lane = threadIdx.x & 63, li = lane & 15, g = lane >> 4;
  const int64_t nbc = cols >> 6;
  const int64_t wave = (static_cast<int64_t>(blockIdx.x) * kFusedThreads + threadIdx.x) >> 6;
  const int64_t bc = wave % nbc, chunk = wave / nbc;
  const int64_t ntiles = (rows + 15) >> 4;
  const int64_t t0 = chunk * tpw;
  if (t0 >= ntiles) return;
  const int64_t t1 = (t0 + tpw < ntiles) ? t0 + tpw : ntiles;
  const int64_t col0 = bc << 6;
  // split operands as packed bf16 pairs: KW / 2 words each
  uint32_t aoh[KS][4][KW / 2], aol[KS][4][KW / 2];
  {
    const int64_t cbase = col0 + 16 * (li >> 2) + (li & 3);
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        float x[KW];
#pragma unroll
        for (int e = 0; e < KW; ++e) {
          const int p = 32 * ks + KW * g + e;
          x[e] = p < r ? A[static_cast<int64_t>(p) * cols + cbase + 4 * t] : 0.f;
        }
        split_pairs<KW>(x, aoh[ks][t], aol[ks][t]);
      }
  }
  // B[row][32 ks + KW g .. + KW - 1] of the lane's row (bscale applied), zero past r
  auto load_tile = [&](int64_t tile, uint4 (&raw)[4], float (&bop)[KS][KW]) {
    const int64_t row = (tile << 4) + li;
    const int64_t rc = row < rows ? row : rows - 1;
    src.load(rc * cols + col0 + 16 * g, raw);
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const int p0 = 32 * ks + KW * g;
      if (kFullR) {   // r == R16, a multiple of 16: the lane's values are all in range or all past r
#pragma unroll
        for (int q = 0; q < KW / 4; ++q) {
          float4 b = make_float4(0.f, 0.f, 0.f, 0.f);
          if (p0 < R16) b = *reinterpret_cast<const float4*>(B + rc * R16 + p0 + 4 * q);
          bop[ks][4 * q] = b.x; bop[ks][4 * q + 1] = b.y; bop[ks][4 * q + 2] = b.z; bop[ks][4 * q + 3] = b.w;
        }
      } else {
#pragma unroll
        for (int e = 0; e < KW; ++e) bop[ks][e] = (p0 + e < r) ? B[rc * r + p0 + e] : 0.f;
      }
      if (Src::kScaleB) {
#pragma unroll
        for (int e = 0; e < KW; ++e) bop[ks][e] *= bscale;
      }
    }
  };
  auto mfma = [](const uint32_t (&a)[KW / 2], const uint32_t (&b)[KW / 2], floatx4 c) -> floatx4 {
    if constexpr (K16) {
      typedef short short4v __attribute__((ext_vector_type(4)));
      return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(short4v, uint2{a[0], a[1]}),
                                                      __builtin_bit_cast(short4v, uint2{b[0], b[1]}), c, 0, 0, 0);
    } else {
      return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, uint4{a[0], a[1], a[2], a[3]}),
                                                     __builtin_bit_cast(bf16x8, uint4{b[0], b[1], b[2], b[3]}), c, 0,
                                                     0, 0);
    }
  };
  auto do_tile = [&](int64_t tile, const uint4 (&raw)[4], const float (&bop)[KS][KW]) {
    floatx4 acc[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) acc[t] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      uint32_t bh[KW / 2], bl[KW / 2];
      split_pairs<KW>(bop[ks], bh, bl);
#pragma unroll
      for (int t = 0; t < 4; ++t) acc[t] = mfma(aoh[ks][t], bh, acc[t]);
#pragma unroll
      for (int t = 0; t < 4; ++t) acc[t] = mfma(aoh[ks][t], bl, acc[t]);
#pragma unroll
      for (int t = 0; t < 4; ++t) acc[t] = mfma(aol[ks][t], bh, acc[t]);
    }
    float v[16];
    src.to_f32(raw, v, lvl2);
    float m = 0.f;
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        v[4 * t + q] -= acc[t][q];
        m = fmaxf(m, fabsf(v[4 * t + q]));
      }
    m = fmaxf(m, __shfl_xor(m, 16));
    m = fmaxf(m, __shfl_xor(m, 32));
    const uint2 w = encode16(v, m, s);
    const int64_t row = (tile << 4) + li;
    if (row < rows) {
      const int64_t e0 = row * cols + col0 + 16 * g;
      reinterpret_cast<uint2*>(packed)[e0 >> 4] = w;
      if (g == 0) absmax[e0 >> 6] = m;
    }
  };
  uint4 raw0[4], raw1[4];
  float bop0[KS][KW], bop1[KS][KW];
  load_tile(t0, raw0, bop0);
  int64_t tile = t0;
  for (; tile + 1 < t1; tile += 2) {
    // the prefetch is unconditional (at the end of the run a harmless repeat of
    // the last tile) and pinned before the compute, so the wait before each
    // tile's MFMA covers that tile's loads only and the next tile's stay in flight
    load_tile(tile + 1, raw1, bop1);
    __builtin_amdgcn_sched_barrier(0);
    do_tile(tile, raw0, bop0);
    load_tile(tile + 2 < t1 ? tile + 2 : t1 - 1, raw0, bop0);
    __builtin_amdgcn_sched_barrier(0);
    do_tile(tile + 1, raw1, bop1);
  }
  if (tile < t1) do_tile(tile, raw0, bop0);
}

// ---------------------------------------------------------------------------
// Double quant of the absmax: group scale = max / 127 (IEEE division), code =
// round-to-nearest-even of a / scale clamped to [0, 127] (0 for a zero group).
// Shared by the double-quant kernel and the dequant that derives it on the fly.
__device__ __forceinline__ float dq_group_scale(float m) { return m / 127.0f; }
__device__ __forceinline__ int dq_code(float a, float sc) {
  return sc != 0.f ? static_cast<int>(fminf(fmaxf(rintf(a / sc), 0.f), 127.f)) : 0;
}

// Double quant: one workgroup of 256 per group of dq_blocksize (= 256) absmax.
// a_out (optional): each block's dequantization scale a' = fl32(q scale), as the
// dequant forms it.
__global__ __launch_bounds__(256) void double_quant_kernel(const float* __restrict__ absmax, int64_t nb, int dqbs,
                                                           int8_t* __restrict__ q, float* __restrict__ scale,
                                                           float* __restrict__ a_out) {
  __shared__ float red[4];
  const int64_t base = static_cast<int64_t>(blockIdx.x) * dqbs;
  const int tid = threadIdx.x;
  const bool ok = tid < dqbs && base + tid < nb;
  const float a = ok ? absmax[base + tid] : 0.f;
  float m = a;
  for (int off = 32; off > 0; off >>= 1) m = fmaxf(m, __shfl_xor(m, off));
  if ((tid & 63) == 0) red[tid >> 6] = m;
  __syncthreads();
  m = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  const float sc = dq_group_scale(m);
  if (tid == 0) scale[blockIdx.x] = sc;
  if (ok) {
    const int c = dq_code(a, sc);
    q[base + tid] = static_cast<int8_t>(c);
    if (a_out != nullptr) a_out[base + tid] = static_cast<float>(c) * sc;
  }
}

// ---------------------------------------------------------------------------
// Dequant: out = deq or W - deq, plus sum of out^2.
//
// Whole 1024-element slices go one per wave: lane L handles elements
// 256 q + 4 L .. + 3 of the slice for q = 0..3, so the code, weight and output
// accesses of every instruction are one contiguous run (the float4 stores write
// 1 KB each).  Storing a thread's 64 contiguous output bytes as four float4
// instead leaves each store instruction strided and costs about 1.6x.  The
// ragged end (n mod 1024 elements) is done by workgroup 0 after its slices.
constexpr int kDeqMaxBlocks = 2048;

__device__ __forceinline__ void load4(const uint16_t* __restrict__ p, float v[4]) {
  const uint2 a = *reinterpret_cast<const uint2*>(p);
  v[0] = __uint_as_float(a.x << 16);
  v[1] = __uint_as_float(a.x & 0xFFFF0000u);
  v[2] = __uint_as_float(a.y << 16);
  v[3] = __uint_as_float(a.y & 0xFFFF0000u);
}
__device__ __forceinline__ void load4(const float* __restrict__ p, float v[4]) {
  const float4 a = *reinterpret_cast<const float4*>(p);
  v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
}

// Dequant scale of block b.  kDQ 0: absmax; 1: qabsmax x dq_scale as given;
// 2: derived from absmax on the fly (the group's maximum recomputed; ragged-end use only).
template <int kDQ>
__device__ __forceinline__ float block_scale(const float* __restrict__ absmax, const int8_t* __restrict__ qa,
                                             const float* __restrict__ dqs, int dqbs, int64_t nb, int64_t b) {
  if (kDQ == 0) return absmax[b];
  if (kDQ == 1) return static_cast<float>(qa[b]) * dqs[b / dqbs];
  const int64_t g0 = b / dqbs * dqbs, g1 = g0 + dqbs < nb ? g0 + dqbs : nb;
  float m = 0.f;
  for (int64_t i = g0; i < g1; ++i) m = fmaxf(m, absmax[i]);
  const float sc = dq_group_scale(m);
  return static_cast<float>(dq_code(absmax[b], sc)) * sc;
}

// kDQ 2 (dq_blocksize 256, 16 slices per group): each wave takes its group's
// maximum over the 256 absmax, forms the scales of its slice itself, and the
// wave of the group's first slice also writes the group's qabsmax and dq_scale;
// groups that start in the ragged end are written by workgroup 0.
template <typename T, bool kHasW, int kDQ>
__global__ __launch_bounds__(kThreads) void dequant_kernel(const uint8_t* __restrict__ packed,
                                                           const float* __restrict__ absmax,
                                                           const int8_t* __restrict__ qa,
                                                           const float* __restrict__ dqs, int dqbs, int64_t n,
                                                           int8_t* __restrict__ qa_out, float* __restrict__ dqs_out,
                                                           float* __restrict__ a_out,
                                                           const T* __restrict__ W, float* __restrict__ out,
                                                           double* __restrict__ partials,
                                                           double* __restrict__ wpartials,
                                                           double* __restrict__ sumsq, Nf4Tables tab) {
  __shared__ float lvl[16];
  __shared__ lvpair lvl2[256];
  __shared__ double red[2 * (kThreads / 64)];
  const bool wsum = kHasW && wpartials != nullptr;
  if (threadIdx.x < 16) lvl[threadIdx.x] = tab.level[threadIdx.x];
  fill_level_pairs(lvl2, tab, threadIdx.x, kThreads);
  __syncthreads();
  const int lane = threadIdx.x & 63;
  const int64_t nslices = n >> 10;
  const int64_t nb = (n + 63) >> 6;
  const int64_t nwaves = static_cast<int64_t>(gridDim.x) * (kThreads / 64);
  double acc = 0.0, wacc = 0.0;
  for (int64_t sl = (static_cast<int64_t>(blockIdx.x) * kThreads + threadIdx.x) >> 6; sl < nslices; sl += nwaves) {
    const int64_t base = (sl << 10) + 4 * lane;
    uint32_t cw[4];
    float a[4], w[4][4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int64_t e = base + 256 * q;
      cw[q] = reinterpret_cast<const uint16_t*>(packed)[e >> 2];
      if (kDQ != 2) a[q] = block_scale<kDQ>(absmax, qa, dqs, dqbs, nb, e >> 6);
      if (kHasW) load4(W + e, w[q]);
    }
    if (kDQ == 2) {
      const int64_t g = sl >> 4, b0 = g << 8;
      float am[4], m = 0.f;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int64_t b = b0 + lane + 64 * i;
        am[i] = b < nb ? absmax[b] : 0.f;
        m = fmaxf(m, am[i]);
      }
#pragma unroll
      for (int off = 32; off > 0; off >>= 1) m = fmaxf(m, __shfl_xor(m, off));
      const float sc = dq_group_scale(m);
#pragma unroll
      for (int q = 0; q < 4; ++q) a[q] = static_cast<float>(dq_code(absmax[(base + 256 * q) >> 6], sc)) * sc;
      if ((sl & 15) == 0) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int64_t b = b0 + lane + 64 * i;
          if (b < nb) {
            const int qc = dq_code(am[i], sc);
            qa_out[b] = static_cast<int8_t>(qc);
            if (a_out != nullptr) a_out[b] = static_cast<float>(qc) * sc;
          }
        }
        if (lane == 0) dqs_out[g] = sc;
      }
    }
    float ss = 0.f, ws = 0.f;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      float o[4];
      const lvpair c01 = lvl2[cw[q] & 0xFFu], c23 = lvl2[(cw[q] >> 8) & 0xFFu];   // elements 0,1 and 2,3
      const float lv[4] = {c01.x, c01.y, c23.x, c23.y};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float d = lv[j] * a[q];
        o[j] = kHasW ? (w[q][j] - d) : d;
        ss = fmaf(o[j], o[j], ss);
        if (kHasW) ws = fmaf(w[q][j], w[q][j], ws);
      }
      if (out != nullptr) *reinterpret_cast<float4*>(out + base + 256 * q) = make_float4(o[0], o[1], o[2], o[3]);
    }
    acc += static_cast<double>(ss);
    wacc += static_cast<double>(ws);
  }
  // ragged end: whole groups of 16 by the threads of workgroup 0, then the last
  // few elements by its thread 0; with kDQ 2 also the double quant of the
  // groups whose first slice is not whole
  if (blockIdx.x == 0) {
    if (kDQ == 2) {
      const int64_t ng = (nb + 255) >> 8;
      for (int64_t g = ((nslices + 15) >> 4) + threadIdx.x; g < ng; g += kThreads) {
        const int64_t g0 = g << 8, g1 = g0 + 256 < nb ? g0 + 256 : nb;
        float m = 0.f;
        for (int64_t b = g0; b < g1; ++b) m = fmaxf(m, absmax[b]);
        const float sc = dq_group_scale(m);
        for (int64_t b = g0; b < g1; ++b) {
          const int qc = dq_code(absmax[b], sc);
          qa_out[b] = static_cast<int8_t>(qc);
          if (a_out != nullptr) a_out[b] = static_cast<float>(qc) * sc;
        }
        dqs_out[g] = sc;
      }
    }
    const int64_t ngroups = n >> 4;
    for (int64_t g = (nslices << 6) + threadIdx.x; g < ngroups; g += kThreads) {
      const float sc = block_scale<kDQ>(absmax, qa, dqs, dqbs, nb, g >> 2);
      const uint2 pw = reinterpret_cast<const uint2*>(packed)[g];
      float ss = 0.f, ws = 0.f;
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const uint32_t code = (((e < 8) ? pw.x : pw.y) >> nib_shift(e)) & 0xFu;
        const float d = lvl[code] * sc;
        const float wv = kHasW ? load1(W, g * 16 + e) : 0.f;
        const float o = kHasW ? (wv - d) : d;
        if (out != nullptr) out[g * 16 + e] = o;
        ss = fmaf(o, o, ss);
        ws = fmaf(wv, wv, ws);
      }
      acc += static_cast<double>(ss);
      wacc += static_cast<double>(ws);
    }
    if (threadIdx.x == 0) {
      float ss = 0.f, ws = 0.f;
      for (int64_t i = ngroups * 16; i < n; ++i) {
        const float sc = block_scale<kDQ>(absmax, qa, dqs, dqbs, nb, i >> 6);
        const uint32_t code = (packed[i >> 1] >> ((i & 1) ? 0 : 4)) & 0xFu;
        const float d = lvl[code] * sc;
        const float wv = kHasW ? load1(W, i) : 0.f;
        const float o = kHasW ? (wv - d) : d;
        if (out != nullptr) out[i] = o;
        ss = fmaf(o, o, ss);
        ws = fmaf(wv, wv, ws);
      }
      acc += static_cast<double>(ss);
      wacc += static_cast<double>(ws);
    }
  }
  for (int off = 32; off > 0; off >>= 1) {
    acc += __shfl_xor(acc, off);
    if (wsum) wacc += __shfl_xor(wacc, off);
  }
  if ((threadIdx.x & 63) == 0) {
    red[threadIdx.x >> 6] = acc;
    red[kThreads / 64 + (threadIdx.x >> 6)] = wacc;
  }
  __syncthreads();
  double t = 0.0, tw = 0.0;
  for (int i = 0; i < kThreads / 64; ++i) {
    t += red[i];
    tw += red[kThreads / 64 + i];
  }
  if (threadIdx.x == 0) {
    if (partials != nullptr) partials[blockIdx.x] = t;
    else if (sumsq != nullptr) atomicAdd(sumsq, t);
    if (wsum) wpartials[blockIdx.x] = tw;
  }
}

__global__ void zero_double_kernel(double* p) { *p = 0.0; }

// Sum of squares of W (for ||W||_F), per-workgroup partials.
template <typename T>
__global__ __launch_bounds__(kThreads) void sumsq_kernel(const T* __restrict__ W, int64_t n,
                                                         double* __restrict__ partials,
                                                         unsigned* __restrict__ counter,
                                                         double* __restrict__ sumsq) {
  __shared__ double red[kThreads / 64];
  const int64_t ngroups = n >> 4;
  const int64_t stride = static_cast<int64_t>(gridDim.x) * kThreads;
  double acc = 0.0;
  for (int64_t g = static_cast<int64_t>(blockIdx.x) * kThreads + threadIdx.x; g < ngroups; g += stride) {
    float v[16];
    load16(W + g * 16, v);
    float ss = 0.f;
#pragma unroll
    for (int e = 0; e < 16; ++e) ss = fmaf(v[e], v[e], ss);
    acc += static_cast<double>(ss);
  }
  if (blockIdx.x == 0 && threadIdx.x == 0)
    for (int64_t i = ngroups * 16; i < n; ++i) {
      const double x = load1(W, i);
      acc += x * x;
    }
  for (int off = 32; off > 0; off >>= 1) acc += __shfl_xor(acc, off);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = acc;
  __syncthreads();
  double t = 0.0;
  for (int i = 0; i < kThreads / 64; ++i) t += red[i];
  if (threadIdx.x == 0) partials[blockIdx.x] = t;
}

int grid_for_groups(int64_t ngroups, int per_thread) {
  int64_t blocks = (ngroups + static_cast<int64_t>(kThreads) * per_thread - 1) / (static_cast<int64_t>(kThreads) * per_thread);
  if (blocks < 1) blocks = 1;
  if (blocks > 65536) blocks = 65536;
  return static_cast<int>(blocks);
}

// Grid of the fused kernel: every block column is cut into c runs of tpw 16-row
// tiles, one wave each.  The chip holds 1024 x occ waves at once (occ: waves per
// SIMD the kernel's registers allow for this r16), so the kernel takes
// ceil(nbc c / (1024 occ)) rounds of a run each; a run costs about tpw + 2 tiles
// (its set-up: A's operands, the tables), and c minimises the total, the fewest
// waves on a tie.
dim3 fused_grid(int64_t rows, int64_t cols, int r16, int& tpw_out) {
  const int64_t nbc = cols / 64, ntiles = (rows + 15) / 16;
  const int64_t slots = 1024 * static_cast<int64_t>(r16 <= 16 ? 4 : (r16 <= 32 ? 3 : 2));
  int64_t best_c = 1, best = -1;
  for (int64_t c = 1; c <= ntiles && c <= 4096; ++c) {
    const int64_t tpw = (ntiles + c - 1) / c;
    if ((ntiles + tpw - 1) / tpw != c) continue;   // same runs as a smaller c
    const int64_t cost = ((nbc * c + slots - 1) / slots) * (tpw + 2);
    if (best < 0 || cost < best) {
      best = cost;
      best_c = c;
    }
  }
  const int64_t tpw = (ntiles + best_c - 1) / best_c;
  tpw_out = static_cast<int>(tpw);
  return dim3(static_cast<unsigned>((nbc * best_c + 3) / 4));
}

template <typename T>
hipError_t quantize_typed(const T* W, int64_t rows, int64_t cols, const float* B, const float* A, int r,
                          uint8_t* packed, float* absmax, hipStream_t s, int bits) {
  const Nf4Tables& tab = nf_tables(bits);
  const int64_t n = rows * cols;
  if (n == 0) return hipSuccess;
  const int64_t nblocks = (n + 63) / 64;
  if (B == nullptr) {
    const int64_t full = n / 64;
    if (full > 0) {
      LQ_LAUNCH("nf4_quantize", quantize_plain_kernel<T>, dim3(grid_for_groups(full * 4, 1)), dim3(kThreads), 0, s, W,
                         full * 4, packed, absmax, tab);
    }
    if (full < nblocks) {
      LQ_LAUNCH("nf4_quantize_generic", quantize_generic_kernel<T>, dim3(1), dim3(kThreads), 0, s, W, n, cols,
                         static_cast<const float*>(nullptr), static_cast<const float*>(nullptr), 0, full, nblocks,
                         packed, absmax, tab);
    }
  } else if (cols % 64 == 0 && r <= kFusedMaxR) {
    const int r16 = (r + 15) / 16 * 16;
    int tpw = 0;
    const dim3 grid = fused_grid(rows, cols, r16, tpw);
    const bool full = (r == r16);
    const WeightSource<T> src{W};
#define LQ_FUSED(R16)                                                                                              \
  do {                                                                                                             \
    if (full)                                                                                                      \
      LQ_LAUNCH("nf4_quantize_fused", (quantize_fused_kernel<WeightSource<T>, R16, true>), grid,                  \
                dim3(kFusedThreads), 0, s, src, rows, cols, B, A, r, 1.f, tpw, packed, absmax, tab);               \
    else                                                                                                           \
      LQ_LAUNCH("nf4_quantize_fused", (quantize_fused_kernel<WeightSource<T>, R16, false>), grid,                 \
                dim3(kFusedThreads), 0, s, src, rows, cols, B, A, r, 1.f, tpw, packed, absmax, tab);               \
  } while (0)
    if (r16 == 16) LQ_FUSED(16);
    else if (r16 == 32) LQ_FUSED(32);
    else if (r16 == 48) LQ_FUSED(48);
    else LQ_FUSED(64);
#undef LQ_FUSED
  } else {
    int64_t grid = (nblocks + (kThreads / 4) - 1) / (kThreads / 4);
    if (grid > 65536) grid = 65536;
    LQ_LAUNCH("nf4_quantize_generic", quantize_generic_kernel<T>, dim3(static_cast<unsigned>(grid)), dim3(kThreads), 0, s, W, n,
                       cols, B, A, r, static_cast<int64_t>(0), nblocks, packed, absmax, tab);
  }
  return hipGetLastError();
}

template <typename T>
hipError_t dequant_typed(const uint8_t* packed, const float* absmax, const int8_t* q, const float* dqs, int64_t n,
                         int dqbs, int8_t* q_out, float* dqs_out, const T* W, float* out, double* partials,
                         double* wpartials, double* sumsq, hipStream_t s, int bits, float* a_out) {
  const Nf4Tables& tab = nf_tables(bits);
  const int grid = dequant_num_partials(n);
  if (partials == nullptr && sumsq != nullptr) LQ_LAUNCH("zero", zero_double_kernel, dim3(1), dim3(1), 0, s, sumsq);
  const int mode = q_out != nullptr ? 2 : (q != nullptr ? 1 : 0);
#define LQ_DEQ(HW, DQ)                                                                                            \
  LQ_LAUNCH("nf4_dequantize", (dequant_kernel<T, HW, DQ>), dim3(grid), dim3(kThreads), 0, s, packed, absmax, q,   \
            dqs, dqbs, n, q_out, dqs_out, a_out, W, out, partials, wpartials, sumsq, tab)
  if (W != nullptr) {
    if (mode == 2) LQ_DEQ(true, 2); else if (mode == 1) LQ_DEQ(true, 1); else LQ_DEQ(true, 0);
  } else {
    if (mode == 2) LQ_DEQ(false, 2); else if (mode == 1) LQ_DEQ(false, 1); else LQ_DEQ(false, 0);
  }
#undef LQ_DEQ
  return hipGetLastError();
}

}  // namespace

int dequant_num_partials(int64_t n) {
  int g = grid_for_groups((n >> 4) + 1, 4);
  return g > kDeqMaxBlocks ? kDeqMaxBlocks : g;
}

hipError_t launch_nf4_quantize(const void* W, loftq_dtype_t wdt, int64_t rows, int64_t cols, const float* B,
                               const float* A, int r, uint8_t* packed, float* absmax, hipStream_t s, int bits) {
  if (wdt == LOFTQ_BF16)
    return quantize_typed(static_cast<const uint16_t*>(W), rows, cols, B, A, r, packed, absmax, s, bits);
  return quantize_typed(static_cast<const float*>(W), rows, cols, B, A, r, packed, absmax, s, bits);
}

// Adapter merge Q' = NF4(deq(Q) + alpha B A) (alpha < 0 takes it out again):
// the fused kernel with deq(Q) as the residual's base, so codes, scales and the
// adapter are read once and deq(Q) never reaches memory; then, when q_out is
// given, the double quant of the new absmax.  Requires cols % 64 == 0 and
// 0 <= r <= 64 (r = 0: B, A unused).  Each block is read and written by one
// wave, codes before scales, so packed_out / absmax_out may be packed / absmax.
hipError_t launch_nf4_merge(const uint8_t* packed, const float* absmax, const int8_t* qa, const float* dqs,
                            int64_t rows, int64_t cols, const float* B, const float* A, int r, float alpha,
                            uint8_t* packed_out, float* absmax_out, int8_t* q_out, float* dqs_out, hipStream_t s) {
  const Nf4Tables& tab = nf4_tables();
  const int64_t n = rows * cols;
  if (n == 0) return hipSuccess;
  if (cols % 64 != 0 || r < 0 || r > kFusedMaxR) return hipErrorInvalidValue;
  const int r16 = r <= 16 ? 16 : (r + 15) / 16 * 16;
  int tpw = 0;
  const dim3 grid = fused_grid(rows, cols, r16, tpw);
  const bool full = (r == r16);
  const float bscale = -alpha;
#define LQ_MERGE(SRC, R16)                                                                                         \
  do {                                                                                                             \
    if (full)                                                                                                      \
      LQ_LAUNCH("nf4_merge", (quantize_fused_kernel<SRC, R16, true>), grid, dim3(kFusedThreads), 0, s, src, rows, \
                cols, B, A, r, bscale, tpw, packed_out, absmax_out, tab);                                          \
    else                                                                                                           \
      LQ_LAUNCH("nf4_merge", (quantize_fused_kernel<SRC, R16, false>), grid, dim3(kFusedThreads), 0, s, src, rows,\
                cols, B, A, r, bscale, tpw, packed_out, absmax_out, tab);                                          \
  } while (0)
#define LQ_MERGE_R(SRC)                \
  do {                                 \
    if (r16 == 16) LQ_MERGE(SRC, 16);  \
    else if (r16 == 32) LQ_MERGE(SRC, 32); \
    else if (r16 == 48) LQ_MERGE(SRC, 48); \
    else LQ_MERGE(SRC, 64);            \
  } while (0)
  if (qa != nullptr) {
    const Nf4Source<true> src{packed, nullptr, qa, dqs, 256};
    LQ_MERGE_R(Nf4Source<true>);
  } else {
    const Nf4Source<false> src{packed, absmax, nullptr, nullptr, 256};
    LQ_MERGE_R(Nf4Source<false>);
  }
#undef LQ_MERGE_R
#undef LQ_MERGE
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || q_out == nullptr) return e;
  return launch_double_quant(absmax_out, (n + 63) / 64, 256, q_out, dqs_out, s);
}

hipError_t launch_double_quant(const float* absmax, int64_t nblocks, int dqbs, int8_t* q, float* scale,
                               hipStream_t s, float* a_out) {
  if (nblocks == 0) return hipSuccess;
  const int64_t groups = (nblocks + dqbs - 1) / dqbs;
  LQ_LAUNCH("double_quant", double_quant_kernel, dim3(static_cast<unsigned>(groups)), dim3(256), 0, s, absmax, nblocks,
                     dqbs, q, scale, a_out);
  return hipGetLastError();
}

hipError_t launch_nf4_dequantize(const uint8_t* packed, const float* absmax, const int8_t* q, const float* dqscale,
                                 int64_t n, int dqbs, const void* W, loftq_dtype_t wdt, float* out, double* partials,
                                 double* wpartials, double* sumsq, hipStream_t s, int8_t* q_out, float* dqs_out,
                                 int bits, float* a_out) {
  if (n == 0) {
    if (sumsq) LQ_LAUNCH("zero", zero_double_kernel, dim3(1), dim3(1), 0, s, sumsq);
    return hipGetLastError();
  }
  if (q_out != nullptr && dqbs != 256) return hipErrorInvalidValue;
  if (wdt == LOFTQ_BF16)
    return dequant_typed(packed, absmax, q, dqscale, n, dqbs, q_out, dqs_out, static_cast<const uint16_t*>(W), out,
                         partials, wpartials, sumsq, s, bits, a_out);
  return dequant_typed(packed, absmax, q, dqscale, n, dqbs, q_out, dqs_out, static_cast<const float*>(W), out,
                       partials, wpartials, sumsq, s, bits, a_out);
}

hipError_t launch_sumsq_weight(const void* W, loftq_dtype_t wdt, int64_t n, double* partials, unsigned* counter,
                               double* sumsq, hipStream_t s) {
  const int nparts = dequant_num_partials(n);
  if (wdt == LOFTQ_BF16)
    LQ_LAUNCH("sumsq_weight", sumsq_kernel<uint16_t>, dim3(nparts), dim3(kThreads), 0, s,
              static_cast<const uint16_t*>(W), n, partials, counter, sumsq);
  else
    LQ_LAUNCH("sumsq_weight", sumsq_kernel<float>, dim3(nparts), dim3(kThreads), 0, s, static_cast<const float*>(W), n,
              partials, counter, sumsq);
  return hipGetLastError();
}

}  // namespace loftq
