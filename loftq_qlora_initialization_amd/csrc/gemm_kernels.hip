// Thin products of the randomized SVD on the bf16 matrix cores:
//   gemm_nn: part[s] = E[:, K_s] P[K_s, :]      (E d x k row-major, P k x l)
//   gemm_tn: part[s] = E[R_s, :]^T Y[R_s, :]    (Y d x l)
// Both stream E exactly once per product; split-K partials across workgroups
// are summed in fixed order by reduce_gram.
//
// fp32 accuracy from bf16 matrix cores: each fp32 value x of E and of the panel is
// split into hi = bf16(x) and lo = bf16(x - hi) (both rounded to nearest even, so
// |x - hi - lo| <= 2^-18 |x|), and E P is accumulated in fp32 as
// E_hi P_hi + E_hi P_lo + E_lo P_hi (the dropped E_lo P_lo is below 2^-16 of each
// term).  Against fp32 matrix cores (v_mfma_f32_16x16x4_f32), whose work bounds
// the wide panels (l = 80: 160 flop per 4 bytes of E), the three bf16 products
// take about a fifth of the matrix-core time.  v_mfma_f32_16x16x32_bf16 takes
// K = 32 per instruction; in K step s lane (li, g) supplies K index 8 g + e
// (e = 0..7) <-> row split_row(s, g, e) of the panel (its split layout,
// split_index: row 32 s + 8 g + e for E P's operand; the rows of each pair of
// steps interleaved for E^T Y's), and E is loaded to match: gemm_nn reads 8
// consecutive columns of a row per lane (with a bf16 weight and cols % 64 == 0
// whole 128-byte lines, reordered through LDS: FormedCo), gemm_tn 4 columns of
// 8 rows.  E is split in registers as it arrives; the panel comes already split
// (split_index), written so by the split-K reduction that produces it.
//
// Out-of-range rows/columns of E are clamped to valid addresses rather than
// branched around: the matching rows of the skinny operand are zero (its
// buffers are zero-padded to the splits' full extent), and garbage output
// rows/columns are never stored.
#include "lowrank.h"
#include "small_solve.h"
#include "split_bf16.h"

namespace loftq {
namespace {

typedef float floatx4 __attribute__((ext_vector_type(4)));


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

typedef float lvpair2 __attribute__((ext_vector_type(2)));

// Where the products take E from: a stored E, or the weight and the codes
// (VirtualE).  fetch4 / fetch8 issue the loads of E[row][c ..] (4 or 8
// consecutive columns; past the last column the addresses are clamped as in
// load_run4, and the skinny operand's matching rows are zero) into a Raw held in
// the register ring; decode, at the step that consumes it, turns the Raw into
// values (a formed E through the level-pair table in LDS), so the loads stay in
// flight as long as a stored E's do.
template <bool VEC>
struct StoredE {
  static constexpr bool kVirtual = false, kCoalesced = false;
  typedef float4 Raw4;
  struct Raw8 { float4 a, b; };
  const float* E;
  __device__ __forceinline__ Raw4 fetch4(int64_t row, int64_t c, int64_t k) const {
    return load_run4<VEC>(E + row * k, c, k);
  }
  __device__ __forceinline__ Raw8 fetch8(int64_t row, int64_t c, int64_t k) const {
    return Raw8{load_run4<VEC>(E + row * k, c, k), load_run4<VEC>(E + row * k, c + 4, k)};
  }
  __device__ __forceinline__ float4 decode4(const Raw4& r, const lvpair2*) const { return r; }
  __device__ __forceinline__ void decode8(const Raw8& r, float (&x)[8], const lvpair2*) const {
    x[0] = r.a.x; x[1] = r.a.y; x[2] = r.a.z; x[3] = r.a.w;
    x[4] = r.b.x; x[5] = r.b.y; x[6] = r.b.z; x[7] = r.b.w;
  }
};
// cols % 8 == 0: an 8-column fetch never straddles the last column.  The block
// scale a' comes from one array (absmax, or the double-quantized scales the
// dequant writes out).
template <bool BF16>
struct FormedE {
  static constexpr bool kVirtual = true, kCoalesced = false;
  struct Raw4 {
    uint32_t w[BF16 ? 2 : 4];   // four weights (bf16 pairs or fp32)
    uint32_t cw;                // their two code bytes
    float a;
  };
  struct Raw8 {
    uint32_t w[BF16 ? 4 : 8];
    uint32_t cw;                // four code bytes
    float a;
  };
  VirtualE v;
  __device__ __forceinline__ Raw4 fetch4(int64_t row, int64_t c, int64_t k) const {
    c = c < k - 4 ? c : k - 4;
    const int64_t e = row * k + c;   // e % 4 == 0: one 64-block, two code bytes
    Raw4 r;
    if constexpr (BF16) {
      const uint2 u = *reinterpret_cast<const uint2*>(static_cast<const uint16_t*>(v.W) + e);
      r.w[0] = u.x; r.w[1] = u.y;
    } else {
      const uint4 u = *reinterpret_cast<const uint4*>(static_cast<const float*>(v.W) + e);
      r.w[0] = u.x; r.w[1] = u.y; r.w[2] = u.z; r.w[3] = u.w;
    }
    r.cw = reinterpret_cast<const uint16_t*>(v.packed)[e >> 2];
    r.a = v.scale[e >> 6];
    return r;
  }
  __device__ __forceinline__ Raw8 fetch8(int64_t row, int64_t c, int64_t k) const {
    c = c < k - 8 ? c : k - 8;
    const int64_t e = row * k + c;   // e % 8 == 0: one 64-block, four code bytes
    Raw8 r;
    if constexpr (BF16) {
      const uint4 u = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(v.W) + e);
      r.w[0] = u.x; r.w[1] = u.y; r.w[2] = u.z; r.w[3] = u.w;
    } else {
      const uint4 u0 = *reinterpret_cast<const uint4*>(static_cast<const float*>(v.W) + e);
      const uint4 u1 = *reinterpret_cast<const uint4*>(static_cast<const float*>(v.W) + e + 4);
      r.w[0] = u0.x; r.w[1] = u0.y; r.w[2] = u0.z; r.w[3] = u0.w;
      r.w[4] = u1.x; r.w[5] = u1.y; r.w[6] = u1.z; r.w[7] = u1.w;
    }
    r.cw = reinterpret_cast<const uint32_t*>(v.packed)[e >> 3];
    r.a = v.scale[e >> 6];
    return r;
  }
  // e = fl32(w - fl32(level[code] a')), element by element as the dequant forms it
  __device__ __forceinline__ static float wval(const uint32_t* w, int j) {
    if constexpr (BF16) return __uint_as_float((j & 1) ? (w[j >> 1] & 0xFFFF0000u) : (w[j >> 1] << 16));
    else return __uint_as_float(w[j]);
  }
  __device__ __forceinline__ float4 decode4(const Raw4& r, const lvpair2* lvl2) const {
    const lvpair2 c01 = lvl2[r.cw & 0xFFu], c23 = lvl2[(r.cw >> 8) & 0xFFu];
    const float d0 = c01.x * r.a, d1 = c01.y * r.a, d2 = c23.x * r.a, d3 = c23.y * r.a;
    return make_float4(wval(r.w, 0) - d0, wval(r.w, 1) - d1, wval(r.w, 2) - d2, wval(r.w, 3) - d3);
  }
  __device__ __forceinline__ void decode8(const Raw8& r, float (&x)[8], const lvpair2* lvl2) const {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const lvpair2 c = lvl2[(r.cw >> (8 * q)) & 0xFFu];
      const float d0 = c.x * r.a, d1 = c.y * r.a;
      x[2 * q] = wval(r.w, 2 * q) - d0;
      x[2 * q + 1] = wval(r.w, 2 * q + 1) - d1;
    }
  }
};
// Level pairs (level[b >> 4], level[b & 15]) of a code byte b (element 2i in the
// high nibble); all threads of the workgroup call it, a barrier follows.
template <typename Src>
__device__ __forceinline__ void fill_level_pairs(const Src& src, lvpair2* lvl2) {
  if constexpr (Src::kVirtual) {
    for (int i = threadIdx.x; i < 256; i += blockDim.x) lvl2[i] = lvpair2{src.v.level[i >> 4], src.v.level[i & 15]};
  }
}

// E P's formed residual with full-line loads (bf16 weight, cols % 64 == 0).  The
// matrix-core operand ties lane L to row L % 16, so a direct operand load reads
// only 64 bytes of each of 16 rows per instruction (half a 128-byte line).  Here
// a 16-row x 64-column piece (two K steps) is loaded with eight lanes per row
// (two instructions of 8 rows x 128 bytes for W, one of 16 rows x 32 bytes for
// the codes), passed through a per-wave LDS slot (stash), and read back in
// operand order (unstash): lane (li, g) gets row li, columns 32 s + 8 g .. + 7
// of K step s, exactly what fetch8 would have loaded, so decode, split and the
// products are unchanged.  The block scale (one per row of the piece) is loaded
// in operand order directly.  Each wave's slot is written and read by that wave
// only; its LDS operations run in order, and the fences below keep the compiler
// from moving them across one another.
struct CoRaw {
  uint4 w[2];   // W: half h holds row 8 h + (lane >> 3), columns 8 (lane & 7) .. + 7
  uint2 c;      // codes of row lane >> 2, elements 16 (lane & 3) .. + 15
  float a;      // the block scale of row lane & 15
};
constexpr int kCoSlot = 160;   // uint4 per 16-row piece: 128 of W, 32 of codes
struct FormedCo : FormedE<true> {
  static constexpr bool kCoalesced = true;
  typedef CoRaw Raw8;
  // rows row0 .. row0 + 15 (clamped to d), columns c0 .. c0 + 63 (c0 % 64 == 0;
  // past the last column the piece repeats the last 64 columns, whose panel rows are zero)
  __device__ __forceinline__ CoRaw fetch_co(int64_t row0, int64_t c0, int64_t d, int64_t k, int lane) const {
    c0 = c0 < k - 64 ? c0 : k - 64;
    const uint16_t* W = static_cast<const uint16_t*>(v.W);
    CoRaw r;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      int64_t rr = row0 + 8 * h + (lane >> 3);
      rr = rr < d ? rr : d - 1;
      r.w[h] = *reinterpret_cast<const uint4*>(W + rr * k + c0 + 8 * (lane & 7));
    }
    int64_t rc = row0 + (lane >> 2);
    rc = rc < d ? rc : d - 1;
    r.c = *reinterpret_cast<const uint2*>(v.packed + ((rc * k + c0) >> 1) + 8 * (lane & 3));
    int64_t ra = row0 + (lane & 15);
    ra = ra < d ? ra : d - 1;
    r.a = v.scale[(ra * k + c0) >> 6];
    return r;
  }
  // W piece p of row q goes to 16-byte slot 8 q + (p ^ (q & 7)): conflict-free
  // writes, and the 16 rows an operand read touches spread over the banks
  __device__ __forceinline__ static void stash(const CoRaw& r, uint4* slot, int lane) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int q = 8 * h + (lane >> 3);
      slot[8 * q + ((lane & 7) ^ (q & 7))] = r.w[h];
    }
    reinterpret_cast<uint2*>(slot + 128)[lane] = r.c;
  }
  __device__ __forceinline__ static FormedE<true>::Raw8 unstash(const uint4* slot, int lane, int s, float a) {
    const int m = lane & 15, g = lane >> 4;
    const uint4 w = slot[8 * m + ((4 * s + g) ^ (m & 7))];
    FormedE<true>::Raw8 r;
    r.w[0] = w.x; r.w[1] = w.y; r.w[2] = w.z; r.w[3] = w.w;
    r.cw = reinterpret_cast<const uint32_t*>(slot + 128)[8 * m + 4 * s + g];
    r.a = a;
    return r;
  }
};
// orders a wave's LDS writes before its reads of other lanes' data (and reads before later writes)
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// ---------------------------------------------------------------------------
// v_mfma_f32_16x16x32_bf16: lane L supplies A[L%16][8(L/16) + e] and
// B[8(L/16) + e][L%16] (e = 0..7) and receives D[4(L/16) + v][L%16] in element v.
__device__ __forceinline__ floatx4 mfma_bf16(const bf16x8& a, const bf16x8& b, floatx4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// Workgroups are handed to the 8 XCDs round-robin in launch order, each XCD with
// an L2 of its own.  The tile of a workgroup comes from its launch index so that
// every XCD takes one contiguous run of tiles (X_FAST: x varies fastest in the
// run): neighbouring tiles that read the same code and scale lines then meet in
// one L2 instead of fetching those lines once per XCD.
template <bool X_FAST>
__device__ __forceinline__ void xcd_tile(int& bx, int& by) {
  const int gx = static_cast<int>(gridDim.x), gy = static_cast<int>(gridDim.y);
  const int i = static_cast<int>(blockIdx.x) + static_cast<int>(blockIdx.y) * gx;
  const int n = gx * gy, q = n >> 3, rem = n & 7, x = i & 7, p = i >> 3;
  const int L = x * q + (x < rem ? x : rem) + p;
  if (X_FAST) { bx = L % gx; by = L / gx; } else { by = L % gy; bx = L / gy; }
}

template <int NT, int RTV = 1>
struct Nn3Cfg {
  static constexpr int RT = RTV;               // 16-row MFMA tiles per wave (nn_staged_rt)
  static constexpr int D = 4;                  // E register ring depth (K steps of 32)
  static constexpr int WR = 4;                 // waves along rows, sharing the staged panel
  static constexpr int PU = NT * 128;          // 16-byte pieces of one K step of the split panel
  static constexpr int PPT = (PU + 255) / 256; // of them per thread
};
// gemm_nnd_kernel: the panel read by every wave itself, two 16-row tiles per wave
template <int NT>
struct NndCfg {
  static constexpr int RT = 2;
  static constexpr int D = 4;
  static constexpr int WR = 4;
  static constexpr int PU = NT * 128;
};
template <int NT>
struct Tn3Cfg {
  static constexpr int D = 2;
  static constexpr int WC = 2;                 // waves along columns (64 columns each)
  static constexpr int WR = 2;                 // waves splitting the workgroup's rows
};

// gemm_nn.  A workgroup of WR waves owns 16 RT WR rows and one
// K range (its split); wave w owns rows row0 .. row0 + 16 RT.  Every wave needs
// the same panel step, so the workgroup stages it once per K step in LDS (double
// buffered, one barrier per step) and the waves read their B operands from there:
// the panel then costs one L2 read per workgroup instead of one per wave.  E runs
// through a D-deep register ring of its own.
// NORMS: the workgroup also sums the squares of the elements of E it forms (each
// exactly once: clamped rows and columns are left out; eight at a time in fp32,
// those sums in fp64) and writes the sum to nparts[workgroup tile]; in a fixed
// order, so the partials are deterministic.
// The waves-per-EU hint keeps two waves per SIMD for the wide panels and two row
// tiles (at l = 80 the variant with the norm sums otherwise needs 268 registers)
// and four for one row tile at l <= 32.
template <int NT, typename Src, bool NORMS, int RTV>
__global__ __launch_bounds__(64 * (Nn3Cfg<NT, RTV>::WR))
__attribute__((amdgpu_waves_per_eu(RTV == 1 && NT <= 2 ? 4 : 2))) void gemm_nn3_kernel(
    Src src, int64_t d, int64_t k, const uint16_t* __restrict__ Xs, int64_t kper,
    float* __restrict__ part, double* __restrict__ nparts) {
  using C = Nn3Cfg<NT, RTV>;
  constexpr int LP = 16 * NT, RT = C::RT, D = C::D, WR = C::WR, PU = C::PU, PPT = C::PPT;
  static_assert(D % 2 == 0 && WR * 64 == 256, "ring parity and the 256-thread panel staging");
  __shared__ uint4 pan[2][256 * PPT];   // rounded up to whole rounds of 256 pieces (the excess never read)
  __shared__ lvpair2 lvl2[Src::kVirtual ? 256 : 1];
  __shared__ uint4 co_lds[Src::kCoalesced ? WR * RT * kCoSlot : 1];
  fill_level_pairs(src, lvl2);            // the barrier before the first step covers it
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int g = lane >> 4, li = lane & 15;
  int tbx, tby;
  xcd_tile<false>(tbx, tby);   // the splits of one row block share their scale lines
  const int64_t row0 = (static_cast<int64_t>(tbx) * WR + w) * 16 * RT;
  const int64_t kb = static_cast<int64_t>(tby) * kper;
  const int nsteps = static_cast<int>(kper / 32);   // a multiple of D
  int64_t erow[RT];
  bool rok[RT];
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    const int64_t r = row0 + rt * 16 + li;
    erow[rt] = r < d ? r : d - 1;
    rok[rt] = r < d;
  }
  double sq = 0.0;
  const uint4* xg = reinterpret_cast<const uint4*>(Xs) + (kb / 32) * PU;
  floatx4 acc[RT][NT];
#pragma unroll
  for (int a = 0; a < RT; ++a)
#pragma unroll
    for (int b = 0; b < NT; ++b) acc[a][b] = floatx4{0.f, 0.f, 0.f, 0.f};
  typename Src::Raw8 eb[D][RT];
  float co_a[RT];   // the block scales of the piece in the LDS slot
  // at an even step: the piece of this step and the next into the wave's LDS slot
  auto co_stash = [&](int u) {
    if constexpr (Src::kCoalesced) {
      if ((u & 1) == 0) {
        wave_lds_sync();   // the last piece's reads are issued before it is overwritten
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) {
          Src::stash(eb[u][rt], co_lds + (w * RT + rt) * kCoSlot, lane);
          co_a[rt] = eb[u][rt].a;
        }
        wave_lds_sync();
      }
    }
  };
  static_assert(PPT <= 3, "at most three panel pieces per thread");
  // Two register sets (a, b, c pieces each) of staged panel steps, as plain
  // variables: the pieces past PU (PU not a multiple of 256) load a duplicate of
  // the last piece and land in the LDS padding.
  uint4 pa0, pb0, pc0, pa1, pb1, pc1;
  const int i0 = tid < PU ? tid : PU - 1;
  const int i1 = tid + 256 < PU ? tid + 256 : PU - 1;
  const int i2 = tid + 512 < PU ? tid + 512 : PU - 1;
#define LQ_PANEL_LOAD(S, J)                                                              \
  do {                                                                                   \
    const int jj_ = (J) < nsteps ? (J) : nsteps - 1;                                     \
    const uint4* src_ = xg + static_cast<int64_t>(jj_) * PU;                             \
    pa##S = src_[i0];                                                                    \
    if constexpr (PPT > 1) pb##S = src_[i1];                                             \
    if constexpr (PPT > 2) pc##S = src_[i2];                                             \
  } while (0)
#define LQ_PANEL_STORE(S, BUF)                                                           \
  do {                                                                                   \
    pan[BUF][tid] = pa##S;                                                               \
    if constexpr (PPT > 1) pan[BUF][tid + 256] = pb##S;                                  \
    if constexpr (PPT > 2) pan[BUF][tid + 512] = pc##S;                                  \
  } while (0)
  auto load_e = [&](int u, int j) {
    if constexpr (Src::kCoalesced) {
      if ((u & 1) == 0) {   // an even slot takes the piece of steps j and j + 1
        j = j < nsteps ? j : nsteps - 2;
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) eb[u][rt] = src.fetch_co(row0 + rt * 16, kb + 32 * j, d, k, lane);
      }
    } else {
      j = j < nsteps ? j : nsteps - 1;   // past the end: a harmless repeat of the last step
      const int64_t c = kb + 32 * j + 8 * g;
#pragma unroll
      for (int rt = 0; rt < RT; ++rt) eb[u][rt] = src.fetch8(erow[rt], c, k);
    }
  };
  // step j from ring slot u and LDS buffer buf
  auto compute = [&](int u, int buf, int j) {
    bf16x8 ah[RT], al[RT], bh[NT], bl[NT];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      bh[nt] = __builtin_bit_cast(bf16x8, pan[buf][(2 * nt) * 64 + lane]);
      bl[nt] = __builtin_bit_cast(bf16x8, pan[buf][(2 * nt + 1) * 64 + lane]);
    }
    if constexpr (Src::kCoalesced) co_stash(u);
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
      float x[8];
      if constexpr (Src::kCoalesced)
        src.decode8(Src::unstash(co_lds + (w * RT + rt) * kCoSlot, lane, u & 1, co_a[rt]), x, lvl2);
      else
        src.decode8(eb[u][rt], x, lvl2);
      if constexpr (NORMS) {
        // the eight squares summed in fp32 (relative error below 2^-21), then in fp64
        const int64_t nv = rok[rt] ? k - (kb + 32 * j + 8 * g) : 0;   // valid columns of the eight
        float s8 = 0.f;
        if (nv >= 8) {
#pragma unroll
          for (int i = 0; i < 8; ++i) s8 = fmaf(x[i], x[i], s8);
        } else {
#pragma unroll
          for (int i = 0; i < 8; ++i)
            if (i < nv) s8 = fmaf(x[i], x[i], s8);
        }
        sq += static_cast<double>(s8);
      }
      split8(x, ah[rt], al[rt]);
    }
    // the three products interleaved over the RT x NT accumulators
#pragma unroll
    for (int rt = 0; rt < RT; ++rt)
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) acc[rt][nt] = mfma_bf16(ah[rt], bh[nt], acc[rt][nt]);
#pragma unroll
    for (int rt = 0; rt < RT; ++rt)
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) acc[rt][nt] = mfma_bf16(ah[rt], bl[nt], acc[rt][nt]);
#pragma unroll
    for (int rt = 0; rt < RT; ++rt)
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) acc[rt][nt] = mfma_bf16(al[rt], bh[nt], acc[rt][nt]);
  };
  // Issue order: the panel of step j + 3 right after step j's barrier, then the E
  // step D ahead into the freed ring slot.  The panel is stored to LDS at the end of
  // step j + 2, where waiting for it leaves the two younger E steps (and the next
  // panel) in flight; the scheduling barriers keep this order.
  {
    LQ_PANEL_LOAD(0, 0);               // step 0 (straight to LDS below)
    uint4 qa = pa0, qb = pb0, qc = pc0;
    LQ_PANEL_LOAD(1, 1);
    LQ_PANEL_LOAD(0, 2);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int u = 0; u < D; ++u) load_e(u, u);
    __builtin_amdgcn_sched_barrier(0);
    pan[0][tid] = qa;
    if constexpr (PPT > 1) pan[0][tid + 256] = qb;
    if constexpr (PPT > 2) pan[0][tid + 512] = qc;
  }
  __syncthreads();
  const int rounds = nsteps / D;
  for (int rd = 0; rd < rounds; ++rd) {
#pragma unroll
    for (int u = 0; u < D; u += 2) {
      const int j = rd * D + u;   // even step j, then odd step j + 1
      compute(u, 0, j);
      __builtin_amdgcn_sched_barrier(0);
      LQ_PANEL_STORE(1, 1);          // the panel of step j + 1
      __syncthreads();
      LQ_PANEL_LOAD(1, j + 3);
      __builtin_amdgcn_sched_barrier(0);
      load_e(u, j + D);
      __builtin_amdgcn_sched_barrier(0);
      compute(u + 1, 1, j + 1);
      __builtin_amdgcn_sched_barrier(0);
      LQ_PANEL_STORE(0, 0);          // the panel of step j + 2
      __syncthreads();
      LQ_PANEL_LOAD(0, j + 4);
      __builtin_amdgcn_sched_barrier(0);
      load_e(u + 1, j + 1 + D);
      __builtin_amdgcn_sched_barrier(0);
    }
  }
#undef LQ_PANEL_LOAD
#undef LQ_PANEL_STORE
#pragma unroll
  for (int rt = 0; rt < RT; ++rt)
#pragma unroll
    for (int nt = 0; nt < NT; ++nt)
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int64_t row = row0 + rt * 16 + 4 * g + v;
        if (row < d) part[(static_cast<int64_t>(tby) * d + row) * LP + nt * 16 + li] = acc[rt][nt][v];
      }
  if constexpr (NORMS) {
    __shared__ double wsq[WR];
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) sq += __shfl_xor(sq, off);
    if (lane == 0) wsq[w] = sq;
    __syncthreads();
    if (tid == 0) {
      double t = 0.0;
#pragma unroll
      for (int q = 0; q < WR; ++q) t += wsq[q];
      nparts[static_cast<int64_t>(tby) * gridDim.x + tbx] = t;
    }
  }
}

// gemm_nn, panel read per wave: every wave loads its own B operands (16 bytes
// per lane and piece; the four waves of a workgroup hit the same lines) into a
// register ring beside E's, so the K loop runs without LDS staging or barriers.
// It reads the panel four times from L2 where gemm_nn3_kernel reads it once, and
// wins while the panel stays small (nn_direct).
template <int NT, typename Src, bool NORMS>
__global__ __launch_bounds__(64 * NndCfg<NT>::WR) void gemm_nnd_kernel(
    Src src, int64_t d, int64_t k, const uint16_t* __restrict__ Xs, int64_t kper,
    float* __restrict__ part, double* __restrict__ nparts) {
  using C = NndCfg<NT>;
  constexpr int LP = 16 * NT, RT = C::RT, D = C::D, WR = C::WR, PU = C::PU;
  __shared__ lvpair2 lvl2[Src::kVirtual ? 256 : 1];
  __shared__ uint4 co_lds[Src::kCoalesced ? WR * RT * kCoSlot : 1];
  if constexpr (Src::kVirtual) {
    fill_level_pairs(src, lvl2);
    __syncthreads();
  }
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int g = lane >> 4, li = lane & 15;
  int tbx, tby;
  xcd_tile<false>(tbx, tby);
  const int64_t row0 = (static_cast<int64_t>(tbx) * WR + w) * 16 * RT;
  const int64_t kb = static_cast<int64_t>(tby) * kper;
  const int nsteps = static_cast<int>(kper / 32);   // a multiple of D
  int64_t erow[RT];
  bool rok[RT];
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    const int64_t r = row0 + rt * 16 + li;
    erow[rt] = r < d ? r : d - 1;
    rok[rt] = r < d;
  }
  double sq = 0.0;
  const uint4* xg = reinterpret_cast<const uint4*>(Xs) + (kb / 32) * PU + lane;
  floatx4 acc[RT][NT];
#pragma unroll
  for (int a = 0; a < RT; ++a)
#pragma unroll
    for (int b = 0; b < NT; ++b) acc[a][b] = floatx4{0.f, 0.f, 0.f, 0.f};
  typename Src::Raw8 eb[D][RT];
  uint4 pb[D][NT][2];
  float co_a[RT];   // the block scales of the piece in the LDS slot (as in gemm_nn3_kernel)
  auto co_stash = [&](int u) {
    if constexpr (Src::kCoalesced) {
      if ((u & 1) == 0) {
        wave_lds_sync();
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) {
          Src::stash(eb[u][rt], co_lds + (w * RT + rt) * kCoSlot, lane);
          co_a[rt] = eb[u][rt].a;
        }
        wave_lds_sync();
      }
    }
  };
  auto load = [&](int u, int j) {
    if constexpr (Src::kCoalesced) {
      if ((u & 1) == 0) {
        const int jj = j < nsteps ? j : nsteps - 2;
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) eb[u][rt] = src.fetch_co(row0 + rt * 16, kb + 32 * jj, d, k, lane);
      }
    } else {
      const int jj = j < nsteps ? j : nsteps - 1;
      const int64_t c = kb + 32 * jj + 8 * g;
#pragma unroll
      for (int rt = 0; rt < RT; ++rt) eb[u][rt] = src.fetch8(erow[rt], c, k);
    }
    j = j < nsteps ? j : nsteps - 1;
#pragma unroll
    for (int nt = 0; nt < NT; ++nt)
#pragma unroll
      for (int h = 0; h < 2; ++h) pb[u][nt][h] = xg[static_cast<int64_t>(j) * PU + (2 * nt + h) * 64];
  };
  auto compute = [&](int u, int j) {
    bf16x8 ah[RT], al[RT], bh[NT], bl[NT];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      bh[nt] = __builtin_bit_cast(bf16x8, pb[u][nt][0]);
      bl[nt] = __builtin_bit_cast(bf16x8, pb[u][nt][1]);
    }
    co_stash(u);
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
      float x[8];
      if constexpr (Src::kCoalesced)
        src.decode8(Src::unstash(co_lds + (w * RT + rt) * kCoSlot, lane, u & 1, co_a[rt]), x, lvl2);
      else
        src.decode8(eb[u][rt], x, lvl2);
      if constexpr (NORMS) {
        const int64_t nv = rok[rt] ? k - (kb + 32 * j + 8 * g) : 0;
        float s8 = 0.f;
        if (nv >= 8) {
#pragma unroll
          for (int i = 0; i < 8; ++i) s8 = fmaf(x[i], x[i], s8);
        } else {
#pragma unroll
          for (int i = 0; i < 8; ++i)
            if (i < nv) s8 = fmaf(x[i], x[i], s8);
        }
        sq += static_cast<double>(s8);
      }
      split8(x, ah[rt], al[rt]);
    }
#pragma unroll
    for (int rt = 0; rt < RT; ++rt)
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) acc[rt][nt] = mfma_bf16(ah[rt], bh[nt], acc[rt][nt]);
#pragma unroll
    for (int rt = 0; rt < RT; ++rt)
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) acc[rt][nt] = mfma_bf16(ah[rt], bl[nt], acc[rt][nt]);
#pragma unroll
    for (int rt = 0; rt < RT; ++rt)
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) acc[rt][nt] = mfma_bf16(al[rt], bh[nt], acc[rt][nt]);
  };
#pragma unroll
  for (int u = 0; u < D; ++u) load(u, u);
  const int rounds = nsteps / D;
  for (int rd = 0; rd + 1 < rounds; ++rd) {
#pragma unroll
    for (int u = 0; u < D; ++u) {
      compute(u, rd * D + u);
      load(u, (rd + 1) * D + u);
      __builtin_amdgcn_sched_barrier(0);
    }
  }
#pragma unroll
  for (int u = 0; u < D; ++u) compute(u, (rounds - 1) * D + u);
#pragma unroll
  for (int rt = 0; rt < RT; ++rt)
#pragma unroll
    for (int nt = 0; nt < NT; ++nt)
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int64_t row = row0 + rt * 16 + 4 * g + v;
        if (row < d) part[(static_cast<int64_t>(tby) * d + row) * LP + nt * 16 + li] = acc[rt][nt][v];
      }
  if constexpr (NORMS) {
    __shared__ double wsq[WR];
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) sq += __shfl_xor(sq, off);
    if (lane == 0) wsq[w] = sq;
    __syncthreads();
    if (tid == 0) {
      double t = 0.0;
#pragma unroll
      for (int q = 0; q < WR; ++q) t += wsq[q];
      nparts[static_cast<int64_t>(tby) * gridDim.x + tbx] = t;
    }
  }
}

// gemm_tn.  Wave (wc, wr) owns one 64-column group (its four interleaved 16-column
// MFMA tiles jm hold columns c0 + 4 m + jm) and its share of the workgroup's rows;
// waves sharing columns are summed through LDS at the end.  Row steps of 32: lane (li, g) loads rows
// split_row(j, g, e, paired) of its range (eight runs of its four columns), and
// tile jm's A operand is component jm of those eight.
template <int NT, typename Src, int LMJ>
__global__ __launch_bounds__(64 * Tn3Cfg<NT>::WC * Tn3Cfg<NT>::WR) void gemm_tn3_kernel(
    Src src, int64_t d, int64_t k, const uint16_t* __restrict__ Ys, int64_t rper,
    float* __restrict__ part, CholJob job) {
  using C = Tn3Cfg<NT>;
  constexpr int LP = 16 * NT, D = C::D, WC = C::WC, WR = C::WR;
  constexpr int kRedFloats = (WR > 1 ? WR - 1 : 1) * WC * 64 * LP;
  constexpr int kJobDoubles = LMJ > 0 ? 5 * (LMJ * (LMJ + 1) / 2) + 64 : 1;
  constexpr int kLdsBytes = 4 * kRedFloats > 8 * kJobDoubles ? 4 * kRedFloats : 8 * kJobDoubles;
  __shared__ __align__(16) char lds_raw[kLdsBytes];
  float* red = reinterpret_cast<float*>(lds_raw);
  int tbx, tby;
  xcd_tile<true>(tbx, tby);   // neighbouring column blocks share their code and scale lines
  // LMJ > 0: the extra last column of workgroups carries a Cholesky job; its
  // row 0 sums the Gram partials of Y and factors them (X = R^-1 for the
  // reduction that follows this product), l <= LMJ.  The plan leaves a CU free
  // for it.
  if constexpr (LMJ > 0) {
    if (tbx == static_cast<int>(gridDim.x) - 1) {
      if (tby == 0) {
        double* lds = reinterpret_cast<double*>(lds_raw);
        const double* gram = gram_sum_block<LMJ>(job.parts, job.P, job.l, lds);
        if (threadIdx.x < 64) chol_inv_to<LMJ>(gram, job.l, job.Xinv, lds);
      }
      return;
    }
  }
  __shared__ lvpair2 lvl2[Src::kVirtual ? 256 : 1];
  if constexpr (Src::kVirtual) {
    fill_level_pairs(src, lvl2);
    __syncthreads();
  }
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, wc = w % WC, wr = w / WC;
  const int g = lane >> 4, li = lane & 15;
  const int64_t bx = tbx, by = tby;   // column block, row split
  const int64_t c0 = (bx * WC + wc) * 64;
  const int64_t cl = c0 + 4 * li;
  const int64_t rw = rper / WR;
  const int64_t rb = by * rper + wr * rw;
  const int nsteps = static_cast<int>(rw / 32);   // a multiple of D
  const uint4* yp = reinterpret_cast<const uint4*>(Ys) + (rb / 32) * NT * 128 + lane;
  floatx4 acc[4][NT];
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int b = 0; b < NT; ++b) acc[a][b] = floatx4{0.f, 0.f, 0.f, 0.f};
  typename Src::Raw4 eb[D][8];
  uint4 yb[D][NT][2];
  auto load = [&](int u, int j) {
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      int64_t r = rb + split_row(j, g, e, true);
      r = r < d ? r : d - 1;
      eb[u][e] = src.fetch4(r, cl, k);
    }
#pragma unroll
    for (int nt = 0; nt < NT; ++nt)
#pragma unroll
      for (int h = 0; h < 2; ++h) yb[u][nt][h] = yp[((static_cast<int64_t>(j) * NT + nt) * 2 + h) * 64];
  };
  auto compute = [&](int u) {
    float4 ev[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) ev[e] = src.decode4(eb[u][e], lvl2);
    bf16x8 bh[NT], bl[NT];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      bh[nt] = __builtin_bit_cast(bf16x8, yb[u][nt][0]);
      bl[nt] = __builtin_bit_cast(bf16x8, yb[u][nt][1]);
    }
#pragma unroll
    for (int jm = 0; jm < 4; ++jm) {
      const float x[8] = {comp(ev[0], jm), comp(ev[1], jm), comp(ev[2], jm), comp(ev[3], jm),
                          comp(ev[4], jm), comp(ev[5], jm), comp(ev[6], jm), comp(ev[7], jm)};
      bf16x8 ah, al;
      split8(x, ah, al);
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) acc[jm][nt] = mfma_bf16(ah, bh[nt], acc[jm][nt]);
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) acc[jm][nt] = mfma_bf16(ah, bl[nt], acc[jm][nt]);
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) acc[jm][nt] = mfma_bf16(al, bh[nt], acc[jm][nt]);
    }
  };
#pragma unroll
  for (int u = 0; u < D; ++u) load(u, u);
  const int rounds = nsteps / D;
  for (int rd = 0; rd + 1 < rounds; ++rd) {
#pragma unroll
    for (int u = 0; u < D; ++u) {
      compute(u);
      load(u, (rd + 1) * D + u);
      __builtin_amdgcn_sched_barrier(0);
    }
  }
#pragma unroll
  for (int u = 0; u < D; ++u) compute(u);
  // lane (li, g), tile jm, component v holds column c0 + 4 (4 g + v) + jm, output n = 16 nt + li
  if (WR > 1) {
    if (wr > 0) {
#pragma unroll
      for (int jm = 0; jm < 4; ++jm)
#pragma unroll
        for (int nt = 0; nt < NT; ++nt)
#pragma unroll
          for (int v = 0; v < 4; ++v)
            red[(((wr - 1) * WC + wc) * 64 + 4 * (4 * g + v) + jm) * LP + nt * 16 + li] = acc[jm][nt][v];
    }
    __syncthreads();
    if (wr > 0) return;
#pragma unroll
    for (int q = 1; q < WR; ++q)
#pragma unroll
      for (int jm = 0; jm < 4; ++jm)
#pragma unroll
        for (int nt = 0; nt < NT; ++nt)
#pragma unroll
          for (int v = 0; v < 4; ++v)
            acc[jm][nt][v] += red[(((q - 1) * WC + wc) * 64 + 4 * (4 * g + v) + jm) * LP + nt * 16 + li];
  }
#pragma unroll
  for (int jm = 0; jm < 4; ++jm)
#pragma unroll
    for (int nt = 0; nt < NT; ++nt)
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int64_t col = c0 + 4 * (4 * g + v) + jm;
        if (col < k) part[(by * k + col) * LP + nt * 16 + li] = acc[jm][nt][v];
      }
}

template <int NT>
GemmShape shape_typed(bool transposed, int64_t d, int64_t k) {
  if (transposed) {
    using C = Tn3Cfg<NT>;
    return GemmShape{64 * C::WC, 32 * C::D * C::WR};
  }
  if (nn_direct(NT, k)) {
    using C = NndCfg<NT>;
    return GemmShape{16 * C::RT * C::WR, 32 * C::D};
  }
  if (nn_staged_rt(NT, d, k) == 2) {
    using C = Nn3Cfg<NT, 2>;
    return GemmShape{16 * C::RT * C::WR, 32 * C::D};
  }
  using C = Nn3Cfg<NT, 1>;
  return GemmShape{16 * C::RT * C::WR, 32 * C::D};
}

template <int NT, typename Src>
void gemm_launch(bool transposed, const Src& src, int64_t d, int64_t k, const uint16_t* panel, const SvdPlan& pl,
                 float* part, const CholJob& job, hipStream_t s, double* nparts) {
  if constexpr (Src::kCoalesced) {
    if (transposed) return;   // never asked: gemm_typed takes this source for E P only
  } else if (transposed) {
    constexpr int threads = 64 * Tn3Cfg<NT>::WC * Tn3Cfg<NT>::WR;
    const dim3 grid(pl.tn_col_blocks + (job.parts != nullptr ? 1 : 0), pl.tn_splits);
#define LQ_TN3(LMJ)                                                                                                   \
  LQ_LAUNCH("gemm_tn", (gemm_tn3_kernel<NT, Src, LMJ>), grid, dim3(threads), 0, s, src, d, k, panel, pl.tn_rper, part, \
            job)
    // register tile of the ride-along Cholesky (l <= 32 only): the smallest of 16 / 24 / 32 rows that holds l
    const int lmj = job.parts == nullptr ? 0 : (job.l <= 16 ? 16 : (job.l <= 24 ? 24 : 32));
    if constexpr (NT <= 2) {
      if (lmj == 16) LQ_TN3(16); else if (lmj == 24) LQ_TN3(24); else if (lmj) LQ_TN3(32); else LQ_TN3(0);
    } else {
      LQ_TN3(0);
    }
#undef LQ_TN3
    return;
  }
  constexpr int threads = 64 * Nn3Cfg<NT>::WR;
  static_assert(NndCfg<NT>::WR == Nn3Cfg<NT>::WR && Nn3Cfg<NT, 2>::WR == Nn3Cfg<NT>::WR, "one workgroup size");
  const bool two = nn_staged_rt(NT, d, k) == 2;
  const dim3 grid(pl.nn_row_blocks, pl.nn_splits);
  const bool direct = nn_direct(NT, k);
  if (direct && nparts != nullptr)
    LQ_LAUNCH("gemm_nn", (gemm_nnd_kernel<NT, Src, true>), grid, dim3(threads), 0, s, src, d, k, panel, pl.nn_kper, part,
              nparts);
  else if (direct)
    LQ_LAUNCH("gemm_nn", (gemm_nnd_kernel<NT, Src, false>), grid, dim3(threads), 0, s, src, d, k, panel, pl.nn_kper,
              part, nparts);
  else if (two && nparts != nullptr)
    LQ_LAUNCH("gemm_nn", (gemm_nn3_kernel<NT, Src, true, 2>), grid, dim3(threads), 0, s, src, d, k, panel, pl.nn_kper,
              part, nparts);
  else if (two)
    LQ_LAUNCH("gemm_nn", (gemm_nn3_kernel<NT, Src, false, 2>), grid, dim3(threads), 0, s, src, d, k, panel, pl.nn_kper,
              part, nparts);
  else if (nparts != nullptr)
    LQ_LAUNCH("gemm_nn", (gemm_nn3_kernel<NT, Src, true, 1>), grid, dim3(threads), 0, s, src, d, k, panel, pl.nn_kper,
              part, nparts);
  else
    LQ_LAUNCH("gemm_nn", (gemm_nn3_kernel<NT, Src, false, 1>), grid, dim3(threads), 0, s, src, d, k, panel, pl.nn_kper,
              part, nparts);
}

template <int NT>
void gemm_typed(bool transposed, const float* E, int64_t d, int64_t k, const uint16_t* panel, const SvdPlan& pl,
                float* part, const CholJob& job, hipStream_t s, const VirtualE* ve, double* np) {
  const bool vec = (k & 3) == 0 && k >= 4;
  const bool vec8 = vec && k >= 8;
  if (ve != nullptr && ve->w_bf16 && !transposed && k % 64 == 0)
    gemm_launch<NT>(false, FormedCo{FormedE<true>{*ve}}, d, k, panel, pl, part, job, s, np);
  else if (ve != nullptr && ve->w_bf16) gemm_launch<NT>(transposed, FormedE<true>{*ve}, d, k, panel, pl, part, job, s, np);
  else if (ve != nullptr) gemm_launch<NT>(transposed, FormedE<false>{*ve}, d, k, panel, pl, part, job, s, np);
  else if (vec8) gemm_launch<NT>(transposed, StoredE<true>{E}, d, k, panel, pl, part, job, s, np);
  else gemm_launch<NT>(transposed, StoredE<false>{E}, d, k, panel, pl, part, job, s, np);
}

}  // namespace

GemmShape gemm_shape(bool transposed, int nt, int64_t d, int64_t k) {
  switch (nt) {
    case 1: return shape_typed<1>(transposed, d, k);
    case 2: return shape_typed<2>(transposed, d, k);
    case 3: return shape_typed<3>(transposed, d, k);
    case 4: return shape_typed<4>(transposed, d, k);
    default: return shape_typed<5>(transposed, d, k);
  }
}

void launch_gemm(bool transposed, const float* E, int64_t d, int64_t k, const uint16_t* panel, const SvdPlan& pl,
                 float* part, const CholJob& job, hipStream_t s, const VirtualE* ve, double* nparts) {
  const CholJob none{nullptr, 0, 0, nullptr};
  const CholJob& j = (transposed && pl.nt <= 2) ? job : none;
  double* np = transposed ? nullptr : nparts;
  switch (pl.nt) {
    case 1: gemm_typed<1>(transposed, E, d, k, panel, pl, part, j, s, ve, np); break;
    case 2: gemm_typed<2>(transposed, E, d, k, panel, pl, part, j, s, ve, np); break;
    case 3: gemm_typed<3>(transposed, E, d, k, panel, pl, part, j, s, ve, np); break;
    case 4: gemm_typed<4>(transposed, E, d, k, panel, pl, part, j, s, ve, np); break;
    default: gemm_typed<5>(transposed, E, d, k, panel, pl, part, j, s, ve, np); break;
  }
}

}  // namespace loftq
