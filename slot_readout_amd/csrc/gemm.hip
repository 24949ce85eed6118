// MFMA-tiled "NT" GEMMs (both operands K-contiguous) for gfx950, with the
// prologues and epilogues of the denoise step fused in:
//   qkv_kernel     q,k,v = (E[ids] + sc_in) [Wq;Wk;Wv]^T      (embedding gather fused)
//   oproj_kernel   h = x + o Wo^T                              (residual fused)
//   lmhead_kernel  l = s_i h E^T, per-(row, vocab tile) max / sum e^(l-m) /
//                  sum e^(l-m)(l-m) / argmax, optional p~ = e^(l - m_tile)
//   scgemm_kernel  sc = sum_v p_v E_v over a vocabulary range (split-K)
//
// One workgroup computes a BM x BN tile with WGM x WGN waves; each wave owns a
// (BM/WGM) x (BN/WGN) block of 16x16 MFMA tiles.  Operand tiles stream through
// double-buffered LDS (16-byte global loads -> registers -> LDS, one barrier per
// K step); fragments are read from LDS with 16-byte (bf16) or 4-byte (fp32)
// reads.  Accumulation is fp32.
#include <algorithm>
#include <type_traits>

#include "common.h"
#include "kernels.h"

namespace dg {

template <typename T> struct BKOf;
template <> struct BKOf<bf16> { static constexpr int v = 32; };
template <> struct BKOf<float> { static constexpr int v = 16; };

template <typename T, int BM, int BN, int WGM, int WGN, int PF = 1, int BK_ = BKOf<T>::v>
struct Gemm {
  static constexpr int BK = BK_;
  static constexpr int NW = WGM * WGN;
  static constexpr int NT = NW * WAVE;
  static constexpr int VEC = 16 / sizeof(T);
  static constexpr int CPR = BK / VEC;      // 16-byte chunks per tile row
  // LDS rows.  The fragment reads (16 rows x 4 chunks of 16 bytes per
  // instruction) are free of bank conflicts on gfx950 for 128-byte rows whose
  // chunks are XOR-swizzled by (row & 7), and for 64-byte rows padded to 96
  // bytes; a 16-byte pad on 128-byte rows costs 2x, no pad and no swizzle 4x
  // (SQ_LDS_BANK_CONFLICT).  Longer rows swizzle over all their chunks.  fp32
  // tiles keep a 16-byte pad.
  static constexpr bool SWZ = sizeof(T) == 2 && BK >= 64;
  static constexpr int PITCH = SWZ ? BK : (sizeof(T) == 2 && BK == 32 ? 48 : BK + VEC);
  __device__ static inline int chunk_at(int row, int c) { return SWZ ? c ^ (row & (CPR - 1)) : c; }
  static constexpr int AI = BM * CPR / NT;  // A chunks per thread per K step
  static constexpr int BI = BN * CPR / NT;
  static constexpr int WM = BM / WGM, WN = BN / WGN;
  static constexpr int TM = WM / 16, TN = WN / 16;
  static constexpr int LDS_BYTES = 2 * (BM + BN) * PITCH * (int)sizeof(T);
  static_assert(BM * CPR % NT == 0 && BN * CPR % NT == 0, "tile/thread mismatch");
  static_assert(WM % 16 == 0 && WN % 16 == 0, "wave tile must be 16-aligned");
  static_assert(PF >= 1 && PF <= 4, "prefetch depth");
  using MF = Mfma<T>;
  using frag = typename MF::frag;

  __device__ static inline int a_row(int it) { return (it * NT + (int)threadIdx.x) / CPR; }
  __device__ static inline int a_kc(int it) { return (it * NT + (int)threadIdx.x) % CPR; }

  // acc += A[rows of tile, kbeg:kend] * B[rows of tile, kbeg:kend]^T
  //
  // Global loads run PF K-steps ahead of the MFMAs through a ring of PF
  // register stages; LDS is double-buffered with one barrier per K step.  The
  // K loop is unrolled by PF so every ring index is a compile-time constant.
  template <class AL, class BL>
  __device__ static void run(char *smem, const AL &al, const BL &bl, int kbeg, int kend,
                             f32x4 (&acc)[TM][TN]) {
    T *lds = reinterpret_cast<T *>(smem);
    const int t = threadIdx.x, lane = t & 63, w = t >> 6;
    const int wm = w / WGN, wn = w % WGN;
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j) acc[i][j] = zero4();
    const int nk = (kend - kbeg) / BK;
    if (nk <= 0) return;
    using RA = typename AL::Raw;
    using RB = typename BL::Raw;
    RA ra[PF][AI];
    RB rb[PF][BI];
    // issue the global loads of step kt; nothing consumes them until sstore
    auto gload = [&](int kt, RA (&xa)[AI], RB (&xb)[BI]) {
      const int k0 = kbeg + kt * BK;
#pragma unroll
      for (int it = 0; it < AI; ++it) xa[it] = al.load(it, k0 + a_kc(it) * VEC);
#pragma unroll
      for (int it = 0; it < BI; ++it) xb[it] = bl.load(it, k0 + a_kc(it) * VEC);
    };
    // finish (mask / transform) the loaded chunks and write them to LDS
    auto sstore = [&](int buf, const RA (&xa)[AI], const RB (&xb)[BI]) {
      T *As = lds + buf * (BM + BN) * PITCH;
      T *Bs = As + BM * PITCH;
#pragma unroll
      for (int it = 0; it < AI; ++it)
        *reinterpret_cast<uint4 *>(As + a_row(it) * PITCH + chunk_at(a_row(it), a_kc(it)) * VEC) =
            al.finish(it, xa[it]);
#pragma unroll
      for (int it = 0; it < BI; ++it)
        *reinterpret_cast<uint4 *>(Bs + a_row(it) * PITCH + chunk_at(a_row(it), a_kc(it)) * VEC) =
            bl.finish(it, xb[it]);
    };
    auto compute = [&](int buf) {
      const T *As = lds + buf * (BM + BN) * PITCH;
      const T *Bs = As + BM * PITCH;
#pragma unroll
      for (int ks = 0; ks < BK / MF::KI; ++ks) {
        frag a[TM], b[TN];
        const int kk = ks * MF::KI + (lane >> 4) * MF::KPL;
        // rows differ from (lane & 15) by multiples of 16, so the swizzle
        // depends on the lane only
        const int ko = SWZ ? chunk_at(lane & 15, kk / VEC) * VEC : kk;
        static_assert(!SWZ || CPR <= 16, "swizzle assumes rows of at most 16 chunks");
#pragma unroll
        for (int i = 0; i < TM; ++i)
          a[i] = *reinterpret_cast<const frag *>(As + (wm * WM + i * 16 + (lane & 15)) * PITCH + ko);
#pragma unroll
        for (int j = 0; j < TN; ++j)
          b[j] = *reinterpret_cast<const frag *>(Bs + (wn * WN + j * 16 + (lane & 15)) * PITCH + ko);
#pragma unroll
        for (int i = 0; i < TM; ++i)
#pragma unroll
          for (int j = 0; j < TN; ++j) acc[i][j] = MF::mma(a[i], b[j], acc[i][j]);
      }
    };
#pragma unroll
    for (int s = 0; s < PF; ++s) gload(s < nk ? s : nk - 1, ra[s], rb[s]);
    sstore(0, ra[0], rb[0]);
    __syncthreads();
    // Main loop: whole groups of PF steps with no conditional loads, so the
    // loads retire in issue order and each store waits only for its own ring
    // slot (a load behind a branch makes the compiler drain every load in
    // flight).  Ring slot j holds step kt, already in LDS: it is refilled with
    // step kt+PF (past the end: the last step again, never used).  Scheduling
    // fences keep the order loads -> MFMAs -> finish/store, so the conversion
    // of freshly loaded data is not hoisted next to the loads.
    int k0 = 0;
    for (; k0 + PF <= nk; k0 += PF) {
#pragma unroll
      for (int j = 0; j < PF; ++j) {
        const int kt = k0 + j;
        gload(kt + PF < nk ? kt + PF : nk - 1, ra[j], rb[j]);
        __builtin_amdgcn_sched_barrier(0);
        compute(kt & 1);
        __builtin_amdgcn_sched_barrier(0);
        sstore((kt + 1) & 1, ra[(j + 1) % PF], rb[(j + 1) % PF]);
        __syncthreads();
      }
    }
    // the last nk - k0 < PF steps, already in their ring slots
#pragma unroll
    for (int j = 0; j < PF - 1; ++j) {
      const int kt = k0 + j;
      if (kt < nk) {
        compute(kt & 1);
        __builtin_amdgcn_sched_barrier(0);
        if (kt + 1 < nk) sstore((kt + 1) & 1, ra[(j + 1) % PF], rb[(j + 1) % PF]);
        __syncthreads();
      }
    }
  }
};

// ---------------------------------------------------------------------------
// operand loaders: fetch(it, k) returns the 16-byte chunk at column k of the
// row this thread loads in chunk slot `it`.  They are branch-free: a row outside
// the matrix points at a valid row and its chunk is replaced by zeros with a
// select, so no load sits behind divergent control flow.
// ---------------------------------------------------------------------------
template <typename T> __device__ inline void store4(T *p, f32x4 v);
template <> __device__ inline void store4<float>(float *p, f32x4 v) {
  *reinterpret_cast<f32x4 *>(p) = v;
}
template <> __device__ inline void store4<bf16>(bf16 *p, f32x4 v) {
  typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
  bf16x4 b;
#pragma unroll
  for (int r = 0; r < 4; ++r) b[r] = (bf16)v[r];
  *reinterpret_cast<bf16x4 *>(p) = b;
}

// Makes a loaded value opaque at this point: uses of it cannot be hoisted
// above, so the wait for the load lands here (at the LDS store), not next to
// the load.
__device__ inline void pin(uint4 &v) {
  asm volatile("" : "+v"(v.x), "+v"(v.y), "+v"(v.z), "+v"(v.w));
}
__device__ inline void pin(float &v) { asm volatile("" : "+v"(v)); }

__device__ inline uint4 keep_if(uint4 v, bool live) {
  return live ? v : uint4{0, 0, 0, 0};
}

typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
__device__ inline uint4 to_uint4(u32x4 v) { return uint4{v.x, v.y, v.z, v.w}; }

template <typename T, int N> struct RowLoader {
  using Raw = u32x4;
  const T *p[N];     // always a dereferenceable row
  bool live[N];
  __device__ inline void set(int it, const T *row, bool ok, const T *fallback) {
    p[it] = ok ? row : fallback;
    live[it] = ok;
  }
  __device__ inline Raw load(int it, int k) const {
    return *reinterpret_cast<const u32x4 *>(p[it] + k);
  }
  __device__ inline uint4 finish(int it, const Raw &r) const {
    uint4 v = to_uint4(r);
    pin(v);
    return keep_if(v, live[it]);
  }
};

// Rows of a matrix read twice over K: column k of a row of K columns for
// k < K, and column k - K for K <= k < 2K (the weight side of a product whose
// other operand is split into hi and lo halves along K).
template <typename T, int N> struct WrapRowLoader {
  using Raw = u32x4;
  const T *p[N];
  bool live[N];
  int K;
  __device__ inline void set(int it, const T *row, bool ok, const T *fallback) {
    p[it] = ok ? row : fallback;
    live[it] = ok;
  }
  __device__ inline Raw load(int it, int k) const {
    return *reinterpret_cast<const u32x4 *>(p[it] + (k < K ? k : k - K));
  }
  __device__ inline uint4 finish(int it, const Raw &r) const {
    uint4 v = to_uint4(r);
    pin(v);
    return keep_if(v, live[it]);
  }
};

// bf16 operand taken from fp32 rows of K columns as two halves along K: for
// k < K the chunk holds hi = bf16(x[k..k+7]), for K <= k < 2K it holds
// lo = bf16(x - hi) of columns k - K.  A product over 2K columns against a
// WrapRowLoader operand then sums hi.w + lo.w = x.w up to 2^-16 of x.
template <int N> struct F32SplitLoader {
  struct Raw { u32x4 a, b; int lo; };
  const float *p[N];
  bool live[N];
  int K;
  __device__ inline void set(int it, const float *row, bool ok, const float *fallback) {
    p[it] = ok ? row : fallback;
    live[it] = ok;
  }
  __device__ inline Raw load(int it, int k) const {
    Raw r;
    r.lo = k >= K;
    const float *q = p[it] + (k < K ? k : k - K);
    r.a = *reinterpret_cast<const u32x4 *>(q);
    r.b = *reinterpret_cast<const u32x4 *>(q + 4);
    return r;
  }
  __device__ inline uint4 finish(int it, const Raw &r) const {
    uint4 ua = to_uint4(r.a), ub = to_uint4(r.b);
    pin(ua);
    pin(ub);
    const float x[8] = {__uint_as_float(ua.x), __uint_as_float(ua.y), __uint_as_float(ua.z),
                        __uint_as_float(ua.w), __uint_as_float(ub.x), __uint_as_float(ub.y),
                        __uint_as_float(ub.z), __uint_as_float(ub.w)};
    Chunk<bf16> c;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const bf16 hi = (bf16)x[e];
      c.v[e] = r.lo ? (bf16)(x[e] - (float)hi) : hi;
    }
    return keep_if(c.u, live[it]);
  }
};

// h as two bf16 halves of one row: hi = bf16(h) at column c, lo = bf16(h - hi)
// at column c + d
__device__ inline void store_split(bf16 *row, int d, int c, float h) {
  const bf16 hi = (bf16)h;
  row[c] = hi;
  row[d + c] = (bf16)(h - (float)hi);
}

// Rows of a matrix stored in blocks of BR rows x 32 columns (block after block
// along K): p is the row's first element in the first block, and column k sits
// k / 32 blocks further.
template <typename T, int N, int BR> struct BlockedRowLoader {
  using Raw = u32x4;
  const T *p[N];
  bool live[N];
  __device__ inline void set(int it, const T *row, bool ok, const T *fallback) {
    p[it] = ok ? row : fallback;
    live[it] = ok;
  }
  __device__ inline Raw load(int it, int k) const {
    return *reinterpret_cast<const u32x4 *>(p[it] + (int64_t)(k >> 5) * (BR * 32) + (k & 31));
  }
  __device__ inline uint4 finish(int it, const Raw &r) const {
    uint4 v = to_uint4(r);
    pin(v);
    return keep_if(v, live[it]);
  }
};

// Rows of an e4m3 (FP8) matrix: each 8-byte load holds the 8 codes of a chunk,
// decoded to bf16 (exactly: every e4m3 value is a bf16 value) at the LDS store.
// The per-row power-of-two scale is applied to the GEMM result.
template <int N> struct Fp8RowLoader {
  using Raw = uint2;
  const uint8_t *p[N];
  bool live[N];
  __device__ inline void set(int it, const uint8_t *row, bool ok, const uint8_t *fallback) {
    p[it] = ok ? row : fallback;
    live[it] = ok;
  }
  __device__ inline Raw load(int it, int k) const {
    return *reinterpret_cast<const uint2 *>(p[it] + k);
  }
  __device__ inline uint4 finish(int it, const Raw &r) const {
    uint2 c = r;
    asm volatile("" : "+v"(c.x), "+v"(c.y));
    uint4 v;
    v.x = __builtin_bit_cast(unsigned, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(c.x, 1.f, false));
    v.y = __builtin_bit_cast(unsigned, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(c.x, 1.f, true));
    v.z = __builtin_bit_cast(unsigned, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(c.y, 1.f, false));
    v.w = __builtin_bit_cast(unsigned, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(c.y, 1.f, true));
    return keep_if(v, live[it]);
  }
};

// x = E[id] + sc_in, rounded to T (SC: sc_in present for the whole launch; a
// compile-time switch, so no load sits behind a branch)
template <typename T, int N, bool SC> struct GatherLoader {
  struct Raw { u32x4 e, s; };
  const T *e[N];
  const T *s[N];
  bool live[N];
  __device__ inline Raw load(int it, int k) const {
    Raw r;
    r.e = *reinterpret_cast<const u32x4 *>(e[it] + k);
    if constexpr (SC) r.s = *reinterpret_cast<const u32x4 *>(s[it] + k);
    else r.s = u32x4{0, 0, 0, 0};
    return r;
  }
  __device__ inline uint4 finish(int it, const Raw &r) const {
    Chunk<T> a;
    a.u = to_uint4(r.e);
    pin(a.u);
    if constexpr (SC) {
      Chunk<T> b;
      b.u = to_uint4(r.s);
      pin(b.u);
#pragma unroll
      for (int i = 0; i < Chunk<T>::N; ++i) a.v[i] = from_f<T>(to_f(a.v[i]) + to_f(b.v[i]));
    }
    return keep_if(a.u, live[it]);
  }
};

// p = p~ * 2^-shift[row][k / VTILE] (the 1/Z of the row is applied to the
// output).  p~ >= 0, so the scaling is a saturating subtract on the exponent
// field: exact, and values that would leave the normal range become 0 (or,
// at the boundary, a subnormal below 2^-126).
__device__ inline uint4 pow2_down(uint4 v, int sh, bf16) {
  typedef unsigned short us8 __attribute__((ext_vector_type(8)));
  const us8 x = __builtin_bit_cast(us8, v);
  const us8 d = (us8)(unsigned short)((sh < 255 ? sh : 255) << 7);
  return __builtin_bit_cast(uint4, __builtin_elementwise_sub_sat(x, d));
}
__device__ inline uint4 pow2_down(uint4 v, int sh, float) {
  const u32x4 x = __builtin_bit_cast(u32x4, v);
  const u32x4 d = (u32x4)((unsigned)(sh < 255 ? sh : 255) << 23);
  return __builtin_bit_cast(uint4, __builtin_elementwise_sub_sat(x, d));
}

// BLK: p~ stored in blocks of 256 rows x 32 columns; p is then the row's first
// element in its first block and column k sits k / 32 blocks further
template <typename T, int N, bool BLK> struct ShiftedRowLoader {
  struct Raw { u32x4 p; int sh; };
  const T *p[N];
  const int32_t *sh[N];
  bool live[N];
  __device__ inline Raw load(int it, int k) const {
    Raw r;
    r.p = *reinterpret_cast<const u32x4 *>(p[it] + (BLK ? (int64_t)(k >> 5) * 8192 + (k & 31) : k));
    r.sh = sh[it][k / VTILE];
    return r;
  }
  __device__ inline uint4 finish(int it, const Raw &r) const {
    uint4 v = to_uint4(r.p);
    pin(v);
    int s = r.sh;
    asm volatile("" : "+v"(s));
    return keep_if(pow2_down(v, s, T{}), live[it]);
  }
};

__device__ inline bool tile_active(const int32_t *active, int64_t m0, int64_t rows, int64_t M,
                                   int C) {
  if (!active) return true;
  const int64_t m1 = (m0 + rows < M ? m0 + rows : M) - 1;
  for (int64_t c = m0 / C; c <= m1 / C; ++c)
    if (active[c]) return true;
  return false;
}

// Self-conditioning GEMM: d tiles of 256 and about one workgroup per CU.
// Keeping whole vocabulary ranges on one XCD (kScGroup, register-staged
// kernel) cuts the p~ re-reads that reach HBM by ~40% but leaves CUs idle at
// d = 2816 (11 tiles per range), and measured slower (555-618 us against
// 481 us), so it is off.  The direct-to-LDS kernel instead deals consecutive
// (range, tile) items to each XCD, which keeps a range's tiles on one or two
// XCDs with every CU busy.  (kScTileD and kScGroup sit in kernels.h, beside
// the split planning that reads them.)

// Split-K partial of one tile: element (row, col) of the tile's accumulators to
// dst[row * ld + col] for row < M, col < ncols (fp32, no epilogue)
template <class G, int WGN>
__device__ inline void store_partial(float *dst, int64_t ld, const f32x4 (&acc)[G::TM][G::TN],
                                     int64_t m0, int64_t c0, int64_t M, int64_t ncols) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int wm = w / WGN, wn = w % WGN;
#pragma unroll
  for (int j = 0; j < G::TN; ++j) {
    const int64_t col = c0 + wn * G::WN + j * 16 + (lane & 15);
    if (col >= ncols) continue;
#pragma unroll
    for (int i = 0; i < G::TM; ++i)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int64_t row = m0 + wm * G::WM + i * 16 + 4 * (lane >> 4) + r;
        if (row < M) dst[row * ld + col] = acc[i][j][r];
      }
  }
}

// Sum of the ns split-K partials of 4 consecutive outputs, in split order (the
// result does not depend on which split finished first).  The loads of up to 8
// splits are issued together, so the reduce waits about one memory latency per
// 8 splits rather than one per split.
__device__ inline float4 sum_partials(const float *part, int64_t split_stride, int64_t off, int ns) {
  float4 s = make_float4(0.f, 0.f, 0.f, 0.f);
  for (int k0 = 0; k0 < ns; k0 += 8) {
    float4 t[8];
#pragma unroll
    for (int j = 0; j < 8; ++j)
      if (k0 + j < ns) t[j] = *reinterpret_cast<const float4 *>(part + (k0 + j) * split_stride + off);
#pragma unroll
    for (int j = 0; j < 8; ++j)
      if (k0 + j < ns) {
        s.x += t[j].x;
        s.y += t[j].y;
        s.z += t[j].z;
        s.w += t[j].w;
      }
  }
  return s;
}

// Split-K reduce of the q,k,v projection: 4 outputs per thread, the same
// epilogue as the unsplit kernel (q scale, k/v row map).  Column ranges are
// multiples of 64, so 4 consecutive outputs never straddle q, k and v.
// Split launches use 64-row tiles; rows of a tile no active canvas touches
// are left unwritten, as the unsplit kernel leaves them.
template <typename T>
__global__ __launch_bounds__(256) void qkv_reduce_kernel(QkvArgs a) {
  const int64_t nc = a.col1 - a.col0, n4 = nc / 4;
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= a.M * n4) return;
  const int64_t row = i / n4;
  const int c4 = (int)(i - row * n4) * 4;
  if (!tile_active(a.active, row / 64 * 64, 64, a.M, a.C)) return;
  const float4 s = sum_partials(a.part, a.M * nc, row * nc + c4, a.ksplit);
  const int col = a.col0 + c4;
  T *base;
  int ld, c;
  float sc = 1.f;
  if (col < a.nq) { base = static_cast<T *>(a.q); ld = a.nq; c = col; sc = a.q_scale; }
  else if (col < a.nq + a.nkv) { base = static_cast<T *>(a.k); ld = a.nkv; c = col - a.nq; }
  else { base = static_cast<T *>(a.v); ld = a.nkv; c = col - a.nq - a.nkv; }
  int64_t orow = row;
  if (col >= a.nq && a.kv_row) orow = a.kv_row[row];
  else if (col >= a.nq && a.kv_cmul > 1) orow = (row / a.C) * a.kv_cmul * a.C + row % a.C;
  if (orow < 0) return;
  const int ncp = col >= a.nq ? a.kv_copies : 0;
  for (int cp = 0; cp <= ncp; ++cp) {
    T *o = base + (orow + (int64_t)cp * a.C) * ld + c;
    o[0] = from_f<T>(s.x * sc);
    o[1] = from_f<T>(s.y * sc);
    o[2] = from_f<T>(s.z * sc);
    o[3] = from_f<T>(s.w * sc);
  }
}

// Split-K reduce of the output projection: h = x + sum of partials, with x
// recomputed from the embedding as in the unsplit kernel
template <typename T>
__global__ __launch_bounds__(256) void oproj_reduce_kernel(OprojArgs a) {
  const int n4 = a.d / 4;
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= a.M * n4) return;
  const int64_t row = i / n4;
  const int c4 = (int)(i - row * n4) * 4;
  if (!tile_active(a.active, row / 64 * 64, 64, a.M, a.C)) return;
  const float4 s = sum_partials(a.part, a.M * a.d, row * a.d + c4, a.ksplit);
  const float acc[4] = {s.x, s.y, s.z, s.w};
  const int id = a.ids[row];
  const bool ok = id >= 0 && id < a.vocab;
  const T *E = static_cast<const T *>(a.embed) + (ok ? (int64_t)id * a.d : 0);
  const T *sc = static_cast<const T *>(a.sc_in);
  if constexpr (std::is_same<T, bf16>::value) {
    if (a.prec) {   // hi | lo halves of a [M, 2d] row
      bf16 *h2 = static_cast<bf16 *>(a.h) + row * 2 * a.d;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        float x = ok ? to_f(E[c4 + e]) : 0.f;
        if (sc) x += to_f(sc[row * a.d + c4 + e]);
        store_split(h2, a.d, c4 + e, acc[e] + x);
      }
      return;
    }
  }
  T *h = static_cast<T *>(a.h) + row * a.d + c4;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    float x = ok ? to_f(E[c4 + e]) : 0.f;
    if (sc) x += to_f(sc[row * a.d + c4 + e]);
    h[e] = from_f<T>(acc[e] + x);
  }
}

// ---------------------------------------------------------------------------
// S0+S1: q,k,v projection with the embedding gather in the A prologue
// ---------------------------------------------------------------------------
template <typename T, int BM, int BN, int WGM, int WGN, int PF, int BK, bool SC>
__global__ __launch_bounds__(WGM *WGN *WAVE) void qkv_kernel(QkvArgs a) {
  using G = Gemm<T, BM, BN, WGM, WGN, PF, BK>;
  __shared__ __attribute__((aligned(16))) char smem[G::LDS_BYTES];
  // the row tiles of one (weight tile, K split) run on one XCD
  int g, mt;
  if (!xcd_group_tile_split((int)cdiv64(a.col1 - a.col0, BN) * a.ksplit, (int)cdiv64(a.M, BM),
                            a.rchunks, &g, &mt))
    return;
  const int nt = g / a.ksplit, ks = g % a.ksplit;
  const int64_t m0 = (int64_t)mt * BM;
  const int n0 = a.col0 + nt * BN;
  if (!tile_active(a.active, m0, BM, a.M, a.C)) return;
  // rows past a count on the device (at most M) are skipped
  int64_t M = a.M;
  if (a.m_dev) {
    const int64_t md = *a.m_dev;
    M = md < M ? md : M;
  }
  if (m0 >= M) return;
  const T *E = static_cast<const T *>(a.embed);
  const T *sc = static_cast<const T *>(a.sc_in);
  const int nq = a.nq, nk = a.nkv, ntot = a.col1, d = a.d;
  GatherLoader<T, G::AI, SC> al;
#pragma unroll
  for (int it = 0; it < G::AI; ++it) {
    const int64_t row = m0 + G::a_row(it);
    const bool in = row < M;
    const int id = in ? a.ids[row] : 0;
    const bool ok = in && id >= 0 && id < a.vocab;
    if (in && !ok && a.flags && G::a_kc(it) == 0) atomicOr(a.flags, DG_FLAG_BAD_TOKEN);
    al.e[it] = E + (ok ? (int64_t)id * d : 0);
    al.s[it] = sc ? sc + (ok ? row * d : 0) : E;
    al.live[it] = ok;
  }
  RowLoader<T, G::BI> bl;
  const T *wq = static_cast<const T *>(a.wq);
#pragma unroll
  for (int it = 0; it < G::BI; ++it) {
    const int n = n0 + G::a_row(it);
    const T *p;
    if (n < nq) p = wq + (int64_t)n * d;
    else if (n < nq + nk) p = static_cast<const T *>(a.wk) + (int64_t)(n - nq) * d;
    else p = static_cast<const T *>(a.wv) + (int64_t)(n < ntot ? n - nq - nk : 0) * d;
    bl.set(it, p, n < ntot, wq);
  }
  f32x4 acc[G::TM][G::TN];
  const int kb = ks * a.kchunk;
  G::run(smem, al, bl, kb, kb + a.kchunk < d ? kb + a.kchunk : d, acc);
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int wm = w / WGN, wn = w % WGN;
  if (a.part) {   // split K: raw partial sums, the reduce applies the epilogue
    const int64_t nc = a.col1 - a.col0;
    store_partial<G, WGN>(a.part + (int64_t)ks * a.M * nc, nc, acc, m0, n0 - a.col0, a.M, nc);
    return;
  }
  // Epilogue through LDS: the tile, scaled and rounded to T, goes to LDS in the
  // MFMA layout, then each thread stores whole 16-byte row chunks, so a wave
  // writes full 128-byte lines of q, k and v (the MFMA layout alone would give
  // 32-byte pieces of four rows per store).  A chunk of VEC columns never
  // straddles q, k and v (their widths are multiples of 64).
  constexpr int OP = BN + G::VEC;   // LDS pitch of the output tile, elements
  static_assert(BM * OP * (int)sizeof(T) <= G::LDS_BYTES, "output tile must fit the K loop's LDS");
  T *ot = reinterpret_cast<T *>(smem);
  __syncthreads();   // every wave is done with the K loop's LDS
#pragma unroll
  for (int j = 0; j < G::TN; ++j) {
    const int cl = wn * G::WN + j * 16 + (lane & 15);
    const float sc = n0 + cl < nq ? a.q_scale : 1.f;
#pragma unroll
    for (int i = 0; i < G::TM; ++i)
#pragma unroll
      for (int r = 0; r < 4; ++r) ot[(wm * G::WM + i * 16 + 4 * (lane >> 4) + r) * OP + cl] =
          from_f<T>(acc[i][j][r] * sc);
  }
  __syncthreads();
  T *q = static_cast<T *>(a.q), *k = static_cast<T *>(a.k), *v = static_cast<T *>(a.v);
  constexpr int CPW = BN / G::VEC;   // 16-byte chunks per tile row
  for (int ch = threadIdx.x; ch < BM * CPW; ch += G::NT) {
    const int rl = ch / CPW, cc = ch % CPW;
    const int64_t row = m0 + rl;
    const int col = n0 + cc * G::VEC;
    if (row >= M || col >= ntot) continue;
    T *base;
    int ld, c;
    if (col < nq) { base = q; ld = nq; c = col; }
    else if (col < nq + nk) { base = k; ld = nk; c = col - nq; }
    else { base = v; ld = nk; c = col - nq - nk; }
    int64_t orow = row;
    if (col >= nq && a.kv_row) orow = a.kv_row[row];
    else if (col >= nq && a.kv_cmul > 1) orow = (row / a.C) * a.kv_cmul * a.C + row % a.C;
    if (orow < 0) continue;
    const uint4 val = *reinterpret_cast<const uint4 *>(ot + rl * OP + cc * G::VEC);
    *reinterpret_cast<uint4 *>(base + orow * ld + c) = val;
    if (col >= nq)
      for (int cp = 1; cp <= a.kv_copies; ++cp)
        *reinterpret_cast<uint4 *>(base + (orow + (int64_t)cp * a.C) * ld + c) = val;
  }
}

// ---------------------------------------------------------------------------
// S3: h = x + o Wo^T, x recomputed from the embedding (fp32, unrounded)
// ---------------------------------------------------------------------------
// PREC (bf16): o is fp32 and enters as hi and lo bf16 halves over 2K columns
// against Wo read twice; h is written as hi | lo halves of [M, 2d] rows.
template <typename T, int BM, int BN, int WGM, int WGN, int PF, int BK, bool PREC = false>
__global__ __launch_bounds__(WGM *WGN *WAVE) void oproj_kernel(OprojArgs a) {
  using G = Gemm<T, BM, BN, WGM, WGN, PF, BK>;
  static_assert(!PREC || std::is_same<T, bf16>::value, "split operands: bf16");
  __shared__ __attribute__((aligned(16))) char smem[G::LDS_BYTES];
  // the row tiles of one (weight tile, K split) run on one XCD
  int g, mt;
  if (!xcd_group_tile_split((int)cdiv64(a.d, BN) * a.ksplit, (int)cdiv64(a.M, BM), a.rchunks, &g, &mt))
    return;
  const int nt = g / a.ksplit, ks = g % a.ksplit;
  const int64_t m0 = (int64_t)mt * BM;
  const int n0 = nt * BN;
  if (!tile_active(a.active, m0, BM, a.M, a.C)) return;
  const int K = a.kdim, d = a.d;
  const int KE = PREC ? 2 * K : K;   // columns of the product
  const T *wo = static_cast<const T *>(a.wo);
  using AL = typename std::conditional<PREC, F32SplitLoader<G::AI>, RowLoader<T, G::AI>>::type;
  using BL = typename std::conditional<PREC, WrapRowLoader<T, G::BI>, RowLoader<T, G::BI>>::type;
  using TA = typename std::conditional<PREC, float, T>::type;
  const TA *o = static_cast<const TA *>(a.o);
  AL al;
  BL bl;
  if constexpr (PREC) {
    al.K = K;
    bl.K = K;
  }
#pragma unroll
  for (int it = 0; it < G::AI; ++it) {
    const int64_t row = m0 + G::a_row(it);
    al.set(it, o + row * K, row < a.M, o);
  }
#pragma unroll
  for (int it = 0; it < G::BI; ++it) {
    const int n = n0 + G::a_row(it);
    bl.set(it, wo + (int64_t)n * K, n < d, wo);
  }
  f32x4 acc[G::TM][G::TN];
  const int kb = ks * a.kchunk;
  G::run(smem, al, bl, kb, kb + a.kchunk < KE ? kb + a.kchunk : KE, acc);
  if (a.part) {   // split K: raw partial sums, the reduce adds the residual
    store_partial<G, WGN>(a.part + (int64_t)ks * a.M * d, d, acc, m0, n0, a.M, d);
    return;
  }
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int wm = w / WGN, wn = w % WGN;
  const T *E = static_cast<const T *>(a.embed);
  const T *sc = static_cast<const T *>(a.sc_in);
  T *h = static_cast<T *>(a.h);
#pragma unroll
  for (int i = 0; i < G::TM; ++i)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int64_t row = m0 + wm * G::WM + i * 16 + 4 * (lane >> 4) + r;
      if (row >= a.M) continue;
      const int id = a.ids[row];
      const bool ok = id >= 0 && id < a.vocab;
#pragma unroll
      for (int j = 0; j < G::TN; ++j) {
        const int col = n0 + wn * G::WN + j * 16 + (lane & 15);
        if (col >= d) continue;
        float x = ok ? to_f(E[(int64_t)id * d + col]) : 0.f;
        if (sc) x += to_f(sc[row * d + col]);
        if constexpr (PREC)
          store_split(h + row * 2 * d, d, col, acc[i][j][r] + x);
        else
          h[row * d + col] = from_f<T>(acc[i][j][r] + x);
      }
    }
}

// ---------------------------------------------------------------------------
// bf16 K loop with direct-to-LDS staging (global_load_lds_dwordx4): each wave
// instruction moves a block of 16 rows x 64 bytes (BK = 32) from global memory
// straight into LDS.  NS stages give NS-1 steps of loads in flight without
// holding staged tiles in registers.  The four 16-byte chunks of a 64-byte row
// sit XOR-swizzled by (row >> 1) & 3.  A 16-byte LDS read is served eight
// lanes at a time over 128 bytes of banks; with this swizzle the eight rows a
// pass reads (rows 8q .. 8q+7 of one logical chunk) land on eight distinct
// 16-byte bank groups (SQ_LDS_BANK_CONFLICT 0; a (row >> 2) & 3 swizzle costs
// 2x on half the passes).  The swizzle is applied on the global side (each lane
// fetches the chunk that belongs at its LDS slot).  Stages live in separate
// LDS arrays, so the compiler can tell a stage being read from the stages
// still being filled and waits only for the loads a read depends on.
// ---------------------------------------------------------------------------
template <int BM, int BN, int WGM, int WGN, int NS>
struct DmaLoop {
  static constexpr int BK = 32, NW = WGM * WGN;
  static constexpr int WM = BM / WGM, WN = BN / WGN, TM = WM / 16, TN = WN / 16;
  static constexpr int QA = BM / 16, NQ = (BM + BN) / 16, QW = NQ / NW;
  static constexpr int STAGE = (BM + BN) * 64;   // bytes
  static_assert(NQ % NW == 0, "16-row blocks must divide among the waves");
  static_assert(NS >= 2 && (NS - 2) * QW < 64, "stage count");
  using MF = Mfma<bf16>;
  using frag = MF::frag;

  // rowa(r) / rowb(r): first element of row r of the A / B tile (always a
  // dereferenceable row); K must be a multiple of BK.  astep / bstep: elements
  // between consecutive K steps of an A / B row (BK for a row-major matrix,
  // BM * BK for one stored in BM x BK blocks).  afix(kt, a) may transform the
  // A fragments of step kt after they are read from LDS.
  template <class RA, class RB, class AF>
  __device__ static void run(char *(&st)[NS], const RA &rowa, const RB &rowb, int K,
                             int64_t astep, int64_t bstep, f32x4 (&acc)[TM][TN], const AF &afix) {
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int wm = w / WGN, wn = w % WGN;
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j) acc[i][j] = zero4();
    const int nk = K / BK;
    // lane l fills slot (row l/4, chunk l%4) of each 16-row block it loads
    const int lc = (lane & 3) ^ ((lane >> 3) & 3);
    const bf16 *gp[QW];
#pragma unroll
    for (int i = 0; i < QW; ++i) {
      const int q = w * QW + i;
      gp[i] = (q < QA ? rowa(16 * q + (lane >> 2)) : rowb(16 * (q - QA) + (lane >> 2))) + 8 * lc;
    }
    auto dma = [&](int kt, char *s) {
#pragma unroll
      for (int i = 0; i < QW; ++i)
        __builtin_amdgcn_global_load_lds(
            gp[i] + kt * (w * QW + i < QA ? astep : bstep),
            (__attribute__((address_space(3))) void *)(s + (w * QW + i) * 1024), 16,
            0, 0);
    };
    // fragment of row (16-aligned base) + lane%16, logical chunk lane/16
    const int pc = 16 * ((lane >> 4) ^ ((lane >> 1) & 3)) + 64 * (lane & 15);
    auto compute = [&](const char *s, int kt) {
      frag a[TM], b[TN];
#pragma unroll
      for (int i = 0; i < TM; ++i)
        a[i] = *reinterpret_cast<const frag *>(s + (wm * WM + i * 16) * 64 + pc);
      afix(kt, a);
#pragma unroll
      for (int j = 0; j < TN; ++j)
        b[j] = *reinterpret_cast<const frag *>(s + (BM + wn * WN + j * 16) * 64 + pc);
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j) acc[i][j] = MF::mma(a[i], b[j], acc[i][j]);
    };
    // vmcnt(n) with the other counters left alone (gfx9 encoding)
    constexpr int WN_ = (NS - 2) * QW;
    constexpr int WAIT = (WN_ & 15) | ((WN_ >> 4) << 14) | (7 << 4) | (15 << 8);
    // step kt lives in stage kt % NS; past the last step the loads repeat it
    // (never read), so every step issues the same number of loads
    auto step = [&](int kt, int j) {
      // this wave's loads of step kt have landed; after the barrier every
      // wave's have, and every wave is done with step kt-1's stage
      __builtin_amdgcn_s_waitcnt(WAIT);
      __builtin_amdgcn_s_barrier();
      dma(kt + NS - 1 < nk ? kt + NS - 1 : nk - 1, st[(j + NS - 1) % NS]);
      compute(st[j], kt);
    };
#pragma unroll
    for (int s = 0; s < NS - 1; ++s) dma(s < nk ? s : nk - 1, st[s]);
    int k0 = 0;
    for (; k0 + NS <= nk; k0 += NS) {
#pragma unroll
      for (int j = 0; j < NS; ++j) step(k0 + j, j);
    }
#pragma unroll
    for (int j = 0; j < NS - 1; ++j)
      if (k0 + j < nk) step(k0 + j, j);
    // the last (repeated) loads land before the workgroup's LDS is released
    __builtin_amdgcn_s_waitcnt((7 << 4) | (15 << 8));
  }
};

// ---------------------------------------------------------------------------
// FP8 (e4m3) K loop with direct-to-LDS staging for the LM head with FP8
// activations: both operands are e4m3 codes (one byte each), K steps of 128
// codes in NS stages (NS - 1 steps of loads in flight), and the 16x16x128
// f8f6f4 MFMA (fp32 accumulation), which takes 32 codes of a row per lane:
// lane l holds row l % 16 and a 32-code group of k chosen by l / 16, the same
// group for both operands (any consistent assignment of k to lanes gives the
// same sum).  Rows are 128 bytes in LDS; chunk c of row r sits at chunk
// c ^ (r & 7), so the 16-byte fragment reads of eight consecutive rows hit
// eight distinct bank groups.  Each wave instruction of global_load_lds_dwordx4
// moves 8 rows x 128 bytes; a lane fetches the chunk that belongs in its slot.
// ---------------------------------------------------------------------------
template <int BM, int BN, int WGM, int WGN, int NS>
struct DmaLoopF8 {
  static constexpr int BK = 128, NW = WGM * WGN;
  static constexpr int WM = BM / WGM, WN = BN / WGN, TM = WM / 16, TN = WN / 16;
  static constexpr int QA = BM / 8, NQ = (BM + BN) / 8, QW = NQ / NW;   // 8-row groups
  static constexpr int STAGE = (BM + BN) * BK;                          // bytes
  static_assert(NQ % NW == 0, "8-row groups must divide among the waves");
  static_assert(NS >= 2 && (NS - 2) * QW < 64, "stage count");
  typedef int v8i __attribute__((ext_vector_type(8)));

  // rowa(r) / rowb(r): first code of row r of the A / B tile (always a
  // dereferenceable row); K (codes per row) must be a multiple of BK
  template <class RA, class RB>
  __device__ static void run(char *(&st)[NS], const RA &rowa, const RB &rowb, int K,
                             f32x4 (&acc)[TM][TN]) {
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int wm = w / WGN, wn = w % WGN;
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j) acc[i][j] = zero4();
    const int nk = K / BK;
    if (nk <= 0) return;
    // lane l fills slot (row l / 8, chunk l % 8) of each 8-row group it loads
    const int r8 = lane >> 3, lc = (lane & 7) ^ r8;
    const uint8_t *gp[QW];
#pragma unroll
    for (int i = 0; i < QW; ++i) {
      const int q = w * QW + i;
      gp[i] = (q < QA ? rowa(8 * q + r8) : rowb(8 * (q - QA) + r8)) + 16 * lc;
    }
    auto dma = [&](int kt, char *s) {
#pragma unroll
      for (int i = 0; i < QW; ++i)
        __builtin_amdgcn_global_load_lds(
            gp[i] + (int64_t)kt * BK,
            (__attribute__((address_space(3))) void *)(s + (w * QW + i) * 1024), 16, 0, 0);
    };
    // fragment of tile row `row`: logical chunks 2g and 2g + 1, g = lane / 16
    const int g = lane >> 4;
    auto frag_at = [&](const char *s, int row) {
      const int sw = row & 7;
      const uint4 lo = *reinterpret_cast<const uint4 *>(s + row * BK + (((2 * g) ^ sw) << 4));
      const uint4 hi = *reinterpret_cast<const uint4 *>(s + row * BK + (((2 * g + 1) ^ sw) << 4));
      v8i f;
      f[0] = (int)lo.x; f[1] = (int)lo.y; f[2] = (int)lo.z; f[3] = (int)lo.w;
      f[4] = (int)hi.x; f[5] = (int)hi.y; f[6] = (int)hi.z; f[7] = (int)hi.w;
      return f;
    };
    auto compute = [&](const char *s) {
      v8i b[TN];
#pragma unroll
      for (int j = 0; j < TN; ++j) b[j] = frag_at(s, BM + wn * WN + j * 16 + (lane & 15));
#pragma unroll
      for (int i = 0; i < TM; ++i) {
        const v8i a = frag_at(s, wm * WM + i * 16 + (lane & 15));
#pragma unroll
        for (int j = 0; j < TN; ++j)
          // formats 0 / 0: e4m3 for both operands; block scales 127 (2^0)
          acc[i][j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b[j], acc[i][j], 0, 0, 0,
                                                                        127, 0, 127);
      }
    };
    // vmcnt(n) with the other counters left alone (gfx9 encoding): the loads
    // of the NS - 2 younger steps may still be in flight
    constexpr int WN_ = (NS - 2) * QW;
    constexpr int WAIT = (WN_ & 15) | ((WN_ >> 4) << 14) | (7 << 4) | (15 << 8);
    // step kt lives in stage kt % NS: wait for this wave's loads of it, then the
    // barrier (every wave's loads landed, every wave done with step kt - 1's
    // stage), then the loads of step kt + NS - 1 into that stage (past the
    // last step they repeat it, never read, so every step issues the same
    // number of loads), then the MFMAs
    auto step = [&](int kt, int j) {
      __builtin_amdgcn_s_waitcnt(WAIT);
      __builtin_amdgcn_s_barrier();
      dma(kt + NS - 1 < nk ? kt + NS - 1 : nk - 1, st[(j + NS - 1) % NS]);
      compute(st[j]);
    };
#pragma unroll
    for (int s = 0; s < NS - 1; ++s) dma(s < nk ? s : nk - 1, st[s]);
    int k0 = 0;
    for (; k0 + NS <= nk; k0 += NS) {
#pragma unroll
      for (int j = 0; j < NS; ++j) step(k0 + j, j);
    }
#pragma unroll
    for (int j = 0; j < NS - 1; ++j)
      if (k0 + j < nk) step(k0 + j, j);
    // the last (repeated) loads land before the workgroup's LDS is released
    __builtin_amdgcn_s_waitcnt((7 << 4) | (15 << 8));
  }
};

// ---------------------------------------------------------------------------
// S4+S5 (tile part): logits of a VTILE-wide vocabulary tile for BN rows, with
// per-(row, tile) softmax statistics.  Computed as C^T: MFMA rows are
// vocabulary entries, MFMA columns are canvas rows, so each row's reduction
// over the vocabulary runs mostly inside a lane.
// ---------------------------------------------------------------------------
// PF < 0 selects the direct-to-LDS K loop with -PF stages (bf16, BK = 32).
// TL: the head is read from its copy in BM x 32 blocks (a.head_tiled).
// F8: the head is read from its e4m3 copy (a.head_fp8, a.head_exp; register K loop)
// HL: h arrives as bf16 hi | lo halves of [rows, 2d] rows (LmheadArgs.hl);
// each row takes two MFMA columns, hi in column block j and lo in block
// j + TN/2 of the same lane, which are added before the epilogue, so the
// vocabulary tile is streamed once for both halves.
// FA (with F8): the activations are e4m3 codes too (a.h_fp8, per-row
// exponents a.h_exp), and the product runs on the FP8 MFMA (DmaLoopF8).
template <typename T, int BM, int BN, int WGM, int WGN, int PF, int BK, bool TL = false, bool F8 = false,
          bool HL = false, bool FA = false>
__global__ __launch_bounds__(WGM *WGN *WAVE) void lmhead_kernel(LmheadArgs a) {
  using G = Gemm<T, BM, BN, WGM, WGN, PF < 0 ? 1 : PF, BK>;
  static_assert(BM == VTILE, "vocabulary tile must match the stats granularity");
  static_assert(!HL || (G::TN % 2 == 0 && sizeof(T) == 2), "split rows: bf16, even column blocks");
  static_assert(!FA || (F8 && !HL && !TL), "FP8 activations go with the e4m3 head");
  // rows per wave / workgroup and 16-row column blocks per wave after the halves combine
  constexpr int TNR = HL ? G::TN / 2 : G::TN;
  constexpr int WNR = HL ? G::WN / 2 : G::WN;
  constexpr int BNR = HL ? BN / 2 : BN;
  __shared__ float red_m[WGM][BN];
  __shared__ int red_i[WGM][BN];
  __shared__ float red_s[WGM][BN];
  __shared__ float red_t[WGM][BN];
  // group = vocabulary tile; its row tiles share the E tile and run on one XCD
  int vt, rt;
  if (!xcd_group_tile(a.vocab / BM, (int)cdiv64(a.nrows, BNR), &vt, &rt)) return;
  const int v0 = vt * BM;
  const int64_t n0 = (int64_t)rt * BNR;
  const int d = a.d;
  if (a.active_rows && !tile_active(a.active_rows, n0, BNR, a.nrows, a.rows_per_flag)) return;
  const T *head = static_cast<const T *>(a.head);
  const T *hh = static_cast<const T *>(a.h);
  // source of tile column r (the B operand): its row of h, and for HL the half;
  // *ok is false for a column past the rows (or without a source row), which
  // then reads row 0 and is never stored
  auto bsrc = [&](int r, bool *ok) -> const T * {
    int real = r, part = 0;
    if constexpr (HL) {
      const int wn_ = r / G::WN, jj = (r % G::WN) / 16;
      real = wn_ * WNR + (jj % TNR) * 16 + (r % 16);
      part = jj / TNR;
    }
    const int64_t n = n0 + real;
    int64_t src = -1;
    if (n < a.nrows) src = a.row_index ? (int64_t)a.row_index[n] : n;
    *ok = src >= 0;
    return hh + (src >= 0 ? src : 0) * (HL ? 2 * (int64_t)d : (int64_t)d) + part * d;
  };
  f32x4 acc[G::TM][G::TN];
  if constexpr (FA) {
    // three stages where they fit in LDS beside the statistics arrays, else two
    constexpr int NSF = (BM + BN) * 128 * 3 <= 144 * 1024 ? 3 : 2;
    using D = DmaLoopF8<BM, BN, WGM, WGN, NSF>;
    static_assert(D::TM == G::TM && D::TN == G::TN, "tile shape");
    __shared__ __attribute__((aligned(1024))) char f0[D::STAGE], f1[D::STAGE],
        f2[NSF > 2 ? D::STAGE : 16];
    char *st[NSF];
    st[0] = f0;
    st[1] = f1;
    if constexpr (NSF > 2) st[2] = f2;
    auto rowa = [&](int r) { return a.head_fp8 + (int64_t)(v0 + r) * d; };
    auto rowb = [&](int r) {
      bool ok;
      const T *p = bsrc(r, &ok);   // its row index, through the bf16 row pointer
      return a.h_fp8 + (p - hh) / d * (int64_t)d;
    };
    D::run(st, rowa, rowb, d, acc);
  } else if constexpr (PF < 0) {
    // rows past the matrix (or without a source row) read row 0: their
    // columns are never stored and columns do not mix
    constexpr int NS = -PF;
    static_assert(NS >= 2 && NS <= 4, "stages");
    using D = DmaLoop<BM, BN, WGM, WGN, NS>;
    __shared__ __attribute__((aligned(1024))) char s0[D::STAGE], s1[D::STAGE],
        s2[NS > 2 ? D::STAGE : 16], s3[NS > 3 ? D::STAGE : 16];
    char *const st4[4] = {s0, s1, s2, s3};
    char *st[NS];
#pragma unroll
    for (int s = 0; s < NS; ++s) st[s] = st4[s];
    const T *ht = static_cast<const T *>(a.head_tiled);
    auto rowa = [&](int r) {
      return TL ? ht + (int64_t)v0 * d + r * 32 : head + (int64_t)(v0 + r) * d;
    };
    auto rowb = [&](int r) {
      bool ok;
      return bsrc(r, &ok);
    };
    D::run(st, rowa, rowb, d, TL ? (int64_t)BM * 32 : (int64_t)32, (int64_t)32, acc,
           [](int, typename D::frag(&)[D::TM]) {});
  } else {
    __shared__ __attribute__((aligned(16))) char smem[G::LDS_BYTES];
    static_assert(!TL || (BK == 32 && sizeof(T) == 2), "blocked head: bf16, BK = 32");
    static_assert(!F8 || (!TL && sizeof(T) == 2), "e4m3 head: bf16 activations, row-major codes");
    using AL = typename std::conditional<
        F8, Fp8RowLoader<G::AI>,
        typename std::conditional<TL, BlockedRowLoader<T, G::AI, BM>, RowLoader<T, G::AI>>::type>::type;
    AL al;
    const T *ht = static_cast<const T *>(a.head_tiled);
#pragma unroll
    for (int it = 0; it < G::AI; ++it) {
      const int v = v0 + G::a_row(it);
      if constexpr (F8)
        al.set(it, a.head_fp8 + (int64_t)v * d, v < a.vocab, a.head_fp8);
      else
        al.set(it, TL ? ht + (int64_t)v0 * d + G::a_row(it) * 32 : head + (int64_t)v * d, v < a.vocab,
               TL ? ht : head);
    }
    RowLoader<T, G::BI> bl;
#pragma unroll
    for (int it = 0; it < G::BI; ++it) {
      bool ok;
      const T *p = bsrc(G::a_row(it), &ok);
      bl.set(it, p, ok, hh);
    }
    G::run(smem, al, bl, 0, d, acc);
  }
  if constexpr (HL) {
#pragma unroll
    for (int i = 0; i < G::TM; ++i)
#pragma unroll
      for (int j = 0; j < TNR; ++j) acc[i][j] += acc[i][j + TNR];
  }

  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int wm = w / WGN, wn = w % WGN;
  // scale, then pass 1: max and lowest argmax per column (= canvas row)
  float mx[TNR];
  int ix[TNR];
  // first vocabulary row of the wave's block.  The excluded id, if any, is
  // entry (iex, rex) of lane group gex in at most one wave: a uniform test and
  // uniform indices, instead of a comparison per value
  const int vw0 = v0 + wm * G::WM;
  const int exr = a.exclude_id1 - 1 - vw0;
  const bool ex_here = a.exclude_id1 > 0 && exr >= 0 && exr < G::WM;
  const int iex = exr >> 4, gex = (exr >> 2) & 3, rex = exr & 3;
#pragma unroll
  for (int j = 0; j < TNR; ++j) {
    const int64_t n = n0 + wn * WNR + j * 16 + (lane & 15);
    float s = a.logit_scale;
    if (a.row_scale && n < a.nrows) s *= a.row_scale[n];
    if constexpr (FA) {   // the row's activation exponent (exact: a power of two)
      if (n < a.nrows) s = ldexpf(s, a.h_exp[a.row_index ? (a.row_index[n] >= 0 ? a.row_index[n] : 0) : n]);
    }
    float m = -INFINITY;
    int id = 0x7fffffff;
#pragma unroll
    for (int i = 0; i < G::TM; ++i)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        float sv = s;
        if constexpr (F8) sv = ldexpf(s, a.head_exp[vw0 + i * 16 + 4 * (lane >> 4) + r]);   // exact: a power of two
        acc[i][j][r] *= sv;
      }
    if (ex_here && (lane >> 4) == gex) {
#pragma unroll
      for (int i = 0; i < G::TM; ++i)
#pragma unroll
        for (int r = 0; r < 4; ++r)
          if (i == iex && r == rex) acc[i][j][r] = -INFINITY;
    }
#pragma unroll
    for (int i = 0; i < G::TM; ++i)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float l = acc[i][j][r];
        if (l > m) { m = l; id = vw0 + i * 16 + 4 * (lane >> 4) + r; }
      }
    // across the four lane groups: larger value, then lower id
#pragma unroll
    for (int o = 16; o <= 32; o <<= 1) {
      const float m2 = __shfl_xor(m, o);
      const int i2 = __shfl_xor(id, o);
      if (m2 > m || (m2 == m && i2 < id)) { m = m2; id = i2; }
    }
    mx[j] = m;
    ix[j] = id;
  }
  // label logits of slot rows: the lane holding (label, row) writes it
  if (a.lab_logit) {
#pragma unroll
    for (int j = 0; j < TNR; ++j) {
      const int64_t n = n0 + wn * WNR + j * 16 + (lane & 15);
      if (n >= a.nrows) continue;
      const int64_t bs = (n / a.lab_span) * a.lab_S + n % a.lab_S;
      int k = a.lab_n[bs];
      k = k < 0 ? 0 : (k > DG_MAX_LABELS ? DG_MAX_LABELS : k);
      const int32_t *labs = a.lab_ids + bs * DG_MAX_LABELS;
      for (int q = 0; q < k; ++q) {
        const int rel = labs[q] - (v0 + wm * G::WM);   // = i*16 + 4*(lane group) + r
        if (rel < 0 || rel >= G::WM || ((rel >> 2) & 3) != (lane >> 4)) continue;
        float val = 0.f;
#pragma unroll
        for (int i = 0; i < G::TM; ++i)
#pragma unroll
          for (int r = 0; r < 4; ++r)
            if (i == (rel >> 4) && r == (rel & 3)) val = acc[i][j][r];
        a.lab_logit[n * DG_MAX_LABELS + q] = val;
      }
    }
  }
  if ((lane >> 4) == 0) {
#pragma unroll
    for (int j = 0; j < TNR; ++j) {
      red_m[wm][wn * WNR + j * 16 + lane] = mx[j];
      red_i[wm][wn * WNR + j * 16 + lane] = ix[j];
    }
  }
  __syncthreads();
#pragma unroll
  for (int j = 0; j < TNR; ++j) {
    const int c = wn * WNR + j * 16 + (lane & 15);
    float m = red_m[0][c];
    int id = red_i[0][c];
#pragma unroll
    for (int q = 1; q < WGM; ++q) {
      const float m2 = red_m[q][c];
      const int i2 = red_i[q][c];
      if (m2 > m || (m2 == m && i2 < id)) { m = m2; id = i2; }
    }
    mx[j] = m;
    ix[j] = id;
  }
  // pass 2: with the tile reference r = tile_ref(m), sum e and e (l - r ln2)
  // for e = e^(l - r ln2) (kept in log2 units: x = l log2 e - r, e = 2^x);
  // p~ = e and logits out
  T *pt = static_cast<T *>(a.ptilde);
  float ss[TNR], tt[TNR];
#pragma unroll
  for (int j = 0; j < TNR; ++j) {
    const int64_t n = n0 + wn * WNR + j * 16 + (lane & 15);
    const bool live = n < a.nrows;
    const float rj = (float)tile_ref(mx[j]);
    // the row's p~ and logits at vocabulary vw0 + 4 (lane >> 4), the lane's
    // first entry; entry vw0 + i*16 + 4 (lane >> 4) is then a constant offset
    // away: i*16 in a row-major row, and in the 256 x 32 blocked layout (vw0 is
    // a multiple of 32) (i >> 1) blocks of 8192 plus (i & 1)*16
    T *pj = nullptr;
    if (pt && live)
      pj = pt + (a.ptilde_blocked ? ((n >> 8) * (a.vocab >> 5) + (vw0 >> 5)) * 8192 + (n & 255) * 32
                                  : n * a.vocab + vw0) + 4 * (lane >> 4);
    float *lj = a.logits && live ? a.logits + n * a.vocab + vw0 + 4 * (lane >> 4) : nullptr;
    float s = 0.f, t = 0.f;
#pragma unroll
    for (int i = 0; i < G::TM; ++i) {
      f32x4 e4;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        // clamped below: e = 2^x is 0 below -149 either way, and an excluded
        // id (l = -inf) then adds 0 to s and t instead of 0 * -inf
        const float x = fmaxf(fmaf(acc[i][j][r], kLog2e, -rj), -256.f);
        // raw v_exp_f32: x <= 0 (r >= m log2 e)
        const float e = __builtin_amdgcn_exp2f(x);
        s += e;
        t += e * x;
        e4[r] = e;
      }
      // four consecutive vocabulary entries of one row: one 8- (bf16) or 16-byte store
      if (pj) store4<T>(pj + (a.ptilde_blocked ? (i >> 1) * 8192 + (i & 1) * 16 : i * 16), e4);
      if (lj) *reinterpret_cast<f32x4 *>(lj + i * 16) = acc[i][j];
    }
    s += __shfl_xor(s, 16);
    t += __shfl_xor(t, 16);
    s += __shfl_xor(s, 32);
    t += __shfl_xor(t, 32);
    ss[j] = s;
    tt[j] = t;
  }
  if ((lane >> 4) == 0) {
#pragma unroll
    for (int j = 0; j < TNR; ++j) {
      red_s[wm][wn * WNR + j * 16 + lane] = ss[j];
      red_t[wm][wn * WNR + j * 16 + lane] = tt[j];
    }
  }
  __syncthreads();
  if (wm == 0 && (lane >> 4) == 0) {
#pragma unroll
    for (int j = 0; j < TNR; ++j) {
      const int c = wn * WNR + j * 16 + lane;
      const int64_t n = n0 + c;
      if (n >= a.nrows) continue;
      float s = 0.f, t = 0.f;
#pragma unroll
      for (int q = 0; q < WGM; ++q) { s += red_s[q][c]; t += red_t[q][c]; }
      float4 st;
      st.x = mx[j];
      st.y = s;
      st.z = t * kLn2;
      st.w = __int_as_float(ix[j]);
      a.stats[n * a.nvt + vt] = st;
    }
  }
}

// ---------------------------------------------------------------------------
// S6: sc = p E over a range of the vocabulary (A = p~ scaled, B = E^T rows)
// ---------------------------------------------------------------------------
// PB: p~ in 256-row blocks (a.ptilde_blocked); BT: E^T read from its 256 x 32
// blocked copy (a.embed_t_tiled, d % 256 == 0)
template <typename T, int BM, int BN, int WGM, int WGN, int PF, int BK, bool PB = false,
          bool BT = false>
__global__ __launch_bounds__(WGM *WGN *WAVE) void scgemm_kernel(ScArgs a) {
  using G = Gemm<T, BM, BN, WGM, WGN, PF, BK>;
  static_assert(!(PB || BT) || (sizeof(T) == 2 && BK % 32 == 0), "blocked operands: bf16, BK % 32 == 0");
  static_assert(!BT || BN == 256, "blocked E^T: 256-wide d tiles");
  __shared__ __attribute__((aligned(16))) char smem[G::LDS_BYTES];
  // group = vocabulary range z; its (row, d) tiles share the p~ slice and run
  // on one XCD
  const int ntn = (int)cdiv64(a.d, BN);
  int z, t;
  if constexpr (kScGroup) {
    if (!xcd_group_tile(a.ksplit, ntn * (int)cdiv64(a.M, BM), &z, &t)) return;
  } else {
    const int nt = ntn * (int)cdiv64(a.M, BM);
    if ((int)blockIdx.x >= a.ksplit * nt) return;
    z = blockIdx.x / nt;
    t = blockIdx.x % nt;
  }
  const int n0 = (t % ntn) * BN;
  const int64_t m0 = (int64_t)(t / ntn) * BM;
  if (!tile_active(a.active, m0, BM, a.M, a.C)) return;
  const int nk = a.vocab / G::BK;
  const int kbeg = (int)((int64_t)z * nk / a.ksplit) * G::BK;
  const int kend = (int)((int64_t)(z + 1) * nk / a.ksplit) * G::BK;
  const T *ptl = static_cast<const T *>(a.ptilde);
  const T *et = static_cast<const T *>(a.embed_t);
  ShiftedRowLoader<T, G::AI, PB> al;
#pragma unroll
  for (int it = 0; it < G::AI; ++it) {
    const int64_t row = m0 + G::a_row(it);
    const bool ok = row < a.M;
    const int64_t r = ok ? row : 0;
    al.p[it] = ptl + (PB ? (r >> 8) * 256 * (int64_t)a.vocab + (r & 255) * 32 : r * a.vocab);
    al.sh[it] = a.shift + r * a.nvt;
    al.live[it] = ok;
  }
  using BL = typename std::conditional<BT, BlockedRowLoader<T, G::BI, 256>, RowLoader<T, G::BI>>::type;
  BL bl;
  const T *ett = static_cast<const T *>(a.embed_t_tiled);
#pragma unroll
  for (int it = 0; it < G::BI; ++it) {
    const int n = n0 + G::a_row(it);
    if constexpr (BT)
      bl.set(it, ett + (int64_t)(n >> 8) * 256 * a.vocab + (n & 255) * 32, n < a.d, ett);
    else
      bl.set(it, et + (int64_t)n * a.vocab, n < a.d, et);
  }
  f32x4 acc[G::TM][G::TN];
  G::run(smem, al, bl, kbeg, kend, acc);
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int wm = w / WGN, wn = w % WGN;
#pragma unroll
  for (int i = 0; i < G::TM; ++i)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int64_t row = m0 + wm * G::WM + i * 16 + 4 * (lane >> 4) + r;
      if (row >= a.M) continue;
#pragma unroll
      for (int j = 0; j < G::TN; ++j) {
        const int col = n0 + wn * G::WN + j * 16 + (lane & 15);
        if (col >= a.d) continue;
        if (a.ksplit == 1)
          static_cast<T *>(a.out)[row * a.d + col] = from_f<T>(acc[i][j][r] * a.inv_z[row]);
        else
          a.part[((int64_t)z * a.M + row) * a.d + col] = acc[i][j][r];
      }
    }
}

// S6 with the direct-to-LDS K loop: p~ (256-row blocks) and E^T (256 x 32
// blocks) stream into four LDS stages without passing through registers, and
// the power-of-two rescale of p~ is applied to the A fragments after they are
// read from LDS.  The shifts of the workgroup's rows and vocabulary tiles are
// staged in LDS once, as bytes (a shift >= 255 already flushes a bf16 to 0),
// laid out so that a lane fetches the shifts of its four fragment rows with one
// 4-byte read.  Requires d % 256 == 0 and at most kScDmaTiles vocabulary tiles
// per split.
constexpr int kScDmaTiles = 64;

template <int WGM, int WGN>
__global__ __launch_bounds__(WGM *WGN *WAVE) void scgemm_dma_kernel(ScArgs a) {
  constexpr int BM = 256, BN = 256, NS = 4;
  using D = DmaLoop<BM, BN, WGM, WGN, NS>;
  static_assert(D::TM == 4, "one 4-byte shift read covers a wave's four fragment rows");
  __shared__ __attribute__((aligned(1024))) char s0[D::STAGE], s1[D::STAGE], s2[D::STAGE],
      s3[D::STAGE];
  __shared__ __attribute__((aligned(16))) unsigned char shl[kScDmaTiles * BM];
  char *st[NS] = {s0, s1, s2, s3};
  const int ntn = a.d / BN;
  const int nt = ntn * (int)cdiv64(a.M, BM);
  // Work item (vocabulary range z, output tile t), in that order, and XCD x
  // (workgroups are dealt to the 8 XCDs round-robin) takes the consecutive items
  // [x * per, (x + 1) * per): the tiles of one range share its p~ in one L2
  // instead of fetching it on every XCD, and no CU is left idle.
  const int total = a.ksplit * nt, per = (total + 7) / 8;
  const int item = (blockIdx.x & 7) * per + (blockIdx.x >> 3);
  if (item >= total) return;
  const int z = item / nt, t = item % nt;
  const int n0 = (t % ntn) * BN;
  const int64_t m0 = (int64_t)(t / ntn) * BM;
  if (!tile_active(a.active, m0, BM, a.M, a.C)) return;
  const int nk = a.vocab / 64;   // split boundaries on 64-entry steps
  const int kbeg = (int)((int64_t)z * nk / a.ksplit) * 64;
  const int kend = (int)((int64_t)(z + 1) * nk / a.ksplit) * 64;
  const int t0 = kbeg / VTILE;
  const int ntl = kend > kbeg ? (kend - 1) / VTILE - t0 + 1 : 0;
  // shift of (row m, tile t) at byte t*256 + (m/64)*64 + (m%16)*4 + (m%64)/16
  for (int i = threadIdx.x; i < ntl * BM; i += WGM * WGN * WAVE) {
    const int tl = i / BM, m = i % BM;
    const int64_t row = m0 + m;
    int sh = row < a.M ? a.shift[row * a.nvt + t0 + tl] : 255;
    sh = sh < 0 ? 0 : (sh > 255 ? 255 : sh);
    shl[tl * BM + (m >> 6) * 64 + (m & 15) * 4 + ((m >> 4) & 3)] = (unsigned char)sh;
  }
  __syncthreads();
  const bf16 *ptl = static_cast<const bf16 *>(a.ptilde);
  const bf16 *ett = static_cast<const bf16 *>(a.embed_t_tiled);
  const int64_t kb = (int64_t)(kbeg >> 5) * 8192;
  // rows of the last row block past M hold stale p~: their outputs are never stored
  const bf16 *pa = ptl + (m0 >> 8) * 256 * (int64_t)a.vocab + kb;
  const bf16 *pb = ett + (int64_t)(n0 >> 8) * 256 * a.vocab + kb;
  auto rowa = [&](int r) { return pa + r * 32; };
  auto rowb = [&](int r) { return pb + r * 32; };
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int wm = w / WGN, wn = w % WGN;
  const unsigned char *shw = shl + wm * 64 + (lane & 15) * 4;
  auto afix = [&](int kt, typename D::frag (&af)[D::TM]) {
    const int tl = ((kbeg + kt * 32) >> 8) - t0;
    const unsigned sh4 = *reinterpret_cast<const unsigned *>(shw + tl * BM);
#pragma unroll
    for (int i = 0; i < D::TM; ++i) {
      const uint4 v = __builtin_bit_cast(uint4, af[i]);
      af[i] = __builtin_bit_cast(typename D::frag, pow2_down(v, (int)((sh4 >> (8 * i)) & 255), bf16{}));
    }
  };
  f32x4 acc[D::TM][D::TN];
  D::run(st, rowa, rowb, kend - kbeg, (int64_t)8192, (int64_t)8192, acc, afix);
#pragma unroll
  for (int i = 0; i < D::TM; ++i)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int64_t row = m0 + wm * D::WM + i * 16 + 4 * (lane >> 4) + r;
      if (row >= a.M) continue;
#pragma unroll
      for (int j = 0; j < D::TN; ++j) {
        const int col = n0 + wn * D::WN + j * 16 + (lane & 15);
        if (a.ksplit == 1)
          static_cast<bf16 *>(a.out)[row * a.d + col] = from_f<bf16>(acc[i][j][r] * a.inv_z[row]);
        else
          a.part[((int64_t)z * a.M + row) * a.d + col] = acc[i][j][r];
      }
    }
}

// fixed-order sum of the split-K partials
template <typename T>
__global__ __launch_bounds__(256) void sc_reduce_kernel(const float *part, const float *inv_z,
                                                        void *out, int64_t n, int d, int ksplit) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= n) return;
  float s = 0.f;
  for (int z = 0; z < ksplit; ++z) s += part[(int64_t)z * n + i];
  static_cast<T *>(out)[i] = from_f<T>(s * inv_z[i / d]);
}

// The same sum for 4 consecutive outputs per thread (d % 4 == 0, so they share
// a row), with the loads of up to 8 splits in flight together; the splits are
// still added in order, so the result is bitwise that of sc_reduce_kernel
template <typename T>
__global__ __launch_bounds__(256) void sc_reduce4_kernel(const float *part, const float *inv_z,
                                                         void *out, int64_t n, int d, int ksplit) {
  const int64_t i = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 4;
  if (i >= n) return;
  const float4 s = sum_partials(part, n, i, ksplit);
  const float iz = inv_z[i / d];
  T *o = static_cast<T *>(out) + i;
  o[0] = from_f<T>(s.x * iz);
  o[1] = from_f<T>(s.y * iz);
  o[2] = from_f<T>(s.z * iz);
  o[3] = from_f<T>(s.w * iz);
}

// ---------------------------------------------------------------------------
// host launchers
// ---------------------------------------------------------------------------
template <typename T, int BM, int BN, int WGM, int WGN, int PF, int BK>
static hipError_t launch_qkv_t(const QkvArgs &a0, hipStream_t st) {
  QkvArgs a = a0;
  const int64_t ng = cdiv64(a.col1 - a.col0, BN) * a.ksplit, nt = cdiv64(a.M, BM);
  a.rchunks = xcd_chunks(ng, nt);
  const dim3 grid = xcd_grid(ng * a.rchunks, cdiv64(nt, a.rchunks));
  if (a.sc_in)
    hipLaunchKernelGGL((qkv_kernel<T, BM, BN, WGM, WGN, PF, BK, true>), grid, dim3(WGM * WGN * WAVE), 0, st, a);
  else
    hipLaunchKernelGGL((qkv_kernel<T, BM, BN, WGM, WGN, PF, BK, false>), grid, dim3(WGM * WGN * WAVE), 0, st, a);
  return hipGetLastError();
}

hipError_t launch_qkv(const QkvArgs &a, bool bf, hipStream_t st) {
  const int64_t ntot = a.col1 - a.col0;
  if (a.M <= 0 || ntot <= 0) return hipSuccess;
  if (a.col0 < 0 || a.col1 > a.nq + 2 * a.nkv) return hipErrorInvalidValue;
  QkvArgs b = a;
  proj_split(a.M, ntot, a.d, bf, &b.ksplit, &b.kchunk);
  if (b.ksplit == 1 || !a.part || a.m_dev) {
    b.part = nullptr;
    b.ksplit = 1;
    b.kchunk = a.d;
  }
  if (bf) {
    // tall and thin at small d (a read batch's k/v rows, a ragged batch):
    // 256-column tiles of 8 waves gather each embedding row for half as many
    // column tiles (read batch 0.369 -> 0.362 ms, ragged step's q/k/v 18.0 ->
    // 16.6 us against 128 x 128)
    if (!b.part && ntot % 256 == 0 && a.M >= 4096 && a.d <= 512)
      return launch_qkv_t<bf16, 128, 256, 2, 4, 2, 64>(b, st);
    if (!b.part && cdiv64(a.M, 128) * cdiv64(ntot, 128) >= 256)
      return launch_qkv_t<bf16, 128, 128, 2, 2, 2, 64>(b, st);
    hipError_t e = launch_qkv_t<bf16, 64, 64, 2, 2, 4, 64>(b, st);
    if (e != hipSuccess || !b.part) return e;
    hipLaunchKernelGGL((qkv_reduce_kernel<bf16>), dim3((unsigned)cdiv64(a.M * (ntot / 4), 256)),
                       dim3(256), 0, st, b);
    return hipGetLastError();
  }
  return launch_qkv_t<float, 64, 64, 2, 2, 1, 16>(b, st);
}

template <typename T, int BM, int BN, int WGM, int WGN, int PF, int BK>
static hipError_t launch_oproj_t(const OprojArgs &a0, hipStream_t st) {
  OprojArgs a = a0;
  const int64_t ng = cdiv64(a.d, BN) * a.ksplit, nt = cdiv64(a.M, BM);
  a.rchunks = xcd_chunks(ng, nt);
  const dim3 grid = xcd_grid(ng * a.rchunks, cdiv64(nt, a.rchunks));
  if constexpr (std::is_same<T, bf16>::value) {
    if (a.prec) {
      hipLaunchKernelGGL((oproj_kernel<T, BM, BN, WGM, WGN, PF, BK, true>), grid, dim3(WGM * WGN * WAVE), 0, st, a);
      return hipGetLastError();
    }
  }
  hipLaunchKernelGGL((oproj_kernel<T, BM, BN, WGM, WGN, PF, BK>), grid, dim3(WGM * WGN * WAVE), 0, st, a);
  return hipGetLastError();
}

hipError_t launch_oproj(const OprojArgs &a, bool bf, hipStream_t st) {
  if (a.M <= 0) return hipSuccess;
  if (a.prec && !bf) return hipErrorInvalidValue;
  OprojArgs b = a;
  const int ke = a.prec ? 2 * a.kdim : a.kdim;   // split halves double the product's K
  proj_split(a.M, a.d, ke, bf, &b.ksplit, &b.kchunk);
  if (b.ksplit == 1 || !a.part) {
    b.part = nullptr;
    b.ksplit = 1;
    b.kchunk = ke;
  }
  if (bf) {
    if (!b.part && cdiv64(a.M, 128) * cdiv64(a.d, 128) >= 512)
      return launch_oproj_t<bf16, 128, 128, 2, 2, 2, 64>(b, st);
    hipError_t e = launch_oproj_t<bf16, 64, 64, 2, 2, 4, 64>(b, st);
    if (e != hipSuccess || !b.part) return e;
    hipLaunchKernelGGL((oproj_reduce_kernel<bf16>), dim3((unsigned)cdiv64(a.M * (a.d / 4), 256)),
                       dim3(256), 0, st, b);
    return hipGetLastError();
  }
  return launch_oproj_t<float, 64, 64, 2, 2, 1, 16>(b, st);
}

// row count up to which the LM head uses 64-row tiles
constexpr int64_t kLmFewRows = 64;
// S8 label logits of slot rows: the scaled logit of each allowed label id at
// each slot row, as one dot product h_n . head_label per (row, label) (the LM
// head's tiles then skip them: there each lane went through its row's labels
// one at a time in a divergent loop, with a select over its accumulators for
// each label in range).  One wave per row, its lanes in groups of GL (a power
// of two, at most 64, with at most four 16-byte chunks of d per lane where d
// allows), one label per group at a time: each lane sums the products of its
// chunks in fp32 (bf16 products are exact in fp32), then a fixed butterfly
// adds the group.  Split rows (HL) take hi + lo of h.  The excluded id gets
// -inf, as in the tiles.
template <typename T, bool HL>
__global__ __launch_bounds__(256) void lab_logit_kernel(LmheadArgs a, int GL) {
  constexpr int VEC = 16 / sizeof(T);
  const int64_t n = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (n >= a.nrows) return;
  if (a.active_rows && !a.active_rows[n / a.rows_per_flag]) return;
  const int64_t src = a.row_index ? (int64_t)a.row_index[n] : n;
  if (src < 0) return;
  const int64_t bs = (n / a.lab_span) * a.lab_S + n % a.lab_S;
  int k = a.lab_n[bs];
  k = k < 0 ? 0 : (k > DG_MAX_LABELS ? DG_MAX_LABELS : k);
  const int32_t *labs = a.lab_ids + bs * DG_MAX_LABELS;
  const int d = a.d, nch = d / VEC;
  const int LG = 64 / GL, g = lane / GL, li = lane % GL;
  const T *hr = static_cast<const T *>(a.h) + src * (HL ? 2 * (int64_t)d : (int64_t)d);
  const T *head = static_cast<const T *>(a.head);
  const float sc = a.logit_scale * (a.row_scale ? a.row_scale[n] : 1.f);
  for (int q0 = 0; q0 < k; q0 += LG) {
    const int q = q0 + g;
    const int id = q < k ? labs[q] : 0;
    const T *er = head + (int64_t)(id >= 0 && id < a.vocab ? id : 0) * d;
    float acc = 0.f;
#pragma unroll 4
    for (int c = li; c < nch; c += GL) {
      Chunk<T> hx, ex;
      hx.u = *reinterpret_cast<const uint4 *>(hr + c * VEC);
      ex.u = *reinterpret_cast<const uint4 *>(er + c * VEC);
      if constexpr (HL) {
        Chunk<T> lo;
        lo.u = *reinterpret_cast<const uint4 *>(hr + d + c * VEC);
#pragma unroll
        for (int e = 0; e < VEC; ++e) acc = fmaf(to_f(hx.v[e]) + to_f(lo.v[e]), to_f(ex.v[e]), acc);
      } else {
#pragma unroll
        for (int e = 0; e < VEC; ++e) acc = fmaf(to_f(hx.v[e]), to_f(ex.v[e]), acc);
      }
    }
    for (int o = GL >> 1; o >= 1; o >>= 1) acc += __shfl_xor(acc, o);
    if (li == 0 && q < k) a.lab_logit[n * DG_MAX_LABELS + q] = id == a.exclude_id1 - 1 ? -INFINITY : acc * sc;
  }
}

// direct-to-LDS stages of the 256-row LM head's K loop.  (For the few-row
// tile, a pure weight stream, 2-4 direct-to-LDS stages measured slower than
// its register-staged loop, which keeps three workgroups per CU.)
constexpr int kLmStages = 4;

// one LM-head launch: the grid covers the rows BN (HL: BN / 2) at a time
template <typename T, int BN, int WGM, int WGN, int PF, int BK, bool TL, bool F8, bool HL, bool FA = false>
static void lmhead_go(const LmheadArgs &a, hipStream_t st) {
  const dim3 grid = xcd_grid(a.vocab / VTILE, cdiv64(a.nrows, HL ? BN / 2 : BN));
  hipLaunchKernelGGL((lmhead_kernel<T, VTILE, BN, WGM, WGN, PF, BK, TL, F8, HL, FA>), grid,
                     dim3(WGM * WGN * WAVE), 0, st, a);
}

// Rows given as hi | lo halves (slot reads): the few-row tile takes 64 rows in
// 128 columns over 8 waves, the large tile 128 rows in 256 columns, each with
// the loop its plain counterpart uses.
static hipError_t launch_lmhead_hl(const LmheadArgs &a, hipStream_t st) {
  const bool few = a.nrows <= kLmFewRows;
  if (a.head_fp8) {
    if (few) lmhead_go<bf16, 128, 4, 2, 2, 32, false, true, true>(a, st);
    else lmhead_go<bf16, 256, 2, 4, 1, 64, false, true, true>(a, st);
  } else if (!few && a.d <= 512 && a.head_tiled) {
    // many rows over a short K loop (a read batch at d 256): 64-row tiles, with
    // VGPRs for two workgroups per CU and two steps of loads in flight
    // (0.371 -> 0.361 ms for 512 canvases against 128-row tiles)
    lmhead_go<bf16, 128, 4, 2, 2, 32, true, false, true>(a, st);
  } else if (few) {
    if (a.head_tiled) lmhead_go<bf16, 128, 4, 2, 1, 32, true, false, true>(a, st);
    else lmhead_go<bf16, 128, 4, 2, 1, 32, false, false, true>(a, st);
  } else if (a.d % 32 == 0) {
    if (a.head_tiled) lmhead_go<bf16, 256, 2, 4, -kLmStages, 32, true, false, true>(a, st);
    else lmhead_go<bf16, 256, 2, 4, -kLmStages, 32, false, false, true>(a, st);
  } else {
    lmhead_go<bf16, 256, 2, 4, 1, 64, false, false, true>(a, st);
  }
  return hipGetLastError();
}

static hipError_t launch_lmhead_tiles(const LmheadArgs &a, bool bf, hipStream_t st);

// The label logits of many rows (a read batch) with a plain (bf16 or fp32)
// head come from lab_logit_kernel, after the tiles: 0.384 -> 0.376 ms for 512
// canvases with up to 26 labels per slot.  For a few rows (a single canvas's
// read: 40 rows, 0.381 against 0.397 ms), an e4m3 head or e4m3 activations the
// tiles write them.
constexpr int64_t kLabKernelRows = 1024;
hipError_t launch_lmhead(const LmheadArgs &a, bool bf, hipStream_t st) {
  if (!a.lab_logit || a.nrows < kLabKernelRows || a.head_fp8 || a.h_fp8 || (a.hl && !bf))
    return launch_lmhead_tiles(a, bf, st);
  LmheadArgs b = a;
  b.lab_logit = nullptr;
  hipError_t e = launch_lmhead_tiles(b, bf, st);
  if (e != hipSuccess || a.nrows <= 0) return e;
  const dim3 grid((unsigned)cdiv64(a.nrows, 4));
  // lanes per label: the smallest power of two giving at most four chunks each
  const int nch = a.d / (bf ? 8 : 4);
  int gl = 1;
  while (gl < 64 && gl * 4 < nch) gl *= 2;
  if (!bf) hipLaunchKernelGGL((lab_logit_kernel<float, false>), grid, dim3(256), 0, st, a, gl);
  else if (a.hl) hipLaunchKernelGGL((lab_logit_kernel<bf16, true>), grid, dim3(256), 0, st, a, gl);
  else hipLaunchKernelGGL((lab_logit_kernel<bf16, false>), grid, dim3(256), 0, st, a, gl);
  return hipGetLastError();
}

static hipError_t launch_lmhead_tiles(const LmheadArgs &a, bool bf, hipStream_t st) {
  if (a.hl) return bf ? launch_lmhead_hl(a, st) : hipErrorInvalidValue;
  if (a.h_fp8) {
    // e4m3 head and e4m3 activations: the FP8 MFMA on 256 x 256 tiles, two
    // stages (measured a little faster than 128-row tiles with three stages,
    // which read each head tile twice and the fragments with less reuse)
    if (!bf || !a.head_fp8 || !a.h_exp || a.d % 128) return hipErrorInvalidValue;
    lmhead_go<bf16, 256, 2, 4, 1, 64, false, true, false, true>(a, st);
    return hipGetLastError();
  }
  if (bf && a.head_fp8) {
    // e4m3 head: register K loop (the codes are decoded on their way into LDS);
    // with half the bytes per step, the few-row tile keeps two steps in flight
    if (a.nrows <= kLmFewRows) {
      const dim3 grid = xcd_grid(a.vocab / VTILE, cdiv64(a.nrows, 64));
      hipLaunchKernelGGL((lmhead_kernel<bf16, VTILE, 64, 4, 1, 2, 32, false, true>), grid, dim3(4 * WAVE), 0, st, a);
    } else {
      const dim3 grid = xcd_grid(a.vocab / VTILE, cdiv64(a.nrows, 256));
      hipLaunchKernelGGL((lmhead_kernel<bf16, VTILE, 256, 2, 4, 1, 64, false, true>), grid, dim3(8 * WAVE), 0, st, a);
    }
  } else if (bf && (a.nrows <= kLmFewRows || (int64_t)(a.vocab / VTILE) * cdiv64(a.nrows, 256) < 64)) {
    // few rows (slot reads): a 64-row tile keeps the MFMA work proportional to
    // the rows and three workgroups per CU keep the vocabulary stream busy.
    // Also when 256-row tiles would leave most CUs idle (a small vocabulary: one
    // canvas at V 2,048 is 8 tiles; 64-row tiles give 32, 22 -> 18 us); there
    // the K loop is short and latency-bound, and the direct-to-LDS loop with
    // four stages keeps three steps in flight (18 -> 15 us)
    const dim3 grid = xcd_grid(a.vocab / VTILE, cdiv64(a.nrows, 64));
    if (a.nrows > kLmFewRows && a.d % 32 == 0) {
      if (a.head_tiled)
        hipLaunchKernelGGL((lmhead_kernel<bf16, VTILE, 64, 4, 1, -4, 32, true>), grid, dim3(4 * WAVE), 0, st, a);
      else
        hipLaunchKernelGGL((lmhead_kernel<bf16, VTILE, 64, 4, 1, -4, 32>), grid, dim3(4 * WAVE), 0, st, a);
    } else if (a.head_tiled)
      hipLaunchKernelGGL((lmhead_kernel<bf16, VTILE, 64, 4, 1, 1, 32, true>), grid, dim3(4 * WAVE), 0, st, a);
    else
      hipLaunchKernelGGL((lmhead_kernel<bf16, VTILE, 64, 4, 1, 1, 32>), grid, dim3(4 * WAVE), 0, st, a);
  } else if (bf) {
    const dim3 grid = xcd_grid(a.vocab / VTILE, cdiv64(a.nrows, 256));
    if (a.d % 32 == 0 && a.head_tiled)
      hipLaunchKernelGGL((lmhead_kernel<bf16, VTILE, 256, 2, 4, -kLmStages, 32, true>), grid, dim3(8 * WAVE), 0, st, a);
    else if (a.d % 32 == 0)
      hipLaunchKernelGGL((lmhead_kernel<bf16, VTILE, 256, 2, 4, -kLmStages, 32>), grid, dim3(8 * WAVE), 0, st, a);
    else
      hipLaunchKernelGGL((lmhead_kernel<bf16, VTILE, 256, 2, 4, 1, 64>), grid, dim3(8 * WAVE), 0, st, a);
  } else {
    const dim3 grid = xcd_grid(a.vocab / VTILE, cdiv64(a.nrows, 64));
    hipLaunchKernelGGL((lmhead_kernel<float, VTILE, 64, 4, 1, 1, 16>), grid, dim3(4 * WAVE), 0, st, a);
  }
  return hipGetLastError();
}

hipError_t launch_scgemm(const ScArgs &a, bool bf, hipStream_t st) {
  if (bf) {
    const dim3 grid = kScGroup ? xcd_grid(a.ksplit, cdiv64(a.d, kScTileD) * cdiv64(a.M, 256))
                               : dim3((unsigned)(a.ksplit * cdiv64(a.d, kScTileD) * cdiv64(a.M, 256)));
    // vocabulary tiles a split can span: its 64-entry steps, rounded up, plus one
    const int64_t tiles = (int64_t)(a.vocab / 64 + a.ksplit - 1) / a.ksplit * 64 / VTILE + 2;
    if (a.ptilde_blocked && a.embed_t_tiled && a.d % 256 == 0 && tiles <= kScDmaTiles)
      hipLaunchKernelGGL((scgemm_dma_kernel<4, 2>),
                         dim3((unsigned)(8 * cdiv64(a.ksplit * cdiv64(a.d, 256) * cdiv64(a.M, 256), 8))),
                         dim3(8 * WAVE), 0, st, a);
    else if (a.ptilde_blocked && a.embed_t_tiled)
      hipLaunchKernelGGL((scgemm_kernel<bf16, 256, kScTileD, 4, 2, 1, 64, true, true>), grid, dim3(8 * WAVE), 0, st, a);
    else if (a.ptilde_blocked)
      hipLaunchKernelGGL((scgemm_kernel<bf16, 256, kScTileD, 4, 2, 1, 64, true>), grid, dim3(8 * WAVE), 0, st, a);
    else
      hipLaunchKernelGGL((scgemm_kernel<bf16, 256, kScTileD, 4, 2, 1, 64>), grid, dim3(8 * WAVE), 0, st, a);
  } else {
    const int64_t nt = cdiv64(a.d, 64) * cdiv64(a.M, 64);
    const dim3 grid = kScGroup ? xcd_grid(a.ksplit, nt) : dim3((unsigned)(a.ksplit * nt));
    hipLaunchKernelGGL((scgemm_kernel<float, 64, 64, 2, 2, 1, 16>), grid, dim3(4 * WAVE), 0, st, a);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || a.ksplit == 1) return e;
  const int64_t n = a.M * a.d;
  if (a.d % 4 == 0) {
    const dim3 g4((unsigned)cdiv64(n / 4, 256));
    if (bf)
      hipLaunchKernelGGL((sc_reduce4_kernel<bf16>), g4, dim3(256), 0, st, a.part, a.inv_z, a.out, n,
                         a.d, a.ksplit);
    else
      hipLaunchKernelGGL((sc_reduce4_kernel<float>), g4, dim3(256), 0, st, a.part, a.inv_z, a.out, n,
                         a.d, a.ksplit);
  } else if (bf) {
    hipLaunchKernelGGL((sc_reduce_kernel<bf16>), dim3((unsigned)cdiv64(n, 256)), dim3(256), 0, st,
                       a.part, a.inv_z, a.out, n, a.d, a.ksplit);
  } else {
    hipLaunchKernelGGL((sc_reduce_kernel<float>), dim3((unsigned)cdiv64(n, 256)), dim3(256), 0, st,
                       a.part, a.inv_z, a.out, n, a.d, a.ksplit);
  }
  return hipGetLastError();
}

}  // namespace dg
