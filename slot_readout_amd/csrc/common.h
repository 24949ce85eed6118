// Shared device helpers for the gfx950 kernels: storage types, MFMA traits,
// wave-level reductions.  Wave size is 64 throughout.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dg {

using bf16 = __bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int WAVE = 64;

// ---------------------------------------------------------------------------
// MFMA traits.  Both instructions are 16x16 output blocks with the same result
// layout: lane l holds D[4*(l/16) + r][l%16], r = 0..3.  Operand fragments:
// A lane l holds A[l%16][KPL*(l/16) .. +KPL-1], B lane l holds B[k same][l%16].
// ---------------------------------------------------------------------------
template <typename T> struct Mfma;

template <> struct Mfma<bf16> {
  static constexpr int KPL = 8;   // k values per lane
  static constexpr int KI = 32;   // k per instruction
  using frag = bf16x8;
  __device__ static inline f32x4 mma(frag a, frag b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
  }
};

template <> struct Mfma<float> {
  static constexpr int KPL = 1;
  static constexpr int KI = 4;
  using frag = float;
  __device__ static inline f32x4 mma(frag a, frag b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
  }
};

// ---------------------------------------------------------------------------
// conversions
// ---------------------------------------------------------------------------
__device__ inline float to_f(float x) { return x; }
__device__ inline float to_f(bf16 x) { return (float)x; }

template <typename T> __device__ inline T from_f(float x);
template <> __device__ inline float from_f<float>(float x) { return x; }
template <> __device__ inline bf16 from_f<bf16>(float x) { return (bf16)x; }

// A 16-byte chunk of T values, viewed elementwise.
template <typename T> struct Chunk {
  static constexpr int N = 16 / sizeof(T);
  union { uint4 u; T v[N]; };
};

__device__ inline f32x4 zero4() { return f32x4{0.f, 0.f, 0.f, 0.f}; }

// ---------------------------------------------------------------------------
// wave reductions (xor butterflies; every lane ends with the result)
// ---------------------------------------------------------------------------
__device__ inline float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
  return v;
}
__device__ inline float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  return v;
}
// reduce across the four 16-lane groups that hold the same MFMA column
// Reductions across the four 16-lane rows of a wave (lanes l, l^16, l^32, l^48)
// with the gfx950 row-swap moves: permlane16_swap(x, x) leaves x of rows {0,0,2,2}
// in one result and of rows {1,1,3,3} in the other; permlane32_swap(x, x) leaves
// rows {0,1,0,1} and {2,3,2,3}.  Every lane combines the same operands in the
// same order, so all four rows hold bitwise identical results.
__device__ inline float row_swap16(float v, float *other) {
  auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  *other = __uint_as_float(r[1]);
  return __uint_as_float(r[0]);
}
__device__ inline float row_swap32(float v, float *other) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  *other = __uint_as_float(r[1]);
  return __uint_as_float(r[0]);
}
__device__ inline float group4_max(float v) {
  float b;
  float a = row_swap16(v, &b);
  v = fmaxf(a, b);
  a = row_swap32(v, &b);
  return fmaxf(a, b);
}
__device__ inline float group4_sum(float v) {
  float b;
  float a = row_swap16(v, &b);
  v = a + b;
  a = row_swap32(v, &b);
  return a + b;
}

__host__ __device__ inline int64_t cdiv64(int64_t a, int64_t b) { return (a + b - 1) / b; }

// Reference of a vocabulary tile whose largest logit is m: r = ceil(m log2 e),
// an integer, so the tile's e^(l - r ln 2) are <= 1 and two tiles' references
// differ by an exact power of two.  The LM head and the vocabulary merge both
// derive r from the stored tile max with this one function.
constexpr float kLog2e = 1.44269504088896341f;
constexpr float kLn2 = 0.693147180559945309f;
__device__ inline int tile_ref(float m) {
  return m > -1e30f ? (int)ceilf(m * kLog2e) : -(1 << 28);
}

// Workgroup id -> (group g, tile t): the nt tiles of a group share an operand
// (a weight tile, a slice of p~).  Workgroups are dealt to the 8 XCDs
// round-robin by id, so whole groups are dealt to one XCD at a time and each
// group's tiles share that XCD's L2.  Launch 8 * cdiv(ngroups, 8) * nt
// workgroups; ids past the last group return false.
__device__ inline bool xcd_group_tile(int ngroups, int nt, int *g, int *t) {
  const int id = blockIdx.x, xcd = id & 7, local = id >> 3;
  *g = xcd + 8 * (local / nt);
  *t = local % nt;
  return *g < ngroups;
}
static inline dim3 xcd_grid(int64_t ngroups, int64_t nt) {
  return dim3((unsigned)(8 * cdiv64(ngroups, 8) * nt));
}

// xcd_group_tile with each group's nt tiles cut into `chunks` runs of
// ceil(nt / chunks) tiles, each run dealt as a group of its own: its tiles
// still share the group's operand on one XCD.  With few groups (a tall
// projection with a handful of weight tiles) whole groups would leave XCDs
// idle; the runs spread the work over all eight.  Launch
// xcd_grid(ngroups * chunks, ceil(nt / chunks)).
__device__ inline bool xcd_group_tile_split(int ngroups, int nt, int chunks, int *g, int *t) {
  const int per = (nt + chunks - 1) / chunks;
  int gg, tt;
  if (!xcd_group_tile(ngroups * chunks, per, &gg, &tt)) return false;
  *g = gg % ngroups;
  *t = (gg / ngroups) * per + tt;
  return *t < nt;
}
// runs per group: none below 16 groups (two per XCD or more keep the
// weight-tile sharing), else enough for at least 32 groups in all, at most
// one run per tile
static inline int xcd_chunks(int64_t ngroups, int64_t nt) {
  if (ngroups >= 16 || nt <= 1) return 1;
  const int64_t c = cdiv64(32, ngroups);
  return (int)(c < nt ? c : nt);
}

}  // namespace dg
