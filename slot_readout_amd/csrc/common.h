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
__device__ inline float group4_max(float v) {
  v = fmaxf(v, __shfl_xor(v, 16));
  v = fmaxf(v, __shfl_xor(v, 32));
  return v;
}
__device__ inline float group4_sum(float v) {
  v += __shfl_xor(v, 16);
  v += __shfl_xor(v, 32);
  return v;
}

__host__ __device__ inline int64_t cdiv64(int64_t a, int64_t b) { return (a + b - 1) / b; }

}  // namespace dg
