// Vocabulary-statistics merge, entropy-bounded commit and small helpers.
#include "common.h"
#include "kernels.h"

namespace dg {

// ---------------------------------------------------------------------------
// Merge the per-(row, vocabulary tile) statistics written by the LM-head
// kernel into the row's softmax summary.  For tile t with (m_t, s_t, t_t):
//   m = max m_t,  Z = sum s_t e^(m_t-m),  T = sum e^(m_t-m) (t_t + (m_t-m) s_t)
//   conf = 1/Z,  H = ln Z - T/Z,  lse = m + ln Z,  argmax = lowest id with l = m.
// One wave per row; tiles are assigned to lanes in a fixed pattern and combined
// with a fixed butterfly, so the result does not depend on scheduling.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void vocab_merge_kernel(VocabMergeArgs a) {
  const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (row >= a.nrows) return;
  const float4 *st = a.stats + row * a.nvt;
  // the row's tile statistics: up to 64 * KC of them stay in registers between
  // the passes (all of them up to a 262,144-entry vocabulary)
  constexpr int KC = 16;
  float4 vc[KC];
#pragma unroll
  for (int q = 0; q < KC; ++q) {
    const int t = lane + 64 * q;
    vc[q] = t < a.nvt ? st[t] : make_float4(-INFINITY, 0.f, 0.f, __int_as_float(0x7fffffff));
  }
  // f(v) over the row's tiles: the register copies, then any beyond them
  auto each = [&](auto f) {
#pragma unroll
    for (int q = 0; q < KC; ++q)
      if (lane + 64 * q < a.nvt) f(vc[q]);
    for (int t = lane + 64 * KC; t < a.nvt; t += 64) f(st[t]);
  };
  float m = -INFINITY;
  int id = 0x7fffffff, R = -(1 << 30);
  each([&](const float4 &v) {
    const int i = __float_as_int(v.w);
    if (v.x > m || (v.x == m && i < id)) { m = v.x; id = i; }
    R = max(R, tile_ref(v.x));
  });
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    const float m2 = __shfl_xor(m, o);
    const int i2 = __shfl_xor(id, o);
    if (m2 > m || (m2 == m && i2 < id)) { m = m2; id = i2; }
    R = max(R, __shfl_xor(R, o));
  }
  // Z = sum_t 2^(r_t - R) S_t and A = sum_t 2^(r_t - R) (T_t + (r_t - R) ln2 S_t),
  // both relative to R ln2: then lse = R ln2 + ln Z and H = ln Z - A / Z
  float Z = 0.f, A = 0.f;
  each([&](const float4 &v) {
    const int dr = tile_ref(v.x) - R;   // <= 0
    const float w = ldexpf(1.f, dr);
    Z += v.y * w;
    A += w * (v.z + (float)dr * kLn2 * v.y);
  });
  Z = wave_sum(Z);
  A = wave_sum(A);
  const float lnZ = __logf(Z);
  const float lse = (float)R * kLn2 + lnZ;
  if (lane == 0) {
    float H = lnZ - A / Z;
    if (H < 0.f) H = 0.f;
    if (a.conf) a.conf[row] = __expf(fmaf(-(float)R, kLn2, m)) / Z;   // e^(m - lse)
    if (a.entropy) a.entropy[row] = H;
    if (a.argmax) a.argmax[row] = id;
    if (a.rowstat) a.rowstat[row] = make_float2(m, lse);
    if (a.inv_z) a.inv_z[row] = 1.f / Z;
  }
  if (a.shift) {
#pragma unroll
    for (int q = 0; q < KC; ++q)
      if (lane + 64 * q < a.nvt) a.shift[row * a.nvt + lane + 64 * q] = R - tile_ref(vc[q].x);
    for (int t = lane + 64 * KC; t < a.nvt; t += 64) a.shift[row * a.nvt + t] = R - tile_ref(st[t].x);
  }
}

hipError_t launch_vocab_merge(const VocabMergeArgs &a, hipStream_t st) {
  if (a.nrows <= 0) return hipSuccess;
  hipLaunchKernelGGL(vocab_merge_kernel, dim3((unsigned)cdiv64(a.nrows, 4)), dim3(256), 0, st, a);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Entropy-bounded commit: one workgroup per canvas, one thread per position.
// rank = number of candidates ahead in (conf desc, position asc) order; the
// entropies are scattered to their ranks, an exclusive prefix is formed by a
// fixed Hillis-Steele scan in LDS, and rank k is accepted iff prefix_k <= tau.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(1024) void commit_kernel(CommitArgs a) {
  __shared__ __attribute__((aligned(16))) float sconf[DG_MAX_CANVAS];
  __shared__ float scan[2][DG_MAX_CANVAS];
  const int b = blockIdx.x, i = threadIdx.x, C = a.C, n = blockDim.x;
  const int64_t base = (int64_t)b * C;
  const bool live = i < C;
  int id = 0;
  float c = 0.f, H = 0.f;
  bool cand = false;
  if (live) {
    id = a.ids[base + i];
    cand = id == a.mask_id;
    c = a.conf[base + i];
    H = a.entropy[base + i];
  }
  // non-candidates (and padding threads) rank below every candidate
  sconf[i] = cand ? c : -INFINITY;
  scan[0][i] = 0.f;
  __syncthreads();
  int rank = 0;
  if (cand) {
    // rank = #{candidates j : c_j > c, or c_j == c and j < i}; four positions
    // per LDS read (a broadcast), no branches
    const float4 *s4 = reinterpret_cast<const float4 *>(sconf);
    int r0 = 0, r1 = 0, r2 = 0, r3 = 0;
#pragma unroll 4
    for (int j4 = 0; j4 < n / 4; ++j4) {
      const float4 q = s4[j4];
      const int j = 4 * j4;
      r0 += (q.x > c) | ((q.x == c) & (j < i));
      r1 += (q.y > c) | ((q.y == c) & (j + 1 < i));
      r2 += (q.z > c) | ((q.z == c) & (j + 2 < i));
      r3 += (q.w > c) | ((q.w == c) & (j + 3 < i));
    }
    rank = (r0 + r1) + (r2 + r3);
    scan[0][rank] = H;
  }
  __syncthreads();
  int src = 0;
  for (int off = 1; off < n; off <<= 1) {
    float x = scan[src][i];
    if (i >= off) x += scan[src][i - off];
    scan[src ^ 1][i] = x;
    __syncthreads();
    src ^= 1;
  }
  // scan[src] now holds the inclusive prefix in rank order
  bool accept = false;
  if (cand) {
    const float excl = rank == 0 ? 0.f : scan[src][rank - 1];
    accept = excl <= a.tau;
  }
  const int total = __syncthreads_count(accept);
  if (live) {
    a.mask[base + i] = accept ? 1 : 0;
    a.out_ids[base + i] = accept ? a.argmax[base + i] : id;
  }
  if (i == 0 && a.n_committed) a.n_committed[b] = total;
}

hipError_t launch_commit(const CommitArgs &a, hipStream_t st) {
  int n = 64;
  while (n < a.C) n <<= 1;
  hipLaunchKernelGGL(commit_kernel, dim3((unsigned)a.B), dim3((unsigned)n), 0, st, a);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// dst[c][r] = src[r][c]  (64 x 64 tiles through LDS)
// ---------------------------------------------------------------------------
template <typename T>
__global__ __launch_bounds__(256) void transpose_kernel(const T *src, T *dst, int rows, int cols) {
  __shared__ T tile[64][65];
  const int r0 = blockIdx.y * 64, c0 = blockIdx.x * 64;
  const int tx = threadIdx.x & 63, ty = threadIdx.x >> 6;
  for (int y = ty; y < 64; y += 4) {
    const int r = r0 + y, c = c0 + tx;
    if (r < rows && c < cols) tile[y][tx] = src[(int64_t)r * cols + c];
  }
  __syncthreads();
  for (int y = ty; y < 64; y += 4) {
    const int c = c0 + y, r = r0 + tx;
    if (r < rows && c < cols) dst[(int64_t)c * rows + r] = tile[tx][y];
  }
}

// [rows, cols] bf16 into blocks of 256 rows x 32 columns, 16 bytes per thread
__global__ __launch_bounds__(256) void tile_lm_kernel(const uint4 *src, uint4 *dst, int rows,
                                                      int cols) {
  const int64_t n = (int64_t)rows * cols / 8;
  const int cb = cols / 32;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256) {
    const int64_t r = i / (cols / 8);
    const int k = (int)(i % (cols / 8)) * 8;
    const int64_t o = ((r / 256) * cb + k / 32) * 8192 + (r % 256) * 32 + k % 32;
    dst[o / 8] = src[i];
  }
}

hipError_t launch_tile_lm(const void *src, void *dst, int rows, int cols, hipStream_t st) {
  if (rows % 256 || cols % 32) return hipErrorInvalidValue;
  const int64_t n = (int64_t)rows * cols / 8;
  const unsigned grid = (unsigned)(cdiv64(n, 256) < 65536 ? cdiv64(n, 256) : 65536);
  hipLaunchKernelGGL(tile_lm_kernel, dim3(grid), dim3(256), 0, st,
                     static_cast<const uint4 *>(src), static_cast<uint4 *>(dst), rows, cols);
  return hipGetLastError();
}

hipError_t launch_transpose(const void *src, void *dst, int rows, int cols, bool bf,
                            hipStream_t st) {
  dim3 grid((unsigned)cdiv64(cols, 64), (unsigned)cdiv64(rows, 64));
  if (bf)
    hipLaunchKernelGGL((transpose_kernel<bf16>), grid, dim3(256), 0, st,
                       static_cast<const bf16 *>(src), static_cast<bf16 *>(dst), rows, cols);
  else
    hipLaunchKernelGGL((transpose_kernel<float>), grid, dim3(256), 0, st,
                       static_cast<const float *>(src), static_cast<float *>(dst), rows, cols);
  return hipGetLastError();
}

// zero-fill with a kernel (kept out of memset nodes so callers can capture it)
__global__ __launch_bounds__(256) void clear_i32_kernel(int32_t *p, int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i < n) p[i] = 0;
}

hipError_t launch_clear_i32(int32_t *p, int64_t n, hipStream_t st) {
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(clear_i32_kernel, dim3((unsigned)cdiv64(n, 256)), dim3(256), 0, st, p, n);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Multi-step loop bookkeeping: one workgroup of 256 threads per canvas.
// ---------------------------------------------------------------------------
__device__ inline bool block_any(bool v) {
  __shared__ int any;
  if (threadIdx.x == 0) any = 0;
  __syncthreads();
  if (v) any = 1;   // every writer stores the same value
  __syncthreads();
  return any != 0;
}

__global__ __launch_bounds__(256) void loop_init_kernel(const int32_t *ids, int C, int mask_id,
                                                        int32_t *commit_step, int32_t *steps,
                                                        int32_t *active) {
  const int64_t base = (int64_t)blockIdx.x * C;
  bool has = false;
  for (int i = threadIdx.x; i < C; i += blockDim.x) {
    commit_step[base + i] = -1;
    has |= ids[base + i] == mask_id;
  }
  const bool a = block_any(has);
  if (threadIdx.x == 0) {
    steps[blockIdx.x] = 0;
    active[blockIdx.x] = a ? 1 : 0;
  }
}

__global__ __launch_bounds__(256) void loop_update_kernel(int32_t *ids, const int32_t *out_ids,
                                                          const uint8_t *mask, int C, int mask_id,
                                                          int t, int32_t *commit_step,
                                                          int32_t *steps, int32_t *active,
                                                          int32_t *n_active) {
  const int b = blockIdx.x;
  if (!active[b]) return;   // uniform per workgroup
  const int64_t base = (int64_t)b * C;
  bool has = false;
  for (int i = threadIdx.x; i < C; i += blockDim.x) {
    int id = ids[base + i];
    if (mask[base + i]) {
      id = out_ids[base + i];
      ids[base + i] = id;
      commit_step[base + i] = t;
    }
    has |= id == mask_id;
  }
  const bool a = block_any(has);
  if (threadIdx.x == 0) {
    steps[b] = t + 1;
    active[b] = a ? 1 : 0;
    if (a) atomicAdd(n_active, 1);
  }
}

hipError_t launch_loop_init(const int32_t *ids, int B, int C, int mask_id, int32_t *commit_step,
                            int32_t *steps, int32_t *active, hipStream_t st) {
  if (B <= 0) return hipSuccess;
  hipLaunchKernelGGL(loop_init_kernel, dim3(B), dim3(256), 0, st, ids, C, mask_id, commit_step,
                     steps, active);
  return hipGetLastError();
}

hipError_t launch_loop_update(int32_t *ids, const int32_t *out_ids, const uint8_t *mask, int B,
                              int C, int mask_id, int t, int32_t *commit_step, int32_t *steps,
                              int32_t *active, int32_t *n_active, hipStream_t st) {
  if (B <= 0) return hipSuccess;
  hipLaunchKernelGGL(loop_update_kernel, dim3(B), dim3(256), 0, st, ids, out_ids, mask, C,
                     mask_id, t, commit_step, steps, active, n_active);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// e4m3 (FP8) copy of the LM head: one workgroup per row.  The exponent e is the
// smallest integer with amax <= 448 * 2^e: with amax = m 2^E (1 <= m < 2) and
// 448 = 1.75 * 2^8, e = E - 8, plus 1 when m > 1.75.  Each value q = x * 2^-e
// (exact) is rounded to nearest, ties to even, in float32: below 2^-6 to a
// multiple of 2^-9 (a subnormal code; 8 * 2^-9 is the code of 2^-6 itself),
// otherwise to a 3-bit mantissa whose carry moves into the exponent field.
// ---------------------------------------------------------------------------
__device__ inline unsigned encode_e4m3(float q) {
  const unsigned sign = (__float_as_uint(q) >> 24) & 0x80u;
  const float a = fabsf(q);
  if (a < 0.015625f) return sign | (unsigned)rintf(a * 512.f);
  int x;
  frexpf(a, &x);                                   // a = f 2^x, 0.5 <= f < 1
  const int E = x - 1;
  const float frac = ldexpf(a, -E) - 1.f;          // exact
  int m3 = (int)rintf(frac * 8.f);
  int e = E;
  if (m3 == 8) { m3 = 0; e += 1; }
  return sign | (unsigned)(((e + 7) << 3) | m3);
}

__global__ __launch_bounds__(256) void quantize_e4m3_kernel(const bf16 *head, uint8_t *codes,
                                                            int32_t *exps, int cols) {
  const int64_t base = (int64_t)blockIdx.x * cols;
  __shared__ float red[256];
  float amax = 0.f;
  for (int k = threadIdx.x; k < cols; k += 256) amax = fmaxf(amax, fabsf(to_f(head[base + k])));
  red[threadIdx.x] = amax;
  __syncthreads();
  for (int o = 128; o > 0; o >>= 1) {
    if (threadIdx.x < o) red[threadIdx.x] = fmaxf(red[threadIdx.x], red[threadIdx.x + o]);
    __syncthreads();
  }
  amax = red[0];
  int e = 0;
  if (amax > 0.f) {
    int x;
    const float f = frexpf(amax, &x);
    e = (x - 1) - 8 + (2.f * f > 1.75f ? 1 : 0);
  }
  if (threadIdx.x == 0) exps[blockIdx.x] = e;
  for (int k = threadIdx.x; k < cols; k += 256)
    codes[base + k] = (uint8_t)encode_e4m3(ldexpf(to_f(head[base + k]), -e));
}

hipError_t launch_quantize_e4m3(const void *head, uint8_t *codes, int32_t *exps, int rows, int cols,
                                hipStream_t st) {
  if (rows <= 0 || cols <= 0) return hipSuccess;
  hipLaunchKernelGGL(quantize_e4m3_kernel, dim3(rows), dim3(256), 0, st,
                     static_cast<const bf16 *>(head), codes, exps, cols);
  return hipGetLastError();
}

}  // namespace dg
