// Structured slot read: label logprobs at decision slots, renormalisation over
// the allowed labels, entropy, and the averaged noise-draw re-read.
//
// The first pass projects q, k, v for the whole canvas (every key), and runs
// attention, the output projection, the LM head and its softmax statistics
// only at the slot rows (gathered by canvas position, compact rows); the LM
// head's epilogue also writes the logits of each slot's allowed labels.  A slot
// whose renormalised entropy exceeds the threshold flags its canvas; flagged
// canvases get n_draws copies with a noise token written at every slot and a
// second batched pass, decided on the device (no host synchronisation).  When
// the LM head's weight stream costs more than the draws' forward pass, the
// draws are instead computed for every canvas in the same pass as the first
// read and used only where a slot is flagged (same results, one weight stream).
#include <algorithm>

#include "common.h"
#include "kernels.h"

namespace dg {

__device__ inline int validate_slot(const SlotArgs &a, int64_t bs) {
  const int pos = a.slot_pos[bs];
  const int k = a.n_labels[bs];
  if (pos < 0 || pos >= a.C) return DG_SLOT_BAD_POS;
  if (k < 1 || k > DG_MAX_LABELS) return DG_SLOT_BAD_COUNT;
  // every label is loaded before any is tested (no exit per label, so the
  // loads are in flight together instead of one after another)
  const int32_t *labs = a.label_ids + bs * DG_MAX_LABELS;
  bool bad = false;
#pragma unroll
  for (int j = 0; j < DG_MAX_LABELS; ++j)
    if (j < k) {
      const int lab = labs[j];
      bad |= lab < 0 || lab >= a.V;
    }
  return bad ? DG_SLOT_BAD_LABEL : DG_SLOT_OK;
}

// rows of the first pass: slot (b, s) is row bs = b*S + s, at position pos of canvas b
__global__ __launch_bounds__(256) void slot_rows_kernel(SlotArgs a) {
  const int64_t bs = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (bs >= (int64_t)a.B * a.S) return;
  const int st = validate_slot(a, bs);
  a.status[bs] = st;
  const int64_t b = bs / a.S;
  const int pos = a.slot_pos[bs];
  const bool in = pos >= 0 && pos < a.C;
  // the LM-head row of the slot: its compact row, or (whole-canvas order) its
  // canvas row
  a.rows[bs] = st == DG_SLOT_OK ? (int32_t)(a.full_canvas ? b * a.C + pos : bs) : -1;
  a.qpos[bs] = in ? pos : -1;
  a.qids[bs] = in ? a.canvas_ids[b * a.C + pos] : 0;
}

// label log-probability in lane j: lp_j = min(l_j - lse, 0) from the scaled
// label logits the LM-head pass wrote for row n
__device__ inline float label_logprob(const SlotArgs &a, int64_t n, int k, int lane) {
  if (lane >= k) return -INFINITY;
  return fminf(a.lab_logit[n * DG_MAX_LABELS + lane] - a.rowstat[n].y, 0.f);
}

struct LabelDist {
  float r;      // renormalised probability in lane j (0 beyond k)
  float H;      // entropy of r (every lane)
  int best;     // lowest index of max r (every lane)
};

__device__ inline LabelDist renormalise(float lp, int k, int lane) {
  const bool on = lane < k;
  const float mx = wave_max(on ? lp : -INFINITY);
  const float e = on ? __expf(lp - mx) : 0.f;
  const float sum = wave_sum(e);
  LabelDist d;
  d.r = e / sum;
  return d;
}

__device__ inline void finish_dist(LabelDist &d, int k, int lane) {
  const bool on = lane < k;
  const float term = (on && d.r > 0.f) ? -d.r * __logf(d.r) : 0.f;
  d.H = fmaxf(wave_sum(term), 0.f);
  float bv = on ? d.r : -1.f;
  int bi = on ? lane : 0x7fffffff;
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    const float v2 = __shfl_xor(bv, o);
    const int i2 = __shfl_xor(bi, o);
    if (v2 > bv || (v2 == bv && i2 < bi)) { bv = v2; bi = i2; }
  }
  d.best = bi;
}

// First read of slot s of canvas b (one wave): outputs, and whether the slot
// is re-read (its flag is stored after the per-canvas flags).
__device__ bool slot_first_one(const SlotArgs &a, int b, int s, int lane) {
  const int64_t bs = (int64_t)b * a.S + s;
  float *lp_out = a.logprobs + bs * DG_MAX_LABELS;
  float *pr_out = a.probs + bs * DG_MAX_LABELS;
  if (a.status[bs] != DG_SLOT_OK) {
    if (lane < DG_MAX_LABELS) { lp_out[lane] = 0.f; pr_out[lane] = 0.f; }
    if (lane == 0) {
      a.entropy[bs] = 0.f;
      a.first_entropy[bs] = 0.f;
      a.best[bs] = -1;
      a.draws_used[bs] = 0;
      a.canvas_flag[a.B + bs] = 0;
    }
    return false;
  }
  const int k = a.n_labels[bs];
  const float lp = label_logprob(a, ((int64_t)b * a.grp_first) * a.S + s, k, lane);
  LabelDist dd = renormalise(lp, k, lane);
  finish_dist(dd, k, lane);
  if (lane < DG_MAX_LABELS) {
    lp_out[lane] = lane < k ? lp : 0.f;
    pr_out[lane] = lane < k ? dd.r : 0.f;
  }
  const bool flag = a.n_draws > 1 && dd.H > a.threshold;
  if (lane == 0) {
    a.entropy[bs] = dd.H;
    a.first_entropy[bs] = dd.H;
    a.best[bs] = dd.best;
    a.draws_used[bs] = 1;
    a.canvas_flag[a.B + bs] = flag ? 1 : 0;
  }
  return flag;
}

// first read: one wave per slot; also decides which canvases need draws
__global__ __launch_bounds__(1024) void slot_first_kernel(SlotArgs a) {
  __shared__ int any_flag;
  const int b = blockIdx.x;
  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63, nw = blockDim.x >> 6;
  if (threadIdx.x == 0) any_flag = 0;
  __syncthreads();
  for (int s = w; s < a.S; s += nw)
    if (slot_first_one(a, b, s, lane) && lane == 0) any_flag = 1;
  __syncthreads();
  if (threadIdx.x == 0) a.canvas_flag[b] = any_flag;
}

// draw canvases: copy of canvas b with noise_ids[d, b, s] at every slot position
__global__ __launch_bounds__(256) void slot_build_draws_kernel(SlotArgs a) {
  const int bd = blockIdx.x;
  const int b = bd / a.n_draws, d = bd % a.n_draws;
  const int act = a.canvas_flag[b];
  if (threadIdx.x == 0) a.draw_active[bd] = act;
  if (!act) return;
  int32_t *dst = a.draw_ids + (int64_t)bd * a.C;
  const int32_t *src = a.canvas_ids + (int64_t)b * a.C;
  __shared__ int last[DG_MAX_CANVAS];
  for (int i = threadIdx.x; i < a.C; i += 256) {
    dst[i] = src[i];
    last[i] = -1;
  }
  __syncthreads();
  // where two slots share a position the later one wins, as when the slots
  // are written in order (the highest slot index at each position, by LDS
  // atomics, then each winner writes)
  for (int s = threadIdx.x; s < a.S; s += 256) {
    const int pos = a.slot_pos[(int64_t)b * a.S + s];
    if (pos >= 0 && pos < a.C) atomicMax(&last[pos], s);
  }
  __syncthreads();
  for (int s = threadIdx.x; s < a.S; s += 256) {
    const int64_t bs = (int64_t)b * a.S + s;
    const int pos = a.slot_pos[bs];
    if (pos < 0 || pos >= a.C) continue;
    int nid = a.noise_ids[((int64_t)d * a.B + b) * a.S + s];
    if (nid < 0 || nid >= a.V) {
      nid = a.mask_id;
      if (a.status[bs] == DG_SLOT_OK) a.status[bs] = DG_SLOT_BAD_NOISE;
    }
    if (last[pos] == s) dst[pos] = nid;
  }
}

// rows of the draw pass: (b, d, s) is row i = (b*nd + d)*S + s, read when slot
// (b, s) is flagged; its query sits at the slot's position of draw canvas b*nd + d
__global__ __launch_bounds__(256) void slot_draw_rows_kernel(SlotArgs a, int32_t *row_active,
                                                             float *rs_draw) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t n = (int64_t)a.B * a.n_draws * a.S;
  if (i >= n) return;
  const int s = (int)(i % a.S);
  const int64_t bd = i / a.S;
  const int64_t b = bd / a.n_draws;
  const int64_t bs = b * a.S + s;
  const bool on = a.canvas_flag[a.B + bs] != 0;
  a.rows[i] = on ? (int32_t)(a.full_canvas ? bd * a.C + a.slot_pos[bs] : i) : -1;
  row_active[i] = on ? 1 : 0;
  rs_draw[i] = a.row_scale ? a.row_scale[bs] : 1.f;
  // draw canvases are written only for flagged canvases
  const int pos = a.slot_pos[bs];
  const bool in = pos >= 0 && pos < a.C && a.draw_active[bd];
  a.qpos[i] = in ? pos : -1;
  a.qids[i] = in ? a.draw_ids[bd * a.C + pos] : 0;
  // k, v of the slot row (its noise token) land at its position in the draw
  // canvas, whose other rows are copies of canvas b's
  if (a.kv_row_slot) a.kv_row_slot[i] = in ? (int32_t)(bd * a.C + pos) : -1;
}

// copies of canvas b's k, v rows (at canvas slot b*nd) into its other draws
// (slots b*nd + 1 .. b*nd + nd - 1), flagged canvases only; 16-byte chunks
__global__ __launch_bounds__(256) void slot_copy_kv_kernel(SlotArgs a, uint4 *k, uint4 *v,
                                                           int64_t canvas_chunks) {
  const int64_t b = blockIdx.y;
  if (!a.canvas_flag[b]) return;
  const int64_t src = b * a.n_draws * canvas_chunks;
  for (int64_t c = (int64_t)blockIdx.x * 256 + threadIdx.x; c < canvas_chunks;
       c += (int64_t)gridDim.x * 256) {
    const uint4 kk = k[src + c], vv = v[src + c];
    for (int j = 1; j < a.n_draws; ++j) {
      k[src + j * canvas_chunks + c] = kk;
      v[src + j * canvas_chunks + c] = vv;
    }
  }
}

// average of the draws in probability space: r = mean r_d, lp = ln mean e^(lp_d)
// (slot bs of a flagged canvas, one wave)
__device__ void slot_average_one(const SlotArgs &a, int64_t bs, int lane) {
  const int64_t b = bs / a.S;
  const int s = (int)(bs % a.S);
  const int k = a.n_labels[bs];
  // r is averaged directly; ln mean_d e^(lp_d) is kept as an online log-sum-exp
  // (lp can sit far below the fp32 range of e^x)
  float racc = 0.f, lm = -INFINITY, ls = 0.f;
  // the label logprobs of up to 8 draws are loaded before their reductions
  // (one memory wait per 8 draws); the draws are still summed in order
  constexpr int PD = 8;
  for (int d0 = 0; d0 < a.n_draws; d0 += PD) {
    float lpv[PD];
#pragma unroll
    for (int j = 0; j < PD; ++j)
      lpv[j] = d0 + j < a.n_draws
                   ? label_logprob(a, (b * a.grp_draw + a.off_draw + d0 + j) * a.S + s, k, lane)
                   : 0.f;
#pragma unroll
    for (int j = 0; j < PD; ++j) {
      if (d0 + j >= a.n_draws) break;
      const float lp = lpv[j];
      const LabelDist dd = renormalise(lp, k, lane);
      racc += dd.r;
      if (lane < k) {
        const float mn = fmaxf(lm, lp);
        ls = ls * __expf(lm - mn) + __expf(lp - mn);
        lm = mn;
      }
    }
  }
  LabelDist fin;
  fin.r = racc / (float)a.n_draws;
  finish_dist(fin, k, lane);
  if (lane < DG_MAX_LABELS) {
    a.logprobs[bs * DG_MAX_LABELS + lane] =
        lane < k ? lm + __logf(ls) - __logf((float)a.n_draws) : 0.f;
    a.probs[bs * DG_MAX_LABELS + lane] = lane < k ? fin.r : 0.f;
  }
  if (lane == 0) {
    a.entropy[bs] = fin.H;
    a.best[bs] = fin.best;
    a.draws_used[bs] = a.n_draws;
  }
}

__global__ __launch_bounds__(256) void slot_average_kernel(SlotArgs a) {
  const int64_t bs = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (bs >= (int64_t)a.B * a.S) return;
  if (!a.canvas_flag[a.B + bs]) return;
  slot_average_one(a, bs, threadIdx.x & 63);
}

// The rest of a one-pass read for canvas b in one workgroup: first read of
// every slot, the canvas's re-read flag, the status of slots whose noise id is
// out of range (re-read canvases only), and the average of the flagged slots.
__global__ __launch_bounds__(1024) void slot_finish_kernel(SlotArgs a) {
  __shared__ int any_flag;
  const int b = blockIdx.x;
  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63, nw = blockDim.x >> 6;
  if (threadIdx.x == 0) any_flag = 0;
  __syncthreads();
  for (int s = w; s < a.S; s += nw)
    if (slot_first_one(a, b, s, lane) && lane == 0) any_flag = 1;
  __syncthreads();
  const bool flagged = any_flag != 0;
  if (threadIdx.x == 0) a.canvas_flag[b] = flagged ? 1 : 0;
  if (!flagged) return;
  for (int s = threadIdx.x; s < a.S; s += blockDim.x) {
    const int64_t bs = (int64_t)b * a.S + s;
    if (a.status[bs] != DG_SLOT_OK) continue;
    for (int d = 0; d < a.n_draws; ++d) {
      const int nid = a.noise_ids[((int64_t)d * a.B + b) * a.S + s];
      if (nid < 0 || nid >= a.V) { a.status[bs] = DG_SLOT_BAD_NOISE; break; }
    }
  }
  for (int s = w; s < a.S; s += nw) {
    const int64_t bs = (int64_t)b * a.S + s;
    if (a.canvas_flag[a.B + bs]) slot_average_one(a, bs, lane);
  }
}

// One pass over the first read and every draw.  Block cb = b*(1+nd) + j
// writes canvas cb: canvas b itself (j = 0) or draw j-1 of it, with its noise
// token at every valid slot position (the mask id for an out-of-range noise
// id; the status for that is set only once the canvas is known to re-read).
// It also writes, for the canvas's slot rows n = cb*S + s, the LM-head row
// (n, or -1 for an invalid slot), the row scale, the query position and the
// token id there, and for j = 0 the slot's validation status.
__global__ __launch_bounds__(256) void slot_spec_build_kernel(SlotArgs a, int32_t *ids, float *rs) {
  const int cb = blockIdx.x;
  const int G = a.n_draws + 1;
  const int b = cb / G, j = cb % G;
  int32_t *dst = ids + (int64_t)cb * a.C;
  const int32_t *src = a.canvas_ids + (int64_t)b * a.C;
  for (int i = threadIdx.x; i < a.C; i += 256) dst[i] = src[i];
  __syncthreads();
  for (int s = threadIdx.x; s < a.S; s += 256) {
    const int64_t bs = (int64_t)b * a.S + s;
    const int st = validate_slot(a, bs);
    if (j == 0) a.status[bs] = st;
    const int64_t n = (int64_t)cb * a.S + s;
    a.rows[n] = st == DG_SLOT_OK ? (int32_t)(a.full_canvas ? (int64_t)cb * a.C + a.slot_pos[bs] : n) : -1;
    rs[n] = a.row_scale ? a.row_scale[bs] : 1.f;
  }
  // the draw's noise ids at the slot positions; where two slots share a
  // position the later one wins, as when the slots are written in order (the
  // highest slot index at each position is found with LDS atomics, then each
  // winner writes)
  if (j > 0) {
    __shared__ int last[DG_MAX_CANVAS];
    for (int i = threadIdx.x; i < a.C; i += 256) last[i] = -1;
    __syncthreads();
    for (int s = threadIdx.x; s < a.S; s += 256) {
      const int pos = a.slot_pos[(int64_t)b * a.S + s];
      if (pos >= 0 && pos < a.C) atomicMax(&last[pos], s);
    }
    __syncthreads();
    for (int s = threadIdx.x; s < a.S; s += 256) {
      const int pos = a.slot_pos[(int64_t)b * a.S + s];
      if (pos < 0 || pos >= a.C || last[pos] != s) continue;
      int nid = a.noise_ids[((int64_t)(j - 1) * a.B + b) * a.S + s];
      if (nid < 0 || nid >= a.V) nid = a.mask_id;
      dst[pos] = nid;
    }
  }
  __syncthreads();
  for (int s = threadIdx.x; s < a.S; s += 256) {
    const int pos = a.slot_pos[(int64_t)b * a.S + s];
    const bool in = pos >= 0 && pos < a.C;
    const int64_t n = (int64_t)cb * a.S + s;
    a.qpos[n] = in ? pos : -1;
    a.qids[n] = in ? dst[pos] : 0;
    // k, v of a draw's slot row land in the draw canvas; canvas b itself gets
    // every row from the base projection
    if (a.kv_row_slot) a.kv_row_slot[n] = in && j > 0 ? (int32_t)((int64_t)cb * a.C + pos) : -1;
  }
  if (j == 0 && a.kv_row_base)
    for (int i = threadIdx.x; i < a.C; i += 256)
      a.kv_row_base[(int64_t)b * a.C + i] = (int32_t)((int64_t)cb * a.C + i);
  if (j == 0 && a.win_pos) {
    // the positions within +-W of any of canvas b's in-range slots, ascending,
    // then the same rows in the projection's list at a range taken from the
    // running total.  Each slot adds +1 at its window's first position and -1
    // past its last; a position is in a window where the running sum of these
    // marks is positive (a scan per 256 positions), and a ballot with the
    // per-wave counts places it.
    __shared__ int cover[DG_MAX_CANVAS + 1];
    __shared__ int wsum[4], wtot[4];
    __shared__ int wbase;
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
    for (int i = threadIdx.x; i <= a.C; i += 256) cover[i] = 0;
    __syncthreads();
    for (int s = threadIdx.x; s < a.S; s += 256) {
      const int q = a.slot_pos[(int64_t)b * a.S + s];
      if (q >= 0 && q < a.C) {   // (W <= C - 1, so q + W does not overflow)
        atomicAdd(&cover[q - a.W > 0 ? q - a.W : 0], 1);
        atomicAdd(&cover[(q + a.W < a.C - 1 ? q + a.W : a.C - 1) + 1], -1);
      }
    }
    __syncthreads();
    int total = 0, run = 0;   // run: the marks before the chunk
    for (int c0 = 0; c0 < a.C; c0 += 256) {
      const int p = c0 + threadIdx.x;
      int x = p < a.C ? cover[p] : 0;
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) {
        const int y = __shfl_up(x, o);
        if (lane >= o) x += y;
      }
      if (lane == 63) wtot[wv] = x;
      __syncthreads();
      int pre = run;
      for (int i = 0; i < wv; ++i) pre += wtot[i];
      const bool in = p < a.C && pre + x > 0;
      const uint64_t m = __ballot(in);
      if (lane == 0) wsum[wv] = __popcll(m);
      __syncthreads();
      int off = total;
      for (int i = 0; i < wv; ++i) off += wsum[i];
      if (in) a.win_pos[(int64_t)b * a.C + off + __popcll(m & ((1ull << lane) - 1))] = p;
      total += wsum[0] + wsum[1] + wsum[2] + wsum[3];
      run += wtot[0] + wtot[1] + wtot[2] + wtot[3];
      __syncthreads();
    }
    if (threadIdx.x == 0) {
      a.win_cnt[b] = total;
      wbase = atomicAdd(a.win_total, total);
    }
    __syncthreads();
    for (int k = threadIdx.x; k < total; k += 256) {
      const int p = a.win_pos[(int64_t)b * a.C + k];
      a.win_ids[wbase + k] = a.canvas_ids[(int64_t)b * a.C + p];
      a.win_rows[wbase + k] = (int32_t)((int64_t)b * a.C + p);
    }
  }
}


hipError_t launch_slot_spec_build(const SlotArgs &a, int32_t *ids, float *rs, hipStream_t st) {
  const int64_t n = (int64_t)a.B * (a.n_draws + 1);
  if (n == 0) return hipSuccess;
  hipLaunchKernelGGL(slot_spec_build_kernel, dim3((unsigned)n), dim3(256), 0, st, a, ids, rs);
  return hipGetLastError();
}

// one wave per slot of a canvas, 1 to 16 waves
static unsigned slot_wave_threads(int S) { return 64u * (unsigned)(S < 1 ? 1 : S > 16 ? 16 : S); }

hipError_t launch_slot_finish(const SlotArgs &a, hipStream_t st) {
  if (a.B == 0) return hipSuccess;
  hipLaunchKernelGGL(slot_finish_kernel, dim3((unsigned)a.B), dim3(slot_wave_threads(a.S)), 0, st, a);
  return hipGetLastError();
}

hipError_t launch_slot_rows(const SlotArgs &a, hipStream_t st) {
  const int64_t n = (int64_t)a.B * a.S;
  if (n == 0) return hipSuccess;
  hipLaunchKernelGGL(slot_rows_kernel, dim3((unsigned)cdiv64(n, 256)), dim3(256), 0, st, a);
  return hipGetLastError();
}

hipError_t launch_slot_first(const SlotArgs &a, hipStream_t st) {
  if (a.B == 0) return hipSuccess;
  hipLaunchKernelGGL(slot_first_kernel, dim3((unsigned)a.B), dim3(slot_wave_threads(a.S)), 0, st, a);
  return hipGetLastError();
}

hipError_t launch_slot_build_draws(const SlotArgs &a, hipStream_t st) {
  hipLaunchKernelGGL(slot_build_draws_kernel, dim3((unsigned)(a.B * a.n_draws)), dim3(256), 0, st, a);
  return hipGetLastError();
}

hipError_t launch_slot_draw_rows2(const SlotArgs &a, int32_t *row_active, float *rs_draw,
                                  hipStream_t st) {
  const int64_t n = (int64_t)a.B * a.n_draws * a.S;
  if (n == 0) return hipSuccess;
  hipLaunchKernelGGL(slot_draw_rows_kernel, dim3((unsigned)cdiv64(n, 256)), dim3(256), 0, st, a,
                     row_active, rs_draw);
  return hipGetLastError();
}

hipError_t launch_slot_copy_kv(const SlotArgs &a, void *k, void *v, int64_t kv_row_bytes,
                               hipStream_t st) {
  if (a.B == 0 || a.n_draws < 2) return hipSuccess;
  if (kv_row_bytes % 16) return hipErrorInvalidValue;
  const int64_t chunks = (int64_t)a.C * kv_row_bytes / 16;
  const unsigned gx = (unsigned)std::min<int64_t>(cdiv64(chunks, 256), 16);
  hipLaunchKernelGGL(slot_copy_kv_kernel, dim3(gx, (unsigned)a.B), dim3(256), 0, st, a,
                     static_cast<uint4 *>(k), static_cast<uint4 *>(v), chunks);
  return hipGetLastError();
}

hipError_t launch_slot_average(const SlotArgs &a, hipStream_t st) {
  const int64_t n = (int64_t)a.B * a.S;
  if (n == 0) return hipSuccess;
  hipLaunchKernelGGL(slot_average_kernel, dim3((unsigned)cdiv64(n, 4)), dim3(256), 0, st, a);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Two-stage reads (one workgroup per canvas, one thread per stage slot)
// ---------------------------------------------------------------------------
__device__ inline bool staged_asked(const StagedArgs &a, int b, int j) {
  const int c = a.ask_slot[j];
  if (c < 0) return true;
  const int64_t bc = (int64_t)b * a.S + c;
  return a.status[bc] == DG_SLOT_OK && a.best[bc] == a.ask_label[j];
}

__global__ __launch_bounds__(64) void staged_gather_kernel(StagedArgs a) {
  const int b = blockIdx.x, j = threadIdx.x;
  if (j >= a.n) return;
  const int s = a.idx[j];
  const int64_t from = (int64_t)b * a.S + s, to = (int64_t)b * a.n + j;
  a.pos_s[to] = a.slot_pos[from];
  a.nlab_s[to] = staged_asked(a, b, j) ? a.n_labels[from] : 1;
  for (int q = 0; q < DG_MAX_LABELS; ++q)
    a.lab_s[to * DG_MAX_LABELS + q] = a.label_ids[from * DG_MAX_LABELS + q];
  if (a.noise_ids)
    for (int d = 0; d < a.nd; ++d)
      a.noise_s[((int64_t)d * a.B + b) * a.n + j] = a.noise_ids[((int64_t)d * a.B + b) * a.S + s];
  if (a.row_scale) a.rs_s[to] = a.row_scale[from];
}

__global__ __launch_bounds__(64) void staged_scatter_kernel(StagedArgs a) {
  const int b = blockIdx.x, j = threadIdx.x;
  if (j >= a.n) return;
  const int s = a.idx[j];
  const int64_t to = (int64_t)b * a.S + s, from = (int64_t)b * a.n + j;
  const bool asked = staged_asked(a, b, j);
  for (int q = 0; q < DG_MAX_LABELS; ++q) {
    a.logprobs[to * DG_MAX_LABELS + q] = asked ? a.lp_s[from * DG_MAX_LABELS + q] : 0.f;
    a.probs[to * DG_MAX_LABELS + q] = asked ? a.pr_s[from * DG_MAX_LABELS + q] : 0.f;
  }
  a.entropy[to] = asked ? a.ent_s[from] : 0.f;
  a.first_entropy[to] = asked ? a.fent_s[from] : 0.f;
  a.best[to] = asked ? a.best_s[from] : -1;
  a.draws_used[to] = asked ? a.draws_s[from] : 0;
  a.status[to] = asked ? a.status_s[from] : DG_SLOT_NOT_ASKED;
}

__global__ __launch_bounds__(256) void staged_pin_kernel(StagedArgs a) {
  const int b = blockIdx.x;
  const int64_t base = (int64_t)b * a.C;
  for (int i = threadIdx.x; i < a.C; i += 256) a.pinned[base + i] = a.canvas[base + i];
  __syncthreads();
  if (threadIdx.x != 0) return;
  // in slot order, so a later slot at the same position wins
  for (int j = 0; j < a.n; ++j) {
    const int64_t bs = (int64_t)b * a.S + a.idx[j];
    if (a.status[bs] != DG_SLOT_OK) continue;
    const int pos = a.slot_pos[bs], k = a.best[bs];
    if (pos < 0 || pos >= a.C || k < 0 || k >= DG_MAX_LABELS) continue;
    a.pinned[base + pos] = a.label_ids[bs * DG_MAX_LABELS + k];
  }
}

hipError_t launch_staged_gather(const StagedArgs &a, hipStream_t st) {
  if (a.B <= 0 || a.n <= 0) return hipSuccess;
  hipLaunchKernelGGL(staged_gather_kernel, dim3(a.B), dim3(64), 0, st, a);
  return hipGetLastError();
}
hipError_t launch_staged_scatter(const StagedArgs &a, hipStream_t st) {
  if (a.B <= 0 || a.n <= 0) return hipSuccess;
  hipLaunchKernelGGL(staged_scatter_kernel, dim3(a.B), dim3(64), 0, st, a);
  return hipGetLastError();
}
hipError_t launch_staged_pin(const StagedArgs &a, hipStream_t st) {
  if (a.B <= 0) return hipSuccess;
  hipLaunchKernelGGL(staged_pin_kernel, dim3(a.B), dim3(256), 0, st, a);
  return hipGetLastError();
}

}  // namespace dg
