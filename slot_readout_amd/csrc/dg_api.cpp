// C-ABI entry points: host-side validation, workspace planning and the launch
// sequence of each call.  Nothing here allocates device memory; only the
// multi-step loop synchronises the host (every check_every steps, to stop once
// no canvas holds a mask id).
#include <algorithm>
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <string>

#include "dg.h"
#include "kernels.h"

namespace {

thread_local std::string g_err;

dg_status fail(dg_status s, const char *fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_err = buf;
  return s;
}

dg_status ok() {
  g_err.clear();
  return DG_OK;
}

dg_status hip_check(hipError_t e, const char *what) {
  if (e == hipSuccess) return DG_OK;
  return fail(DG_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

#define DG_TRY_HIP(expr, what)                       \
  do {                                               \
    dg_status _s = hip_check((expr), (what));        \
    if (_s != DG_OK) return _s;                      \
  } while (0)

bool aligned16(const void *p) { return p == nullptr || (reinterpret_cast<uintptr_t>(p) & 15) == 0; }

size_t tsize(const dg_dims &d) { return d.dtype == DG_BF16 ? 2 : 4; }

dg_status check_dims(const dg_dims *d) {
  if (!d) return fail(DG_ERR_INVALID_ARG, "dims is NULL");
  if (d->dtype != DG_F32 && d->dtype != DG_BF16)
    return fail(DG_ERR_UNSUPPORTED, "dtype %d is neither DG_F32 nor DG_BF16", d->dtype);
  if (d->head_dim != 64 && d->head_dim != 512)
    return fail(DG_ERR_UNSUPPORTED, "head_dim %d: supported head widths are 64 and 512", d->head_dim);
  if (d->head_dim == 512 && d->dtype == DG_F32)
    return fail(DG_ERR_UNSUPPORTED, "head_dim 512 is supported with bf16 storage only");
  if (d->d_model <= 0 || d->d_model % 32 != 0)
    return fail(DG_ERR_INVALID_ARG, "d_model %d must be a positive multiple of 32", d->d_model);
  // bf16 projections step through d_model 64 columns at a time
  if (d->dtype == DG_BF16 && d->d_model % 64 != 0)
    return fail(DG_ERR_UNSUPPORTED, "bf16 storage needs d_model %d to be a multiple of 64", d->d_model);
  if (d->n_kv_heads <= 0 || d->n_q_heads <= 0 || d->n_q_heads % d->n_kv_heads != 0)
    return fail(DG_ERR_INVALID_ARG, "n_q_heads %d must be a positive multiple of n_kv_heads %d",
                d->n_q_heads, d->n_kv_heads);
  if (d->vocab <= 0 || d->vocab % dg::VTILE != 0)
    return fail(DG_ERR_INVALID_ARG, "vocab %d must be a positive multiple of %d", d->vocab, dg::VTILE);
  if (d->canvas < 1 || d->canvas > DG_MAX_CANVAS)
    return fail(DG_ERR_INVALID_ARG, "canvas %d outside [1, %d]", d->canvas, DG_MAX_CANVAS);
  if (d->window < 0) return fail(DG_ERR_INVALID_ARG, "window %d < 0", d->window);
  if (d->mask_id < 0 || d->mask_id >= d->vocab)
    return fail(DG_ERR_INVALID_ARG, "mask_id %d outside [0, vocab)", d->mask_id);
  return DG_OK;
}

// Size limits shared by the calls and their workspace queries: canvas rows
// (batch * canvas, times the canvases per batch entry of a read) and slot rows
// are addressed as int32, and prompt lengths leave room for the attention
// plan's key spans.
constexpr int64_t kMaxRows = INT32_MAX;
constexpr int32_t kMaxPrompt = 1 << 30;

bool sizes_fit(const dg_dims &d, int64_t canvases, int32_t max_prompt, int64_t slot_rows = 0) {
  return canvases * d.canvas <= kMaxRows && slot_rows <= kMaxRows && max_prompt <= kMaxPrompt;
}

dg_status check_sizes(const dg_dims &d, int64_t canvases, int32_t max_prompt, int64_t slot_rows = 0) {
  if (sizes_fit(d, canvases, max_prompt, slot_rows)) return DG_OK;
  return fail(DG_ERR_INVALID_ARG,
              "sizes out of range: %lld canvases of %d rows, %lld slot rows (at most 2^31 - 1 rows), "
              "max_prompt %d (at most 2^30)",
              (long long)canvases, d.canvas, (long long)slot_rows, max_prompt);
}

dg_status check_model(const dg_dims *d, int32_t batch, int32_t max_prompt, const dg_weights *w,
                      const dg_prompt_kv *kv) {
  dg_status s = check_dims(d);
  if (s != DG_OK) return s;
  if (batch < 0) return fail(DG_ERR_INVALID_ARG, "batch %d < 0", batch);
  if (max_prompt < 0) return fail(DG_ERR_INVALID_ARG, "max_prompt %d < 0", max_prompt);
  s = check_sizes(*d, batch, max_prompt);
  if (s != DG_OK) return s;
  if (!w) return fail(DG_ERR_INVALID_ARG, "weights is NULL");
  if (!w->embed || !w->wq || !w->wk || !w->wv || !w->wo)
    return fail(DG_ERR_INVALID_ARG, "embed, wq, wk, wv and wo are required");
  if (!kv) return fail(DG_ERR_INVALID_ARG, "prompt_kv is NULL");
  if (!kv->cu_seqlens) return fail(DG_ERR_INVALID_ARG, "prompt_kv.cu_seqlens is NULL");
  if (kv->max_len < 0 || kv->total_len < 0)
    return fail(DG_ERR_INVALID_ARG, "prompt_kv max_len/total_len must be >= 0");
  if (kv->max_len > max_prompt)
    return fail(DG_ERR_INVALID_ARG, "prompt_kv.max_len %d exceeds the planned max_prompt %d",
                kv->max_len, max_prompt);
  if (kv->max_len > 0 && (!kv->k || !kv->v))
    return fail(DG_ERR_INVALID_ARG, "prompt_kv.k/v are NULL but max_len > 0");
  const void *ptrs[] = {w->embed, w->embed_t, w->lm_head, w->wq, w->wk, w->wv, w->wo, w->lm_tiled,
                        w->embed_t_tiled, w->lm_fp8, w->lm_fp8_exp, kv->k, kv->v};
  for (const void *p : ptrs)
    if (!aligned16(p)) return fail(DG_ERR_INVALID_ARG, "weight / KV pointers must be 16-byte aligned");
  if (w->lm_fp8 && d->dtype != DG_BF16)
    return fail(DG_ERR_UNSUPPORTED, "the e4m3 LM head (weights.lm_fp8) needs bf16 storage");
  if (!w->lm_fp8 != !w->lm_fp8_exp)
    return fail(DG_ERR_INVALID_ARG, "weights.lm_fp8 and lm_fp8_exp go together");
  if (w->lm_fp8_act && !w->lm_fp8)
    return fail(DG_ERR_INVALID_ARG, "weights.lm_fp8_act needs the e4m3 head (lm_fp8)");
  if (w->lm_fp8_act && d->d_model % 128)
    return fail(DG_ERR_UNSUPPORTED, "FP8 activations need d_model a multiple of 128 (got %d)",
                d->d_model);
  return DG_OK;
}

// A window of C - 1 or more already reaches every canvas key, so the kernels
// take min(W, C - 1): the same keys, and no int overflow in the window bounds
// for a W near INT_MAX (a natural way to ask for full attention).
int window_of(const dg_dims &d) { return d.window < d.canvas - 1 ? d.window : d.canvas - 1; }

struct Arena {
  size_t off = 0;
  size_t take(size_t bytes) {
    const size_t o = off;
    off += (bytes + 255) & ~size_t(255);
    return o;
  }
};

struct AttnPlan {
  int nsplit = 1, chunk = 64;
  size_t part_o = 0, part_ml = 0;
};

// qn queries per canvas: every position, or qn gathered ones; prec: fp32
// partials (the split-probability attention of slot reads)
// cpp: consecutive canvases sharing a prompt (gathered queries of such
// canvases may share a tile)
AttnPlan plan_attention(const dg_dims &d, int nc, int max_prompt, int qn = -1, bool prec = false,
                        int cpp = 1) {
  AttnPlan p;
  const bool gathered = qn >= 0;
  if (!gathered) qn = d.canvas;
  int bound = 1;
  dg::attn_plan(nc, d.canvas, qn, gathered, d.n_q_heads, d.n_kv_heads, window_of(d), d.head_dim,
                max_prompt, cpp, &p.nsplit, &p.chunk, &bound);
  // partials sized by the bound, so that a workspace planned for max_prompt
  // also holds the partials of every shorter prompt (the rounded split count
  // is not monotone in the prompt length)
  if (bound > 1) {
    const size_t R = (size_t)nc * d.n_q_heads * qn;
    p.part_o = (size_t)bound * R * d.head_dim * (prec ? sizeof(float) : tsize(d));
    p.part_ml = (size_t)bound * R * sizeof(float2);
  }
  return p;
}

// fp32 split-K partials of a projection of M rows x ncols outputs over K (0: unsplit)
size_t proj_part_bytes(const dg_dims &d, int64_t M, int64_t ncols, int K) {
  const int ks = dg::proj_ksplit(M, ncols, K, d.dtype == DG_BF16);
  return ks > 1 ? (size_t)ks * M * ncols * sizeof(float) : 0;
}

struct StepPlan {
  size_t q, k, v, o, part_o, part_ml, proj_part, h, hq, hexp, stats, ptilde, shift, inv_z, sc_part,
      total;
  AttnPlan attn;
  int ksplit;
};

StepPlan plan_step(const dg_dims &d, int B, int max_prompt) {
  StepPlan p{};
  const size_t M = (size_t)B * d.canvas, ts = tsize(d);
  const size_t nq = (size_t)d.n_q_heads * d.head_dim, nkv = (size_t)d.n_kv_heads * d.head_dim;
  const int nvt = d.vocab / dg::VTILE;
  const bool bf = d.dtype == DG_BF16;
  Arena a;
  p.q = a.take(M * nq * ts);
  p.k = a.take(M * nkv * ts);
  p.v = a.take(M * nkv * ts);
  p.o = a.take(M * nq * ts);
  p.attn = plan_attention(d, B, max_prompt);
  p.part_o = a.take(p.attn.part_o);
  p.part_ml = a.take(p.attn.part_ml);
  p.proj_part = a.take(std::max(proj_part_bytes(d, M, nq + 2 * nkv, d.d_model),
                                proj_part_bytes(d, M, d.d_model, (int)nq)));
  p.h = a.take(M * d.d_model * ts);
  // e4m3 codes and exponents of h (FP8 activations; bf16 only)
  p.hq = a.take(bf ? M * d.d_model : 0);
  p.hexp = a.take(bf ? M * sizeof(int32_t) : 0);
  p.stats = a.take(M * nvt * sizeof(float4));
  // bf16 p~ is stored in blocks of 256 rows: whole row blocks are allocated
  p.ptilde = a.take((bf ? (M + 255) / 256 * 256 : M) * d.vocab * ts);
  p.shift = a.take(M * nvt * sizeof(int32_t));
  p.inv_z = a.take(M * sizeof(float));
  p.ksplit = dg::sc_ksplit((int64_t)M, d.d_model, d.vocab, bf);
  p.sc_part = a.take(p.ksplit > 1 ? (size_t)p.ksplit * M * d.d_model * sizeof(float) : 0);
  p.total = a.off;
  return p;
}

// Workspace of the multi-step loop: a step's workspace, then the loop state.
struct LoopPlan {
  StepPlan step;
  size_t conf, entropy, argmax, sc0, sc1, cmask, out_ids, n_commit, active, n_active, total;
};

LoopPlan plan_loop(const dg_dims &d, int B, int max_prompt) {
  LoopPlan p{};
  p.step = plan_step(d, B, max_prompt);
  const size_t M = (size_t)B * d.canvas;
  Arena a;
  a.off = (p.step.total + 255) & ~size_t(255);
  p.conf = a.take(M * sizeof(float));
  p.entropy = a.take(M * sizeof(float));
  p.argmax = a.take(M * sizeof(int32_t));
  p.sc0 = a.take(M * d.d_model * tsize(d));
  p.sc1 = a.take(M * d.d_model * tsize(d));
  p.cmask = a.take(M);
  p.out_ids = a.take(M * sizeof(int32_t));
  p.n_commit = a.take((size_t)B * sizeof(int32_t));
  p.active = a.take((size_t)B * sizeof(int32_t));
  p.n_active = a.take(sizeof(int32_t));
  p.total = a.off;
  return p;
}

struct SlotPlan {
  size_t q, k, v, o, part_o, part_ml, proj_part, h, rows, qpos, qids, kv_row_base, kv_row_slot, stats,
      rowstat, lab_logit, flags, draw_active, draw_ids, row_active, rs_draw, kpatch, vpatch, win_pos,
      win_cnt, win_ids, win_rows, win_total, total;
  AttnPlan first, draws;
  bool spec, prec, full, patch;
};

// Whether the draws are computed for every canvas in the first read's pass.
// That saves one stream of the LM-head weights (V x d), and costs the draws'
// forward pass when no slot turns out to need a re-read: the q/k/v projection
// of every canvas row, attention over the prompt and the canvas for the slot
// rows (a whole query tile of them), and the output projection of the slot
// rows.  Both are estimated with sustained rates of about 5 TB/s and
// 1 PFLOP/s (bf16; 0.1 PFLOP/s fp32).
// (full: the whole-canvas order, whose draws run q, attention and the output
// projection over every canvas row)
// With patched draws (slot-row order, head_dim 64 bf16) the draws of a canvas
// project only their slot rows and read the base canvas's k, v, and their
// gathered queries share the prompt's attention tile with the first read's; a
// second pass, on the other hand, streams every prompt again. So there the
// draws' slot-row projections and attention are weighed against the LM-head
// stream plus a second stream of the prompts' k, v. (For the 512-canvas read
// batch with 1,024-token prompts the one pass measured 0.55 ms against 0.69 ms
// when every canvas re-reads, and 0.525 against 0.533 ms when none does.)
bool speculate_draws(const dg_dims &d, int B, int S, int nd, int max_prompt, bool full = false) {
  if (nd <= 1 || B <= 0) return false;
  const double head_s = (double)d.vocab * d.d_model * (double)tsize(d) / 5e12;
  const double hq = (double)d.n_q_heads * d.head_dim, hkv = (double)d.n_kv_heads * d.head_dim;
  if (!full && dg::attn_patch_supported(d.head_dim, d.dtype == DG_BF16, S)) {
    const double per_draw = 2.0 * d.d_model * (hq + 2.0 * hkv) * S + 2.0 * hq * d.d_model * S +
                            4.0 * hq * ((double)max_prompt + d.canvas) * S;
    const double draw_s = (double)B * nd * per_draw / 1e15;
    const double kv_s = (double)B * max_prompt * 2.0 * hkv * (double)tsize(d) / 5e12;
    return draw_s < head_s + kv_s;
  }
  const int qt = dg::attn_query_tile(d.head_dim);
  const double s_att = full ? (double)d.canvas : (double)((S + qt - 1) / qt) * qt;
  const double per_canvas = 2.0 * d.d_model * (hq + 2.0 * hkv) * d.canvas +
                            2.0 * hq * d.d_model * (full ? d.canvas : S) +
                            4.0 * hq * ((double)max_prompt + d.canvas) * s_att;
  const double draw_s = (double)B * nd * per_canvas / (d.dtype == DG_BF16 ? 1e15 : 1e14);
  return draw_s < head_s;
}

// A read needs the hidden state only at its slot rows: the k/v projection runs
// over every canvas row (all keys); the q projection, attention and the output
// projection over the slot rows alone (gathered queries, compact rows).  The
// whole-canvas order (full) runs q, attention and the output projection over
// every canvas row, as the layers below the last one of a deeper model need,
// and the LM head at the slot rows.
// spec: -1 decides by speculate_draws, 0 / 1 forces the two-pass / one-pass order
SlotPlan plan_slot(const dg_dims &d, int B, int S, int max_prompt, int nd, int spec = -1,
                   bool full = false) {
  SlotPlan p{};
  p.spec = spec < 0 ? speculate_draws(d, B, S, nd, max_prompt, full) : spec != 0;
  p.full = full;
  // bf16 slot rows carry the attention output in fp32 and the hidden state
  // as bf16 hi | lo halves (see read_prec)
  const bool prec = d.dtype == DG_BF16;
  p.prec = prec;
  // patched draws (slot-row order, head_dim 64 bf16): the draws read their
  // base canvas's k, v with their own slot rows in place, so only the base
  // canvases' k, v are stored, plus the draws' slot rows
  p.patch = !full && nd > 1 && dg::attn_patch_supported(d.head_dim, d.dtype == DG_BF16, S);
  const int ncmax = p.spec ? B * (nd + 1) : (nd > 1 ? B * nd : B);
  const size_t M = (size_t)ncmax * d.canvas, ts = tsize(d);
  const size_t kvrows = p.patch ? (size_t)B * d.canvas : M;   // rows of k, v
  const size_t nq = (size_t)d.n_q_heads * d.head_dim, nkv = (size_t)d.n_kv_heads * d.head_dim;
  const int nvt = d.vocab / dg::VTILE;
  const size_t nrows = (size_t)B * S * (p.spec ? nd + 1 : (nd > 1 ? nd : 1));
  // rows of q, o and h: the slot rows, or every canvas row (full)
  const size_t hrows = full ? M : nrows;
  Arena a;
  p.q = a.take(hrows * nq * ts);
  p.k = a.take(kvrows * nkv * ts);
  p.v = a.take(kvrows * nkv * ts);
  p.kpatch = a.take(p.patch ? nrows * nkv * ts : 0);
  p.vpatch = a.take(p.patch ? nrows * nkv * ts : 0);
  p.o = a.take(hrows * nq * (prec ? sizeof(float) : ts));
  const int qn = full ? -1 : S;
  // the two-pass first read (one canvas per prompt); the one-pass read or the
  // draw pass (canvases of one prompt: first read and draws, or the draws)
  p.first = plan_attention(d, B, max_prompt, qn, prec, 1);
  p.draws = plan_attention(d, ncmax, max_prompt, qn, prec, p.spec ? nd + 1 : nd);
  const size_t po = p.first.part_o > p.draws.part_o ? p.first.part_o : p.draws.part_o;
  const size_t pm = p.first.part_ml > p.draws.part_ml ? p.first.part_ml : p.draws.part_ml;
  p.part_o = a.take(po);
  p.part_ml = a.take(pm);
  {
    // every projection a read launches: k/v of whole canvases, q (or, for the
    // speculated draws, q/k/v) of slot rows, the output projection of slot rows
    size_t pp = 0;
    const int64_t C = d.canvas, Bs = (int64_t)B * S;
    const int64_t kv_rows[] = {B * C, (nd > 1 ? (int64_t)nd : 1) * B * C};
    const int64_t q_rows[] = {Bs, (nd > 1 ? (int64_t)nd : 1) * Bs, (int64_t)(nd + 1) * Bs};
    for (int64_t m : kv_rows) pp = std::max(pp, proj_part_bytes(d, m, 2 * nkv, d.d_model));
    if (full) {   // q, k, v and the output projection of every canvas row
      const int64_t f_rows[] = {B * C, (int64_t)ncmax * C};
      for (int64_t m : f_rows) {
        pp = std::max(pp, proj_part_bytes(d, m, nq + 2 * nkv, d.d_model));
        pp = std::max(pp, proj_part_bytes(d, m, d.d_model, (int)(prec ? 2 * nq : nq)));
      }
    }
    for (int64_t m : q_rows) {
      pp = std::max(pp, proj_part_bytes(d, m, nq, d.d_model));
      pp = std::max(pp, proj_part_bytes(d, m, nq + 2 * nkv, d.d_model));
      pp = std::max(pp, proj_part_bytes(d, m, d.d_model, (int)(prec ? 2 * nq : nq)));
    }
    p.proj_part = a.take(pp);
  }
  p.h = a.take(hrows * d.d_model * ts * (prec ? 2 : 1));
  p.rows = a.take(nrows * sizeof(int32_t));
  p.qpos = a.take(nrows * sizeof(int32_t));
  p.qids = a.take(nrows * sizeof(int32_t));
  p.kv_row_base = a.take(p.spec && !full && !p.patch ? (size_t)B * d.canvas * sizeof(int32_t) : 0);
  // one-pass: draw slot rows' k, v rows; two-pass: those of the draw pass
  p.kv_row_slot = a.take(!full && nd > 1 && !p.patch ? nrows * sizeof(int32_t) : 0);
  p.stats = a.take(nrows * nvt * sizeof(float4));
  p.rowstat = a.take(nrows * sizeof(float2));
  p.lab_logit = a.take(nrows * DG_MAX_LABELS * sizeof(float));
  p.flags = a.take(((size_t)B + (size_t)B * S) * sizeof(int32_t));
  p.draw_active = a.take((size_t)B * (nd > 1 ? nd : 1) * sizeof(int32_t));
  p.draw_ids = a.take(nd > 1 ? (size_t)ncmax * d.canvas * sizeof(int32_t) : 0);
  p.row_active = a.take(nrows * sizeof(int32_t));
  p.rs_draw = a.take(nrows * sizeof(float));
  // one-pass patched reads: the rows within the slots' windows (see SlotArgs)
  const bool win = p.spec && p.patch;
  const size_t bc = win ? (size_t)B * d.canvas * sizeof(int32_t) : 0;
  p.win_pos = a.take(bc);
  p.win_cnt = a.take(win ? (size_t)B * sizeof(int32_t) : 0);
  p.win_ids = a.take(bc);
  p.win_rows = a.take(bc);
  p.win_total = a.take(win ? sizeof(int32_t) : 0);
  p.total = a.off;
  return p;
}

// Workspace bytes that hold a read of any prompt length up to max_prompt.
// The one-pass order needs more than the two-pass one, and is chosen for
// shorter prompts (the draws' forward pass grows with the prompt), so a read
// of a shorter prompt may take the one-pass order where max_prompt's does
// not: both are then covered.  Each order's size is non-decreasing in the
// prompt length.
size_t slot_ws_bound(const dg_dims &d, int B, int S, int max_prompt, int nd, bool full = false) {
  size_t t = plan_slot(d, B, S, max_prompt, nd, -1, full).total;
  if (speculate_draws(d, B, S, nd, 0, full))
    t = std::max(t, plan_slot(d, B, S, max_prompt, nd, 1, full).total);
  return t;
}

// records the caller's stage events (if any) around each stage of a call
struct Stages {
  void **ev = nullptr;
  hipStream_t st = nullptr;
  dg_status mark(int stage, int edge) const {
    if (!ev) return DG_OK;
    return hip_check(hipEventRecord(static_cast<hipEvent_t>(ev[2 * stage + edge]), st),
                     "stage event record");
  }
};

#define DG_MARK(stages, stage, edge)                  \
  do {                                                 \
    dg_status _m = (stages).mark((stage), (edge));     \
    if (_m != DG_OK) return _m;                        \
  } while (0)

template <typename P> P *at(void *ws, size_t off) {
  return reinterpret_cast<P *>(static_cast<char *>(ws) + off);
}

// the blocked copy of the LM head, where the kernels read it (bf16, d % 32 == 0)
const void *lm_tiled_of(const dg_dims &d, const dg_weights *w) {
  return d.dtype == DG_BF16 && d.d_model % 32 == 0 ? w->lm_tiled : nullptr;
}

const void *embed_t_tiled_of(const dg_dims &d, const dg_weights *w) {
  return d.dtype == DG_BF16 && d.d_model % 256 == 0 ? w->embed_t_tiled : nullptr;
}

// The softmax scale in log2 units rides on q, so attention exponentiates
// scores directly (one rounding of q either way).
float q_scale_of(const dg_dims &d) {
  return (float)(1.4426950408889634 / std::sqrt((double)d.head_dim));
}

// Queries of a pass: every canvas position, or qn gathered rows per canvas
// (positions qpos, token ids qids; -1 = none), for which attention and the
// output projection write compact rows cb*qn + i.
struct Gather {
  const int32_t *qpos = nullptr, *qids = nullptr;
  int qn = 0;
  bool qkv_done = false;   // q (compact), k and v are already projected
  // Precise rows (bf16 reads): attention takes the probabilities as bf16
  // hi + lo terms and writes o in fp32; the output projection takes o as hi
  // and lo halves and writes h as bf16 hi | lo halves ([rows, 2d]), which the
  // LM head sums.  Without it, a slot's logprob carries the bf16 rounding of
  // p, o and h, an error that grows with |logprob| (about 4e-4 |lp| at the
  // headline dims); with it, only that of the stored q, k, v remains.
  bool prec = false;
  // canvas c's k, v are written to / read from canvas slot c * kv_cmul (the
  // two-pass read keeps each canvas's k, v where its first draw will be)
  int kv_cmul = 1;
  // patched draws: the draws' slot rows of k, v (attention reads the base
  // canvases' k, v elsewhere), for canvases c with c % canvases_per_prompt >=
  // patch_from
  const void *kpatch = nullptr, *vpatch = nullptr;
  int patch_from = 0;
  // patched tiles read only these base rows (AttnArgs::win_pos), or null
  const int32_t *win_pos = nullptr, *win_cnt = nullptr;
  // encoder mode: the canvases are causal prompt chunks (AttnArgs::chunks)
  const int4 *chunks = nullptr;
};

// S0..S3 of one pass over nc canvases: q,k,v -> attention -> h
dg_status run_block(const dg_dims &d, const dg_weights *w, const dg_prompt_kv *kv, int nc,
                    int canvas_per_prompt, const int32_t *ids, const void *sc_in,
                    const int32_t *active, int32_t *flags, void *q, void *k, void *v, void *o,
                    const AttnPlan &ap, void *part_o, float2 *part_ml, float *proj_part, void *h,
                    hipStream_t st, const Stages &sg = Stages(), const Gather &gq = Gather()) {
  const bool bf = d.dtype == DG_BF16;
  const int64_t M = (int64_t)nc * d.canvas;
  dg::QkvArgs qa{};
  qa.ids = ids;
  qa.embed = w->embed;
  qa.sc_in = sc_in;
  qa.wq = w->wq;
  qa.wk = w->wk;
  qa.wv = w->wv;
  qa.q = q;
  qa.k = k;
  qa.v = v;
  qa.active = active;
  qa.flags = flags;
  qa.M = M;
  qa.d = d.d_model;
  qa.nq = d.n_q_heads * d.head_dim;
  qa.nkv = d.n_kv_heads * d.head_dim;
  qa.vocab = d.vocab;
  qa.C = d.canvas;
  qa.q_scale = q_scale_of(d);
  qa.col0 = 0;
  qa.col1 = qa.nq + 2 * qa.nkv;
  qa.kv_row = nullptr;
  qa.kv_cmul = gq.kv_cmul;
  qa.part = proj_part;
  DG_MARK(sg, DG_STAGE_QKV, 0);
  if (gq.qpos && !gq.qkv_done) {
    // k, v of every canvas row; q of the gathered rows only (compact).  A
    // gathered pass takes no self-conditioning input (reads have none).
    if (sc_in) return fail(DG_ERR_INVALID_ARG, "gathered queries take no sc_in");
    qa.col0 = qa.nq;
    DG_TRY_HIP(dg::launch_qkv(qa, bf, st), "k/v projection launch");
    dg::QkvArgs qg = qa;
    qg.ids = gq.qids;
    qg.sc_in = nullptr;
    qg.flags = nullptr;
    qg.M = (int64_t)nc * gq.qn;
    qg.C = gq.qn;
    qg.col0 = 0;
    qg.col1 = qa.nq;
    DG_TRY_HIP(dg::launch_qkv(qg, bf, st), "q projection launch");
  } else if (!gq.qpos) {
    DG_TRY_HIP(dg::launch_qkv(qa, bf, st), "qkv projection launch");
  }
  DG_MARK(sg, DG_STAGE_QKV, 1);

  dg::AttnArgs aa{};
  aa.q = q;
  aa.k = k;
  aa.v = v;
  aa.kp = kv->k;
  aa.vp = kv->v;
  aa.cu = kv->cu_seqlens;
  aa.active = active;
  aa.flags = flags;
  aa.qpos = gq.qpos;
  aa.qn = gq.qpos ? gq.qn : d.canvas;
  aa.o = o;
  aa.part_o = part_o;
  aa.part_ml = part_ml;
  aa.total_len = kv->total_len;
  aa.nc = nc;
  aa.C = d.canvas;
  aa.Hq = d.n_q_heads;
  aa.Hkv = d.n_kv_heads;
  aa.W = window_of(d);
  aa.max_len = kv->max_len;
  aa.nsplit = ap.nsplit;
  aa.chunk = ap.chunk;
  aa.canvas_per_prompt = canvas_per_prompt;
  aa.prec = gq.prec ? 1 : 0;
  aa.kv_cmul = gq.kv_cmul;
  aa.kpatch = gq.kpatch;
  aa.vpatch = gq.vpatch;
  aa.patch_from = gq.patch_from;
  aa.win_pos = gq.win_pos;
  aa.win_cnt = gq.win_cnt;
  aa.chunks = gq.chunks;
  DG_MARK(sg, DG_STAGE_ATTENTION, 0);
  DG_TRY_HIP(dg::launch_attention(aa, d.head_dim, bf, st), "attention launch");
  DG_MARK(sg, DG_STAGE_ATTENTION, 1);

  dg::OprojArgs oa{};
  oa.o = o;
  oa.wo = w->wo;
  oa.ids = gq.qpos ? gq.qids : ids;
  oa.embed = w->embed;
  oa.sc_in = gq.qpos ? nullptr : sc_in;
  oa.h = h;
  oa.active = active;
  oa.M = gq.qpos ? (int64_t)nc * gq.qn : M;
  oa.d = d.d_model;
  oa.kdim = d.n_q_heads * d.head_dim;
  oa.vocab = d.vocab;
  oa.C = gq.qpos ? gq.qn : d.canvas;
  oa.part = proj_part;
  oa.prec = gq.prec ? 1 : 0;
  DG_MARK(sg, DG_STAGE_OPROJ, 0);
  DG_TRY_HIP(dg::launch_oproj(oa, bf, st), "output projection launch");
  DG_MARK(sg, DG_STAGE_OPROJ, 1);
  return DG_OK;
}

// Argument checks of a denoise step (no HIP calls).
dg_status check_step_args(const dg_dims *dims, const dg_weights *w, const dg_prompt_kv *kv,
                          int32_t batch, const int32_t *canvas_ids, const void *sc_in,
                          const float *conf, const float *entropy, const int32_t *argmax,
                          const void *sc_out, const dg_debug *debug) {
  dg_status s = check_model(dims, batch, kv ? kv->max_len : 0, w, kv);
  if (s != DG_OK) return s;
  const dg_dims &d = *dims;
  if (batch == 0) return ok();
  if (!canvas_ids || !conf || !entropy || !argmax)
    return fail(DG_ERR_INVALID_ARG, "canvas_ids, conf, entropy and argmax are required");
  const void *et_tiled = embed_t_tiled_of(d, w);
  if (sc_out && !w->embed_t && !et_tiled)
    return fail(DG_ERR_INVALID_ARG,
                "sc_out requires weights.embed_t (see dg_prepare_embed_t) or embed_t_tiled");
  if (!aligned16(sc_in) || !aligned16(sc_out))
    return fail(DG_ERR_INVALID_ARG, "sc_in and sc_out must be 16-byte aligned");
  if (debug && (!aligned16(debug->attn_out) || !aligned16(debug->hidden_out)))
    return fail(DG_ERR_INVALID_ARG, "debug outputs must be 16-byte aligned");
  return DG_OK;
}

// One denoise step on a validated call with a planned workspace (no flag
// clear).  active: per-canvas flags or null; canvases whose flag is 0 are
// skipped by the projections, attention, the LM head and p.E, and their
// outputs are left unspecified.  exclude_id >= 0 removes that id from the
// vocabulary softmax (the multi-step loop removes the mask id).
dg_status step_core(const dg_dims &d, const dg_weights *w, const dg_prompt_kv *kv, int batch,
                    const int32_t *canvas_ids, const void *sc_in, float logit_scale,
                    const float *row_scale, float *conf, float *entropy, int32_t *argmax,
                    void *sc_out, const dg_debug *debug, int32_t *dev_flags,
                    const int32_t *active, void *workspace, const StepPlan &p, hipStream_t st,
                    int exclude_id = -1) {
  const bool bf = d.dtype == DG_BF16;
  const int64_t M = (int64_t)batch * d.canvas;
  const int nvt = d.vocab / dg::VTILE;
  void *o = (debug && debug->attn_out) ? debug->attn_out : at<char>(workspace, p.o);
  void *h = (debug && debug->hidden_out) ? debug->hidden_out : at<char>(workspace, p.h);
  Stages sg;
  sg.ev = debug ? debug->stage_events : nullptr;
  sg.st = st;
  dg_status s = run_block(d, w, kv, batch, 1, canvas_ids, sc_in, active, dev_flags, at<char>(workspace, p.q),
                at<char>(workspace, p.k), at<char>(workspace, p.v), o, p.attn,
                at<char>(workspace, p.part_o), at<float2>(workspace, p.part_ml),
                at<float>(workspace, p.proj_part), h, st, sg);
  if (s != DG_OK) return s;

  dg::LmheadArgs la{};
  la.head = w->lm_head ? w->lm_head : w->embed;
  la.head_tiled = lm_tiled_of(d, w);
  la.head_fp8 = static_cast<const uint8_t *>(w->lm_fp8);
  la.head_exp = w->lm_fp8_exp;
  la.h = h;
  la.logit_scale = logit_scale;
  la.row_scale = row_scale;
  la.stats = at<float4>(workspace, p.stats);
  la.ptilde = sc_out ? at<char>(workspace, p.ptilde) : nullptr;
  la.ptilde_blocked = bf;
  la.logits = debug ? debug->logits_out : nullptr;
  la.nrows = M;
  la.active_rows = active;
  la.rows_per_flag = d.canvas;
  la.exclude_id1 = exclude_id + 1;
  la.d = d.d_model;
  la.vocab = d.vocab;
  la.nvt = nvt;
  DG_MARK(sg, DG_STAGE_LMHEAD, 0);
  if (bf && w->lm_fp8 && w->lm_fp8_act) {
    // per-row e4m3 activations (rows of inactive canvases are quantised too:
    // their tiles are skipped by the LM head)
    la.h_fp8 = at<uint8_t>(workspace, p.hq);
    la.h_exp = at<int32_t>(workspace, p.hexp);
    DG_TRY_HIP(dg::launch_quantize_e4m3(h, at<uint8_t>(workspace, p.hq), at<int32_t>(workspace, p.hexp),
                                        (int)M, d.d_model, st),
               "activation quantisation launch");
  }
  DG_TRY_HIP(dg::launch_lmhead(la, bf, st), "LM head launch");
  DG_MARK(sg, DG_STAGE_LMHEAD, 1);

  dg::VocabMergeArgs va{};
  va.stats = la.stats;
  va.nrows = M;
  va.nvt = nvt;
  va.conf = conf;
  va.entropy = entropy;
  va.argmax = argmax;
  va.shift = sc_out ? at<int32_t>(workspace, p.shift) : nullptr;
  va.inv_z = sc_out ? at<float>(workspace, p.inv_z) : nullptr;
  DG_MARK(sg, DG_STAGE_VOCAB_MERGE, 0);
  DG_TRY_HIP(dg::launch_vocab_merge(va, st), "vocabulary merge launch");
  DG_MARK(sg, DG_STAGE_VOCAB_MERGE, 1);

  DG_MARK(sg, DG_STAGE_SELFCOND, 0);
  if (sc_out) {
    dg::ScArgs sa{};
    sa.ptilde = la.ptilde;
    sa.shift = va.shift;
    sa.inv_z = va.inv_z;
    sa.ptilde_blocked = la.ptilde_blocked;
    sa.embed_t = w->embed_t;
    sa.embed_t_tiled = embed_t_tiled_of(d, w);
    sa.part = at<float>(workspace, p.sc_part);
    sa.out = sc_out;
    sa.M = M;
    sa.d = d.d_model;
    sa.vocab = d.vocab;
    sa.nvt = nvt;
    sa.ksplit = p.ksplit;
    sa.active = active;
    sa.C = d.canvas;
    DG_TRY_HIP(dg::launch_scgemm(sa, bf, st), "self-conditioning launch");
  }
  DG_MARK(sg, DG_STAGE_SELFCOND, 1);
  return DG_OK;
}


// k, v cache rows of n_tokens prompt tokens (the block's projections of E[id])
dg_status prefill_rows(const dg_dims &d, const dg_weights *w, int64_t n_tokens,
                       const int32_t *prompt_ids, void *k_out, void *v_out, int32_t *dev_flags,
                       hipStream_t st) {
  dg::QkvArgs qa{};
  qa.ids = prompt_ids;
  qa.embed = w->embed;
  qa.wq = w->wk;   // no q column is computed; any valid matrix pointer
  qa.wk = w->wk;
  qa.wv = w->wv;
  qa.k = k_out;
  qa.v = v_out;
  qa.flags = dev_flags;
  qa.M = n_tokens;
  qa.d = d.d_model;
  qa.nq = d.n_q_heads * d.head_dim;
  qa.nkv = d.n_kv_heads * d.head_dim;
  qa.vocab = d.vocab;
  qa.C = d.canvas;
  qa.q_scale = 1.f;
  qa.col0 = qa.nq;                 // the k and v columns of [q | k | v]
  qa.col1 = qa.nq + 2 * qa.nkv;
  DG_TRY_HIP(dg::launch_qkv(qa, d.dtype == DG_BF16, st), "prefill projection launch");
  return DG_OK;
}

// Workspace of the encoder-mode forward: B sequences of at most max_len tokens
// in J = ceil(max_len / C) chunks of C rows each.
struct EncodePlan {
  size_t q, k, v, o, h, part_o, part_ml, proj_part, ids, chunks, active, total;
  AttnPlan attn;
  int J;
  bool too_big;   // more chunk rows than int32 addresses (no plan)
};

EncodePlan plan_encode(const dg_dims &d, int B, int max_len) {
  EncodePlan p{};
  const int64_t J = ((int64_t)max_len + d.canvas - 1) / d.canvas;
  const int64_t NC = (int64_t)B * J, M = NC * d.canvas;
  p.J = (int)J;
  if (NC == 0) return p;   // nothing to run: no workspace
  if (M > INT32_MAX) {     // the chunk rows are addressed as int32
    p.too_big = true;
    return p;
  }
  const size_t ts = tsize(d);
  const size_t nq = (size_t)d.n_q_heads * d.head_dim, nkv = (size_t)d.n_kv_heads * d.head_dim;
  Arena a;
  p.q = a.take(M * nq * ts);
  p.k = a.take(M * nkv * ts);
  p.v = a.take(M * nkv * ts);
  p.o = a.take(M * nq * ts);
  p.h = a.take(M * d.d_model * ts);
  p.attn = plan_attention(d, (int)NC, max_len);
  // split partials: the most that any shorter max_len needs (more chunks can
  // mean fewer splits), so that the size only grows with max_len
  // (past 1024 chunks per sequence there are enough tiles that neither the
  // attention nor the projections split)
  size_t po = 0, pml = 0, pp = 0;
  for (int j = 1; j <= p.J; j = (j < 1024 || j == p.J) ? j + 1 : p.J) {
    const int64_t nc = (int64_t)B * j, m = nc * d.canvas;
    const AttnPlan ap = plan_attention(d, (int)nc, std::min(max_len, j * d.canvas));
    po = std::max(po, ap.part_o);
    pml = std::max(pml, ap.part_ml);
    pp = std::max(pp, std::max(proj_part_bytes(d, m, nq + 2 * nkv, d.d_model),
                               proj_part_bytes(d, m, d.d_model, (int)nq)));
  }
  p.part_o = a.take(po);
  p.part_ml = a.take(pml);
  p.proj_part = a.take(pp);
  p.ids = a.take(M * sizeof(int32_t));
  p.chunks = a.take(NC * sizeof(int4));
  p.active = a.take(NC * sizeof(int32_t));
  p.total = a.off;
  return p;
}

}  // namespace

extern "C" {

// detail message of a failed call made from another source file of the library
// (not part of the exported interface)
__attribute__((visibility("hidden"))) dg_status dg_internal_fail(dg_status s, const char *msg) {
  return fail(s, "%s", msg);
}

const char *dg_status_string(dg_status s) {
  // a C caller may pass any int: read the value as one (a C++ load of an
  // enum outside its enumerators' range is undefined)
  int code;
  std::memcpy(&code, &s, sizeof code);
  switch (code) {
    case DG_OK: return "ok";
    case DG_ERR_INVALID_ARG: return "invalid argument";
    case DG_ERR_TOO_MANY_LABELS: return "too many labels (more than the 26 single-token labels A..Z)";
    case DG_ERR_UNSUPPORTED: return "unsupported configuration";
    case DG_ERR_WORKSPACE: return "workspace too small";
    case DG_ERR_HIP: return "HIP runtime error";
  }
  return "unknown status";
}

const char *dg_last_error(void) { return g_err.c_str(); }

const char *dg_version(void) { return "dg 0.1.0 (gfx950)"; }

dg_status dg_check_label_count(int32_t n) {
  if (n < 1) return fail(DG_ERR_INVALID_ARG, "a question needs at least one alternative (got %d)", n);
  if (n > DG_MAX_LABELS)
    return fail(DG_ERR_TOO_MANY_LABELS, "too many labels: %d > %d", n, DG_MAX_LABELS);
  return ok();
}

dg_status dg_denoise_step_validate(const dg_dims *dims, int32_t batch, int32_t max_prompt,
                                   const dg_weights *w, const dg_prompt_kv *kv) {
  dg_status s = check_model(dims, batch, max_prompt, w, kv);
  return s == DG_OK ? ok() : s;
}

dg_status dg_slot_read_validate(const dg_dims *dims, int32_t batch, int32_t n_slots,
                                int32_t n_draws, float entropy_threshold) {
  dg_status s = check_dims(dims);
  if (s != DG_OK) return s;
  if (batch < 0) return fail(DG_ERR_INVALID_ARG, "batch %d < 0", batch);
  if (n_slots < 0) return fail(DG_ERR_INVALID_ARG, "n_slots %d < 0", n_slots);
  if (n_draws < 1 || n_draws > 16) return fail(DG_ERR_INVALID_ARG, "n_draws %d outside [1, 16]", n_draws);
  if (!(entropy_threshold >= 0.f)) return fail(DG_ERR_INVALID_ARG, "entropy_threshold must be >= 0");
  // a read holds up to 1 + n_draws canvases per batch entry
  s = check_sizes(*dims, (int64_t)batch * (n_draws + 1), 0, (int64_t)batch * n_slots * (n_draws + 1));
  if (s != DG_OK) return s;
  return ok();
}

dg_status dg_commit_validate(int32_t batch, int32_t canvas) {
  if (batch < 0) return fail(DG_ERR_INVALID_ARG, "batch %d < 0", batch);
  if (canvas < 1 || canvas > DG_MAX_CANVAS)
    return fail(DG_ERR_INVALID_ARG, "canvas %d outside [1, %d]", canvas, DG_MAX_CANVAS);
  if ((int64_t)batch * canvas > kMaxRows)
    return fail(DG_ERR_INVALID_ARG, "batch %d x canvas %d exceeds 2^31 - 1 rows", batch, canvas);
  return ok();
}

size_t dg_denoise_step_workspace(const dg_dims *dims, int32_t batch, int32_t max_prompt) {
  if (check_dims(dims) != DG_OK || batch < 0 || max_prompt < 0 || !sizes_fit(*dims, batch, max_prompt))
    return 0;
  return plan_step(*dims, batch, max_prompt).total;
}

dg_status dg_denoise_step(const dg_dims *dims, const dg_weights *w, const dg_prompt_kv *kv,
                          int32_t batch, const int32_t *canvas_ids, const void *sc_in,
                          float logit_scale, const float *row_scale, float *conf, float *entropy,
                          int32_t *argmax, void *sc_out, const dg_debug *debug,
                          int32_t *dev_flags, void *workspace, size_t ws_bytes, void *stream) {
  dg_status s = check_step_args(dims, w, kv, batch, canvas_ids, sc_in, conf, entropy, argmax,
                                sc_out, debug);
  if (s != DG_OK || batch == 0) return s;
  if (!aligned16(workspace)) return fail(DG_ERR_INVALID_ARG, "workspace must be 16-byte aligned");
  const StepPlan p = plan_step(*dims, batch, kv->max_len);
  if (!workspace || ws_bytes < p.total)
    return fail(DG_ERR_WORKSPACE, "workspace of %zu bytes is smaller than the %zu bytes needed",
                ws_bytes, p.total);
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (dev_flags) DG_TRY_HIP(dg::launch_clear_i32(dev_flags, 1, st), "flag clear launch");
  s = step_core(*dims, w, kv, batch, canvas_ids, sc_in, logit_scale, row_scale, conf, entropy,
                argmax, sc_out, debug, dev_flags, nullptr, workspace, p, st);
  return s != DG_OK ? s : ok();
}

size_t dg_denoise_loop_workspace(const dg_dims *dims, int32_t batch, int32_t max_prompt) {
  if (check_dims(dims) != DG_OK || batch < 0 || max_prompt < 0 || !sizes_fit(*dims, batch, max_prompt))
    return 0;
  return plan_loop(*dims, batch, max_prompt).total;
}

dg_status dg_denoise_loop(const dg_dims *dims, const dg_weights *w, const dg_prompt_kv *kv,
                          int32_t batch, int32_t *canvas_ids, const void *sc_in,
                          float logit_scale, const float *row_scale, float threshold_nats,
                          int32_t max_steps, int32_t check_every, int32_t *commit_step,
                          int32_t *steps_taken, int32_t *steps_launched, int32_t *dev_flags,
                          void *workspace, size_t ws_bytes, void *stream) {
  if (steps_launched) *steps_launched = 0;
  // the loop makes progress only when every step commits: tau >= 0 accepts
  // the most confident candidate at least
  if (!(threshold_nats >= 0.f))
    return fail(DG_ERR_INVALID_ARG, "threshold %g: the loop needs a threshold >= 0", threshold_nats);
  if (max_steps < 0 || check_every < 1)
    return fail(DG_ERR_INVALID_ARG, "max_steps %d must be >= 0 and check_every %d >= 1", max_steps,
                check_every);
  if (!commit_step || !steps_taken)
    return fail(DG_ERR_INVALID_ARG, "commit_step and steps_taken are required");
  // the step's own checks, with stand-in outputs (they live in the workspace)
  static const float f_dummy[4] = {0, 0, 0, 0};
  static const int32_t i_dummy[4] = {0, 0, 0, 0};
  dg_status s = check_step_args(dims, w, kv, batch, canvas_ids, sc_in, f_dummy, f_dummy, i_dummy,
                                f_dummy, nullptr);
  if (s != DG_OK || batch == 0) return s;
  if (!w->embed_t && !embed_t_tiled_of(*dims, w))
    return fail(DG_ERR_INVALID_ARG, "the loop feeds p.E back: weights.embed_t or embed_t_tiled is required");
  s = dg_commit_validate(batch, dims->canvas);
  if (s != DG_OK) return s;
  if (!aligned16(workspace)) return fail(DG_ERR_INVALID_ARG, "workspace must be 16-byte aligned");
  const dg_dims &d = *dims;
  const LoopPlan p = plan_loop(d, batch, kv->max_len);
  if (!workspace || ws_bytes < p.total)
    return fail(DG_ERR_WORKSPACE, "workspace of %zu bytes is smaller than the %zu bytes needed",
                ws_bytes, p.total);
  hipStream_t st = static_cast<hipStream_t>(stream);
  float *conf = at<float>(workspace, p.conf), *ent = at<float>(workspace, p.entropy);
  int32_t *am = at<int32_t>(workspace, p.argmax);
  void *sc[2] = {at<char>(workspace, p.sc0), at<char>(workspace, p.sc1)};
  uint8_t *cmask = at<uint8_t>(workspace, p.cmask);
  int32_t *out_ids = at<int32_t>(workspace, p.out_ids);
  int32_t *ncommit = at<int32_t>(workspace, p.n_commit);
  int32_t *active = at<int32_t>(workspace, p.active);
  int32_t *n_active = at<int32_t>(workspace, p.n_active);
  if (dev_flags) DG_TRY_HIP(dg::launch_clear_i32(dev_flags, 1, st), "flag clear launch");
  DG_TRY_HIP(dg::launch_loop_init(canvas_ids, batch, d.canvas, d.mask_id, commit_step, steps_taken,
                                  active, st),
             "loop init launch");
  dg::CommitArgs ca{};
  ca.ids = canvas_ids;
  ca.conf = conf;
  ca.entropy = ent;
  ca.argmax = am;
  ca.mask = cmask;
  ca.out_ids = out_ids;
  ca.n_committed = ncommit;
  ca.B = batch;
  ca.C = d.canvas;
  ca.mask_id = d.mask_id;
  ca.tau = threshold_nats;
  for (int t = 0; t < max_steps; ++t) {
    // step t reads the canvas and the previous step's p.E, and writes its own
    const void *sc_t = t == 0 ? sc_in : sc[(t + 1) & 1];
    s = step_core(d, w, kv, batch, canvas_ids, sc_t, logit_scale, row_scale, conf, ent, am,
                  sc[t & 1], nullptr, dev_flags, active, workspace, p.step, st, d.mask_id);
    if (s != DG_OK) return s;
    DG_TRY_HIP(dg::launch_commit(ca, st), "commit launch");
    DG_TRY_HIP(dg::launch_clear_i32(n_active, 1, st), "counter clear launch");
    DG_TRY_HIP(dg::launch_loop_update(canvas_ids, out_ids, cmask, batch, d.canvas, d.mask_id, t,
                                      commit_step, steps_taken, active, n_active, st),
               "loop update launch");
    if (steps_launched) *steps_launched = t + 1;
    if ((t + 1) % check_every == 0 && t + 1 < max_steps) {
      int32_t left = 0;
      DG_TRY_HIP(hipMemcpyAsync(&left, n_active, sizeof left, hipMemcpyDeviceToHost, st),
                 "active-count read-back");
      DG_TRY_HIP(hipStreamSynchronize(st), "loop check synchronisation");
      if (left == 0) break;
    }
  }
  return ok();
}


dg_status dg_prefill_kv(const dg_dims *dims, const dg_weights *w, int64_t n_tokens,
                        const int32_t *prompt_ids, void *k_out, void *v_out,
                        int32_t *dev_flags, void *stream) {
  dg_status s = check_dims(dims);
  if (s != DG_OK) return s;
  if (!w || !w->embed || !w->wk || !w->wv)
    return fail(DG_ERR_INVALID_ARG, "prefill needs weights.embed, wk and wv");
  if (n_tokens < 0) return fail(DG_ERR_INVALID_ARG, "n_tokens %lld < 0", (long long)n_tokens);
  if (n_tokens == 0) return ok();
  if (!prompt_ids || !k_out || !v_out)
    return fail(DG_ERR_INVALID_ARG, "prompt_ids, k_out and v_out are required");
  if (!aligned16(w->embed) || !aligned16(w->wk) || !aligned16(w->wv) || !aligned16(k_out) ||
      !aligned16(v_out))
    return fail(DG_ERR_INVALID_ARG, "weights and the k/v outputs must be 16-byte aligned");
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (dev_flags) DG_TRY_HIP(dg::launch_clear_i32(dev_flags, 1, st), "flag clear launch");
  s = prefill_rows(*dims, w, n_tokens, prompt_ids, k_out, v_out, dev_flags, st);
  return s != DG_OK ? s : ok();
}

size_t dg_prefill_encode_workspace(const dg_dims *dims, int32_t batch, int32_t max_len) {
  if (check_dims(dims) != DG_OK || batch < 0 || max_len < 0 || max_len > kMaxPrompt) return 0;
  const EncodePlan p = plan_encode(*dims, batch, max_len);
  return p.too_big ? 0 : p.total;
}

dg_status dg_prefill_encode(const dg_dims *dims, const dg_weights *w, int32_t batch,
                            const int32_t *cu_seqlens, int32_t max_len, int64_t total_len,
                            const int32_t *prompt_ids, void *k_out, void *v_out, void *hidden_out,
                            void *attn_out, int32_t *dev_flags, void *workspace, size_t ws_bytes,
                            void *stream) {
  dg_status s = check_dims(dims);
  if (s != DG_OK) return s;
  if (batch < 0) return fail(DG_ERR_INVALID_ARG, "batch %d < 0", batch);
  if (max_len < 0 || total_len < 0)
    return fail(DG_ERR_INVALID_ARG, "max_len and total_len must be >= 0");
  if (max_len > kMaxPrompt) return fail(DG_ERR_INVALID_ARG, "max_len %d exceeds 2^30", max_len);
  const bool fwd = hidden_out || attn_out;
  if (!w || !w->embed || !w->wk || !w->wv || (fwd && (!w->wq || !w->wo)))
    return fail(DG_ERR_INVALID_ARG,
                "the encoder needs weights.embed, wk and wv (and wq, wo for hidden_out / attn_out)");
  if (total_len > 0 && (!prompt_ids || !k_out || !v_out))
    return fail(DG_ERR_INVALID_ARG, "prompt_ids, k_out and v_out are required");
  if (fwd && batch > 0 && !cu_seqlens) return fail(DG_ERR_INVALID_ARG, "cu_seqlens is required");
  const void *ptrs[] = {w->embed, w->wq, w->wk, w->wv, w->wo, k_out, v_out, hidden_out, attn_out, workspace};
  for (const void *p : ptrs)
    if (!aligned16(p)) return fail(DG_ERR_INVALID_ARG, "weights, outputs and workspace must be 16-byte aligned");
  const dg_dims &d = *dims;
  hipStream_t st = static_cast<hipStream_t>(stream);
  const bool run = fwd && batch > 0 && max_len > 0 && total_len > 0;
  const EncodePlan p = plan_encode(d, run ? batch : 0, run ? max_len : 0);
  if (p.too_big)
    return fail(DG_ERR_INVALID_ARG, "batch %d x %d chunks of %d tokens exceed 2^31 - 1 rows", batch, p.J,
                d.canvas);
  if (run && (!workspace || ws_bytes < p.total))
    return fail(DG_ERR_WORKSPACE, "workspace of %zu bytes is smaller than the %zu bytes needed",
                ws_bytes, p.total);
  if (dev_flags) DG_TRY_HIP(dg::launch_clear_i32(dev_flags, 1, st), "flag clear launch");
  if (total_len > 0) {
    s = prefill_rows(d, w, total_len, prompt_ids, k_out, v_out, dev_flags, st);
    if (s != DG_OK) return s;
  }
  if (!run) return ok();
  dg::EncodeArgs ea{};
  ea.cu = cu_seqlens;
  ea.prompt_ids = prompt_ids;
  ea.flags = dev_flags;
  ea.ids_pad = at<int32_t>(workspace, p.ids);
  ea.chunks = at<int4>(workspace, p.chunks);
  ea.active = at<int32_t>(workspace, p.active);
  ea.h_pad = at<char>(workspace, p.h);
  ea.o_pad = at<char>(workspace, p.o);
  ea.hidden_out = hidden_out;
  ea.attn_out = attn_out;
  ea.total_len = total_len;
  ea.h_row_bytes = (int64_t)d.d_model * tsize(d);
  ea.o_row_bytes = (int64_t)d.n_q_heads * d.head_dim * tsize(d);
  ea.B = batch;
  ea.J = p.J;
  ea.C = d.canvas;
  ea.max_len = max_len;
  DG_TRY_HIP(dg::launch_encode_plan(ea, st), "encoder chunk plan launch");
  const dg_prompt_kv kv{k_out, v_out, cu_seqlens, max_len, total_len};
  Gather g;
  g.chunks = ea.chunks;
  const int nc = batch * p.J;
  s = run_block(d, w, &kv, nc, 1, ea.ids_pad, nullptr, ea.active, dev_flags, at<char>(workspace, p.q),
                at<char>(workspace, p.k), at<char>(workspace, p.v), at<char>(workspace, p.o), p.attn,
                at<char>(workspace, p.part_o), at<float2>(workspace, p.part_ml),
                at<float>(workspace, p.proj_part), at<char>(workspace, p.h), st, Stages(), g);
  if (s != DG_OK) return s;
  if (hidden_out || attn_out) {
    if (!hidden_out) {   // attention rows only: the scatter copies hidden rows first
      ea.hidden_out = attn_out;
      ea.h_pad = ea.o_pad;
      ea.h_row_bytes = ea.o_row_bytes;
      ea.attn_out = nullptr;
    }
    DG_TRY_HIP(dg::launch_encode_scatter(ea, st), "encoder output copy launch");
  }
  return ok();
}

dg_status dg_commit(int32_t batch, int32_t canvas, int32_t mask_id, const int32_t *canvas_ids,
                    const float *conf, const float *entropy, const int32_t *argmax,
                    float threshold_nats, uint8_t *commit_mask, int32_t *out_ids,
                    int32_t *n_committed, void *stream) {
  dg_status s = dg_commit_validate(batch, canvas);
  if (s != DG_OK) return s;
  if (std::isnan(threshold_nats)) return fail(DG_ERR_INVALID_ARG, "threshold is NaN");
  if (batch == 0) return ok();
  if (!canvas_ids || !conf || !entropy || !argmax || !commit_mask || !out_ids)
    return fail(DG_ERR_INVALID_ARG, "commit arrays must not be NULL (n_committed may be)");
  dg::CommitArgs ca{};
  ca.ids = canvas_ids;
  ca.conf = conf;
  ca.entropy = entropy;
  ca.argmax = argmax;
  ca.mask = commit_mask;
  ca.out_ids = out_ids;
  ca.n_committed = n_committed;
  ca.B = batch;
  ca.C = canvas;
  ca.mask_id = mask_id;
  ca.tau = threshold_nats;
  DG_TRY_HIP(dg::launch_commit(ca, static_cast<hipStream_t>(stream)), "commit launch");
  return ok();
}

}  // extern "C"

namespace {

size_t slot_read_workspace(const dg_dims *dims, int32_t batch, int32_t n_slots, int32_t max_prompt,
                           int32_t n_draws, bool full) {
  if (check_dims(dims) != DG_OK || batch < 0 || n_slots < 0 || max_prompt < 0 || n_draws < 1 ||
      n_draws > 16 ||
      !sizes_fit(*dims, (int64_t)batch * (n_draws + 1), max_prompt, (int64_t)batch * n_slots * (n_draws + 1)))
    return 0;
  return slot_ws_bound(*dims, batch, n_slots, max_prompt, n_draws, full);
}

// The slot read in the slot-row order (full = false) or the whole-canvas order.
dg_status slot_read(const dg_dims *dims, const dg_weights *w, const dg_prompt_kv *kv,
                    int32_t batch, const int32_t *canvas_ids, int32_t n_slots,
                    const int32_t *slot_pos, const int32_t *label_ids, const int32_t *n_labels,
                    const int32_t *noise_ids, float logit_scale, const float *row_scale,
                    float entropy_threshold, int32_t n_draws, float *logprobs, float *probs,
                    float *entropy, float *first_entropy, int32_t *best, int32_t *draws_used,
                    int32_t *status, void *workspace, size_t ws_bytes, void *stream, bool full) {
  dg_status s = dg_slot_read_validate(dims, batch, n_slots, n_draws, entropy_threshold);
  if (s != DG_OK) return s;
  s = check_model(dims, batch, kv ? kv->max_len : 0, w, kv);
  if (s != DG_OK) return s;
  const dg_dims &d = *dims;
  if (batch == 0 || n_slots == 0) return ok();
  if (!canvas_ids || !slot_pos || !label_ids || !n_labels || !logprobs || !probs || !entropy ||
      !first_entropy || !best || !draws_used || !status)
    return fail(DG_ERR_INVALID_ARG, "slot-read input and output arrays must not be NULL");
  if (n_draws > 1 && !noise_ids) return fail(DG_ERR_INVALID_ARG, "noise_ids is required when n_draws > 1");
  if (!aligned16(workspace)) return fail(DG_ERR_INVALID_ARG, "workspace must be 16-byte aligned");
  const SlotPlan p = plan_slot(d, batch, n_slots, kv->max_len, n_draws, -1, full);
  if (!workspace || ws_bytes < p.total)
    return fail(DG_ERR_WORKSPACE, "workspace of %zu bytes is smaller than the %zu bytes needed",
                ws_bytes, p.total);
  hipStream_t st = static_cast<hipStream_t>(stream);
  const bool bf = d.dtype == DG_BF16;
  const int nvt = d.vocab / dg::VTILE;
  void *q = at<char>(workspace, p.q), *k = at<char>(workspace, p.k), *v = at<char>(workspace, p.v);
  void *o = at<char>(workspace, p.o), *h = at<char>(workspace, p.h);
  void *part_o = at<char>(workspace, p.part_o);
  float2 *part_ml = at<float2>(workspace, p.part_ml);
  float *proj_part = at<float>(workspace, p.proj_part);

  dg::SlotArgs sa{};
  sa.slot_pos = slot_pos;
  sa.label_ids = label_ids;
  sa.n_labels = n_labels;
  sa.noise_ids = noise_ids;
  sa.rowstat = at<float2>(workspace, p.rowstat);
  sa.lab_logit = at<float>(workspace, p.lab_logit);
  sa.row_scale = row_scale;
  sa.logit_scale = logit_scale;
  sa.threshold = entropy_threshold;
  sa.B = batch;
  sa.S = n_slots;
  sa.C = d.canvas;
  sa.V = d.vocab;
  sa.d = d.d_model;
  sa.n_draws = n_draws;
  sa.rows = at<int32_t>(workspace, p.rows);
  sa.status = status;
  sa.logprobs = logprobs;
  sa.probs = probs;
  sa.entropy = entropy;
  sa.first_entropy = first_entropy;
  sa.best = best;
  sa.draws_used = draws_used;
  sa.canvas_flag = at<int32_t>(workspace, p.flags);
  sa.draw_active = at<int32_t>(workspace, p.draw_active);
  sa.canvas_ids = canvas_ids;
  sa.draw_ids = at<int32_t>(workspace, p.draw_ids);
  sa.qpos = at<int32_t>(workspace, p.qpos);
  sa.qids = at<int32_t>(workspace, p.qids);
  const bool kv_copy = p.spec && !full && !p.patch;
  sa.kv_row_base = kv_copy ? at<int32_t>(workspace, p.kv_row_base) : nullptr;
  sa.kv_row_slot = !full && n_draws > 1 && !p.patch ? at<int32_t>(workspace, p.kv_row_slot) : nullptr;
  void *kpatch = p.patch ? at<char>(workspace, p.kpatch) : nullptr;
  void *vpatch = p.patch ? at<char>(workspace, p.vpatch) : nullptr;
  sa.mask_id = d.mask_id;
  sa.full_canvas = full ? 1 : 0;
  Gather gq;
  if (!full) {   // whole canvas: no gathered queries (qpos null)
    gq.qpos = sa.qpos;
    gq.qids = sa.qids;
    gq.qn = n_slots;
  }
  gq.prec = p.prec;

  dg::LmheadArgs la{};
  la.head = w->lm_head ? w->lm_head : w->embed;
  la.head_tiled = lm_tiled_of(d, w);
  la.head_fp8 = static_cast<const uint8_t *>(w->lm_fp8);
  la.head_exp = w->lm_fp8_exp;
  la.h = h;
  la.row_index = sa.rows;
  la.logit_scale = logit_scale;
  la.stats = at<float4>(workspace, p.stats);
  la.lab_ids = label_ids;
  la.lab_n = n_labels;
  la.lab_logit = at<float>(workspace, p.lab_logit);
  la.lab_S = n_slots;
  la.d = d.d_model;
  la.vocab = d.vocab;
  la.nvt = nvt;
  la.hl = p.prec ? 1 : 0;
  dg::VocabMergeArgs va{};
  va.stats = la.stats;
  va.nvt = nvt;
  va.rowstat = at<float2>(workspace, p.rowstat);
  float *rs_draw = at<float>(workspace, p.rs_draw);

  if (p.spec) {
    // first read and every draw in one pass: canvas b*(1+nd) + j, slot rows
    // n = (b*(1+nd) + j)*S + s; the draws are used only where a slot is flagged
    const int G = n_draws + 1;
    sa.grp_first = G;
    sa.grp_draw = G;
    sa.off_draw = 1;
    // patched draws: a base canvas's k, v are read only within its slots'
    // windows, so only those rows are projected (a list built with the canvases)
    const bool win = p.patch && !full;
    if (win) {
      sa.W = window_of(d);
      sa.win_pos = at<int32_t>(workspace, p.win_pos);
      sa.win_cnt = at<int32_t>(workspace, p.win_cnt);
      sa.win_ids = at<int32_t>(workspace, p.win_ids);
      sa.win_rows = at<int32_t>(workspace, p.win_rows);
      sa.win_total = at<int32_t>(workspace, p.win_total);
      DG_TRY_HIP(dg::launch_clear_i32(sa.win_total, 1, st), "window row count clear launch");
    }
    DG_TRY_HIP(dg::launch_slot_spec_build(sa, sa.draw_ids, rs_draw, st), "read canvas launch");
    if (full) {
      // every row of the B*G canvases through S0..S3, then the slot rows' LM head
      s = run_block(d, w, kv, batch * G, G, sa.draw_ids, nullptr, nullptr, nullptr, q, k, v, o,
                    p.draws, part_o, part_ml, proj_part, h, st, Stages(), gq);
      if (s != DG_OK) return s;
      la.nrows = (int64_t)batch * G * n_slots;
      la.row_scale = rs_draw;
      la.lab_span = G * n_slots;
      DG_TRY_HIP(dg::launch_lmhead(la, bf, st), "slot LM head launch");
      va.nrows = la.nrows;
      DG_TRY_HIP(dg::launch_vocab_merge(va, st), "slot vocabulary merge launch");
      DG_TRY_HIP(dg::launch_slot_finish(sa, st), "slot read finish launch");
      return ok();
    }
    // The draws differ from canvas b only at the slot positions: k, v of
    // canvas b are projected once and written into its draws as well, then the
    // draws' slot rows are projected (over those copies) with the q of every
    // slot row.
    dg::QkvArgs qa{};
    qa.ids = canvas_ids;
    qa.embed = w->embed;
    qa.wq = w->wq;
    qa.wk = w->wk;
    qa.wv = w->wv;
    qa.q = q;
    qa.k = k;
    qa.v = v;
    qa.M = (int64_t)batch * d.canvas;
    qa.d = d.d_model;
    qa.nq = d.n_q_heads * d.head_dim;
    qa.nkv = d.n_kv_heads * d.head_dim;
    qa.vocab = d.vocab;
    qa.C = d.canvas;
    qa.q_scale = q_scale_of(d);
    qa.col0 = qa.nq;
    qa.col1 = qa.nq + 2 * qa.nkv;
    qa.kv_row = sa.kv_row_base;
    qa.part = proj_part;
    // patched draws: canvas b's k, v once (rows b*C), read by every draw
    qa.kv_copies = p.patch ? 0 : G - 1;   // else the draws' copies of canvas b's k, v
    if (win) {   // the listed rows only (their count is on the device)
      qa.ids = sa.win_ids;
      qa.kv_row = sa.win_rows;
      qa.m_dev = sa.win_total;
    }
    DG_TRY_HIP(dg::launch_qkv(qa, bf, st), "k/v projection launch");
    dg::QkvArgs qg = qa;
    qg.kv_copies = 0;
    qg.m_dev = nullptr;
    qg.ids = sa.qids;
    qg.M = (int64_t)batch * G * n_slots;
    qg.C = n_slots;
    qg.col0 = 0;
    qg.kv_row = sa.kv_row_slot;
    if (p.patch) {   // the slot rows' k, v to their compact rows
      qg.k = kpatch;
      qg.v = vpatch;
      qg.kv_row = nullptr;
    }
    DG_TRY_HIP(dg::launch_qkv(qg, bf, st), "slot-row projection launch");
    Gather gd = gq;
    gd.qkv_done = true;
    if (p.patch) {   // the first read (j = 0) keeps its base rows
      gd.kpatch = kpatch;
      gd.vpatch = vpatch;
      gd.patch_from = 1;
      if (win) {
        gd.win_pos = sa.win_pos;
        gd.win_cnt = sa.win_cnt;
      }
    }
    s = run_block(d, w, kv, batch * G, G, sa.draw_ids, nullptr, nullptr, nullptr, q, k, v, o,
                  p.draws, part_o, part_ml, proj_part, h, st, Stages(), gd);
    if (s != DG_OK) return s;
    la.nrows = (int64_t)batch * G * n_slots;
    la.row_scale = rs_draw;
    la.lab_span = G * n_slots;
    DG_TRY_HIP(dg::launch_lmhead(la, bf, st), "slot LM head launch");
    va.nrows = la.nrows;
    DG_TRY_HIP(dg::launch_vocab_merge(va, st), "slot vocabulary merge launch");
    DG_TRY_HIP(dg::launch_slot_finish(sa, st), "slot read finish launch");
    return ok();
  }

  // first read over the prefilled canvases.  With draws to come (slot-row
  // order), canvas b's k, v go to canvas slot b * n_draws, where its first draw
  // will be; a re-read copies them to its other draws and projects only the
  // draws' slot rows.
  sa.grp_first = 1;
  sa.grp_draw = n_draws;
  sa.off_draw = 0;
  const bool draw_copies = !full && n_draws > 1 && !p.patch;
  Gather g1 = gq;
  if (draw_copies) g1.kv_cmul = n_draws;
  DG_TRY_HIP(dg::launch_slot_rows(sa, st), "slot row launch");
  s = run_block(d, w, kv, batch, 1, canvas_ids, nullptr, nullptr, nullptr, q, k, v, o, p.first,
                part_o, part_ml, proj_part, h, st, Stages(), g1);
  if (s != DG_OK) return s;
  la.nrows = (int64_t)batch * n_slots;
  la.row_scale = row_scale;
  la.lab_span = n_slots;
  DG_TRY_HIP(dg::launch_lmhead(la, bf, st), "slot LM head launch");
  va.nrows = la.nrows;
  DG_TRY_HIP(dg::launch_vocab_merge(va, st), "slot vocabulary merge launch");
  DG_TRY_HIP(dg::launch_slot_first(sa, st), "slot first-read launch");
  if (n_draws == 1) return ok();

  // re-read of flagged canvases: n_draws noise copies in one batched pass
  DG_TRY_HIP(dg::launch_slot_build_draws(sa, st), "draw canvas launch");
  int32_t *row_active = at<int32_t>(workspace, p.row_active);
  DG_TRY_HIP(dg::launch_slot_draw_rows2(sa, row_active, rs_draw, st), "draw row launch");
  Gather gd = gq;
  if (draw_copies) {
    // the draws differ from canvas b only at the slot positions: copy b's k, v
    // into its other draws, then project q, k, v of the draws' slot rows, whose
    // k, v land at their positions in the draw canvases
    const size_t nkv = (size_t)d.n_kv_heads * d.head_dim;
    DG_TRY_HIP(dg::launch_slot_copy_kv(sa, k, v, (int64_t)(nkv * tsize(d)), st), "draw k/v copy launch");
    dg::QkvArgs qd{};
    qd.ids = sa.qids;
    qd.embed = w->embed;
    qd.wq = w->wq;
    qd.wk = w->wk;
    qd.wv = w->wv;
    qd.q = q;
    qd.k = k;
    qd.v = v;
    qd.active = sa.draw_active;
    qd.M = (int64_t)batch * n_draws * n_slots;
    qd.d = d.d_model;
    qd.nq = d.n_q_heads * d.head_dim;
    qd.nkv = (int)nkv;
    qd.vocab = d.vocab;
    qd.C = n_slots;            // rows per draw canvas (its active flag)
    qd.q_scale = q_scale_of(d);
    qd.col0 = 0;
    qd.col1 = qd.nq + 2 * qd.nkv;
    qd.kv_row = sa.kv_row_slot;
    qd.part = proj_part;
    DG_TRY_HIP(dg::launch_qkv(qd, bf, st), "draw slot-row projection launch");
    gd.qkv_done = true;
  } else if (p.patch) {
    // patched draws: the draws read canvas b's k, v (rows b*C) with their own
    // slot rows, projected here to compact rows
    dg::QkvArgs qd{};
    qd.ids = sa.qids;
    qd.embed = w->embed;
    qd.wq = w->wq;
    qd.wk = w->wk;
    qd.wv = w->wv;
    qd.q = q;
    qd.k = kpatch;
    qd.v = vpatch;
    qd.active = sa.draw_active;
    qd.M = (int64_t)batch * n_draws * n_slots;
    qd.d = d.d_model;
    qd.nq = d.n_q_heads * d.head_dim;
    qd.nkv = d.n_kv_heads * d.head_dim;
    qd.vocab = d.vocab;
    qd.C = n_slots;            // rows per draw canvas (its active flag)
    qd.q_scale = q_scale_of(d);
    qd.col0 = 0;
    qd.col1 = qd.nq + 2 * qd.nkv;
    qd.part = proj_part;
    DG_TRY_HIP(dg::launch_qkv(qd, bf, st), "draw slot-row projection launch");
    gd.qkv_done = true;
    gd.kpatch = kpatch;
    gd.vpatch = vpatch;
    gd.patch_from = 0;
  }
  s = run_block(d, w, kv, batch * n_draws, n_draws, sa.draw_ids, nullptr, sa.draw_active, nullptr,
                q, k, v, o, p.draws, part_o, part_ml, proj_part, h, st, Stages(), gd);
  if (s != DG_OK) return s;
  la.nrows = (int64_t)batch * n_draws * n_slots;
  la.active_rows = row_active;
  la.rows_per_flag = 1;
  la.row_scale = rs_draw;
  la.lab_span = n_draws * n_slots;
  DG_TRY_HIP(dg::launch_lmhead(la, bf, st), "draw LM head launch");
  va.nrows = la.nrows;
  DG_TRY_HIP(dg::launch_vocab_merge(va, st), "draw vocabulary merge launch");
  DG_TRY_HIP(dg::launch_slot_average(sa, st), "draw average launch");
  return ok();
}

}  // namespace

extern "C" {

size_t dg_slot_read_workspace(const dg_dims *dims, int32_t batch, int32_t n_slots,
                              int32_t max_prompt, int32_t n_draws) {
  return slot_read_workspace(dims, batch, n_slots, max_prompt, n_draws, false);
}

size_t dg_slot_read_full_canvas_workspace(const dg_dims *dims, int32_t batch, int32_t n_slots,
                                          int32_t max_prompt, int32_t n_draws) {
  return slot_read_workspace(dims, batch, n_slots, max_prompt, n_draws, true);
}

dg_status dg_slot_read(const dg_dims *dims, const dg_weights *w, const dg_prompt_kv *kv,
                       int32_t batch, const int32_t *canvas_ids, int32_t n_slots,
                       const int32_t *slot_pos, const int32_t *label_ids, const int32_t *n_labels,
                       const int32_t *noise_ids, float logit_scale, const float *row_scale,
                       float entropy_threshold, int32_t n_draws, float *logprobs, float *probs,
                       float *entropy, float *first_entropy, int32_t *best, int32_t *draws_used,
                       int32_t *status, void *workspace, size_t ws_bytes, void *stream) {
  return slot_read(dims, w, kv, batch, canvas_ids, n_slots, slot_pos, label_ids, n_labels,
                   noise_ids, logit_scale, row_scale, entropy_threshold, n_draws, logprobs, probs,
                   entropy, first_entropy, best, draws_used, status, workspace, ws_bytes, stream,
                   false);
}

dg_status dg_slot_read_full_canvas(const dg_dims *dims, const dg_weights *w,
                                   const dg_prompt_kv *kv, int32_t batch,
                                   const int32_t *canvas_ids, int32_t n_slots,
                                   const int32_t *slot_pos, const int32_t *label_ids,
                                   const int32_t *n_labels, const int32_t *noise_ids,
                                   float logit_scale, const float *row_scale,
                                   float entropy_threshold, int32_t n_draws, float *logprobs,
                                   float *probs, float *entropy, float *first_entropy,
                                   int32_t *best, int32_t *draws_used, int32_t *status,
                                   void *workspace, size_t ws_bytes, void *stream) {
  return slot_read(dims, w, kv, batch, canvas_ids, n_slots, slot_pos, label_ids, n_labels,
                   noise_ids, logit_scale, row_scale, entropy_threshold, n_draws, logprobs, probs,
                   entropy, first_entropy, best, draws_used, status, workspace, ws_bytes, stream,
                   true);
}

}  // extern "C"

namespace {
// Workspace of a two-stage read: the stage copies, then dg_slot_read's.
struct StagedPlan {
  size_t pos, lab, nlab, noise, rs, lp, pr, ent, fent, best, draws, status, pinned, inner,
      inner_bytes, total;
};

StagedPlan plan_staged(const dg_dims &d, int B, int S, int max_prompt, int nd) {
  StagedPlan p{};
  const size_t BS = (size_t)B * S;
  Arena a;
  p.pos = a.take(BS * 4);
  p.lab = a.take(BS * DG_MAX_LABELS * 4);
  p.nlab = a.take(BS * 4);
  p.noise = a.take((size_t)(nd > 1 ? nd : 1) * BS * 4);
  p.rs = a.take(BS * 4);
  p.lp = a.take(BS * DG_MAX_LABELS * 4);
  p.pr = a.take(BS * DG_MAX_LABELS * 4);
  p.ent = a.take(BS * 4);
  p.fent = a.take(BS * 4);
  p.best = a.take(BS * 4);
  p.draws = a.take(BS * 4);
  p.status = a.take(BS * 4);
  p.pinned = a.take((size_t)B * d.canvas * 4);
  // a stage reads any number of the slots, and the read's workspace is not
  // monotone in the slot count (speculated draws, split-K partials): take the
  // largest over 1..S
  p.inner_bytes = slot_ws_bound(d, B, S, max_prompt, nd);
  for (int n = 1; n < S; ++n)
    p.inner_bytes = std::max(p.inner_bytes, slot_ws_bound(d, B, n, max_prompt, nd));
  p.inner = a.take(p.inner_bytes);
  p.total = a.off;
  return p;
}
}  // namespace

extern "C" {

size_t dg_slot_read_staged_workspace(const dg_dims *dims, int32_t batch, int32_t n_slots,
                                     int32_t max_prompt, int32_t n_draws) {
  if (dg_slot_read_validate(dims, batch, n_slots, n_draws, 0.1f) != DG_OK || max_prompt < 0 ||
      max_prompt > kMaxPrompt)
    return 0;
  return plan_staged(*dims, batch, n_slots, max_prompt, n_draws).total;
}

dg_status dg_slot_read_staged(const dg_dims *dims, const dg_weights *w, const dg_prompt_kv *kv,
                              int32_t batch, const int32_t *canvas_ids, int32_t n_slots,
                              const int32_t *slot_pos, const int32_t *label_ids,
                              const int32_t *n_labels, const int32_t *noise_ids,
                              const int32_t *slot_stage, const int32_t *ask_if_slot,
                              const int32_t *ask_if_label, float logit_scale,
                              const float *row_scale, float entropy_threshold, int32_t n_draws,
                              float *logprobs, float *probs, float *entropy, float *first_entropy,
                              int32_t *best, int32_t *draws_used, int32_t *status,
                              void *workspace, size_t ws_bytes, void *stream) {
  dg_status s = dg_slot_read_validate(dims, batch, n_slots, n_draws, entropy_threshold);
  if (s != DG_OK) return s;
  if (n_slots > DG_MAX_STAGED_SLOTS)
    return fail(DG_ERR_INVALID_ARG, "n_slots %d exceeds %d for a staged read", n_slots,
                DG_MAX_STAGED_SLOTS);
  if (n_slots > 0 && (!slot_stage || !ask_if_slot || !ask_if_label))
    return fail(DG_ERR_INVALID_ARG, "slot_stage, ask_if_slot and ask_if_label are required");
  dg::StagedArgs st0{}, st1{};
  for (int q = 0; q < n_slots; ++q) {
    if (slot_stage[q] != 0 && slot_stage[q] != 1)
      return fail(DG_ERR_INVALID_ARG, "slot %d: stage %d is neither 0 nor 1", q, slot_stage[q]);
    const int c = ask_if_slot[q];
    if (c != -1) {
      if (slot_stage[q] != 1 || c < 0 || c >= n_slots || slot_stage[c] != 0)
        return fail(DG_ERR_INVALID_ARG, "slot %d: ask_if_slot %d must name a stage-0 slot of a "
                    "stage-1 question", q, c);
      if (ask_if_label[q] < 0 || ask_if_label[q] >= DG_MAX_LABELS)
        return fail(DG_ERR_INVALID_ARG, "slot %d: ask_if_label %d outside [0, %d)", q,
                    ask_if_label[q], DG_MAX_LABELS);
    }
    dg::StagedArgs &g = slot_stage[q] == 0 ? st0 : st1;
    g.idx[g.n] = q;
    g.ask_slot[g.n] = c;
    g.ask_label[g.n] = c >= 0 ? ask_if_label[q] : 0;
    ++g.n;
  }
  s = check_model(dims, batch, kv ? kv->max_len : 0, w, kv);
  if (s != DG_OK) return s;
  if (batch == 0 || n_slots == 0) return ok();
  if (!canvas_ids || !slot_pos || !label_ids || !n_labels || !logprobs || !probs || !entropy ||
      !first_entropy || !best || !draws_used || !status)
    return fail(DG_ERR_INVALID_ARG, "slot-read input and output arrays must not be NULL");
  if (n_draws > 1 && !noise_ids) return fail(DG_ERR_INVALID_ARG, "noise_ids is required when n_draws > 1");
  if (!aligned16(workspace)) return fail(DG_ERR_INVALID_ARG, "workspace must be 16-byte aligned");
  const dg_dims &d = *dims;
  const StagedPlan p = plan_staged(d, batch, n_slots, kv->max_len, n_draws);
  if (!workspace || ws_bytes < p.total)
    return fail(DG_ERR_WORKSPACE, "workspace of %zu bytes is smaller than the %zu bytes needed",
                ws_bytes, p.total);
  hipStream_t hs = static_cast<hipStream_t>(stream);
  for (dg::StagedArgs *g : {&st0, &st1}) {
    g->S = n_slots;
    g->B = batch;
    g->C = d.canvas;
    g->nd = n_draws;
    g->slot_pos = slot_pos;
    g->label_ids = label_ids;
    g->n_labels = n_labels;
    g->noise_ids = n_draws > 1 ? noise_ids : nullptr;
    g->row_scale = row_scale;
    g->pos_s = at<int32_t>(workspace, p.pos);
    g->lab_s = at<int32_t>(workspace, p.lab);
    g->nlab_s = at<int32_t>(workspace, p.nlab);
    g->noise_s = at<int32_t>(workspace, p.noise);
    g->rs_s = at<float>(workspace, p.rs);
    g->lp_s = at<float>(workspace, p.lp);
    g->pr_s = at<float>(workspace, p.pr);
    g->ent_s = at<float>(workspace, p.ent);
    g->fent_s = at<float>(workspace, p.fent);
    g->best_s = at<int32_t>(workspace, p.best);
    g->draws_s = at<int32_t>(workspace, p.draws);
    g->status_s = at<int32_t>(workspace, p.status);
    g->logprobs = logprobs;
    g->probs = probs;
    g->entropy = entropy;
    g->first_entropy = first_entropy;
    g->best = best;
    g->draws_used = draws_used;
    g->status = status;
    g->canvas = canvas_ids;
    g->pinned = at<int32_t>(workspace, p.pinned);
  }
  void *inner = at<char>(workspace, p.inner);
  auto read_stage = [&](const dg::StagedArgs &g, const int32_t *ids) -> dg_status {
    if (g.n == 0) return DG_OK;
    DG_TRY_HIP(dg::launch_staged_gather(g, hs), "stage gather launch");
    dg_status r = dg_slot_read(dims, w, kv, batch, ids, g.n, g.pos_s, g.lab_s, g.nlab_s,
                               g.noise_ids ? g.noise_s : nullptr, logit_scale,
                               row_scale ? g.rs_s : nullptr, entropy_threshold, n_draws,
                               const_cast<float *>(g.lp_s), const_cast<float *>(g.pr_s),
                               const_cast<float *>(g.ent_s), const_cast<float *>(g.fent_s),
                               const_cast<int32_t *>(g.best_s), const_cast<int32_t *>(g.draws_s),
                               const_cast<int32_t *>(g.status_s), inner, p.inner_bytes, stream);
    if (r != DG_OK) return r;
    DG_TRY_HIP(dg::launch_staged_scatter(g, hs), "stage scatter launch");
    return DG_OK;
  };
  s = read_stage(st0, canvas_ids);
  if (s != DG_OK) return s;
  if (st1.n > 0) {
    DG_TRY_HIP(dg::launch_staged_pin(st0, hs), "answer pinning launch");
    s = read_stage(st1, st0.pinned);
    if (s != DG_OK) return s;
  }
  return ok();
}

dg_status dg_prepare_embed_t(const dg_dims *dims, const void *embed, void *embed_t, void *stream) {
  dg_status s = check_dims(dims);
  if (s != DG_OK) return s;
  if (!embed || !embed_t) return fail(DG_ERR_INVALID_ARG, "embed and embed_t are required");
  DG_TRY_HIP(dg::launch_transpose(embed, embed_t, dims->vocab, dims->d_model,
                                  dims->dtype == DG_BF16, static_cast<hipStream_t>(stream)),
             "transpose launch");
  return ok();
}

dg_status dg_prepare_lm_tiled(const dg_dims *dims, const void *head, void *lm_tiled,
                              void *stream) {
  dg_status s = check_dims(dims);
  if (s != DG_OK) return s;
  if (!head || !lm_tiled) return fail(DG_ERR_INVALID_ARG, "head and lm_tiled are required");
  if (!aligned16(head) || !aligned16(lm_tiled))
    return fail(DG_ERR_INVALID_ARG, "head and lm_tiled must be 16-byte aligned");
  if (dims->dtype != DG_BF16 || dims->d_model % 32)
    return fail(DG_ERR_UNSUPPORTED, "the blocked LM head needs bf16 and d_model %% 32 == 0");
  DG_TRY_HIP(dg::launch_tile_lm(head, lm_tiled, dims->vocab, dims->d_model,
                                static_cast<hipStream_t>(stream)),
             "LM head tiling launch");
  return ok();
}

dg_status dg_prepare_lm_fp8(const dg_dims *dims, const void *head, void *codes, int32_t *exps,
                            void *stream) {
  dg_status s = check_dims(dims);
  if (s != DG_OK) return s;
  if (!head || !codes || !exps) return fail(DG_ERR_INVALID_ARG, "head, codes and exps are required");
  if (!aligned16(head) || !aligned16(codes) || !aligned16(exps))
    return fail(DG_ERR_INVALID_ARG, "head, codes and exps must be 16-byte aligned");
  if (dims->dtype != DG_BF16)
    return fail(DG_ERR_UNSUPPORTED, "the e4m3 LM head is made from a bf16 head");
  DG_TRY_HIP(dg::launch_quantize_e4m3(head, static_cast<uint8_t *>(codes), exps, dims->vocab,
                                      dims->d_model, static_cast<hipStream_t>(stream)),
             "e4m3 quantisation launch");
  return ok();
}

dg_status dg_prepare_embed_t_tiled(const dg_dims *dims, const void *embed_t,
                                   void *embed_t_tiled, void *stream) {
  dg_status s = check_dims(dims);
  if (s != DG_OK) return s;
  if (!embed_t || !embed_t_tiled)
    return fail(DG_ERR_INVALID_ARG, "embed_t and embed_t_tiled are required");
  if (!aligned16(embed_t) || !aligned16(embed_t_tiled))
    return fail(DG_ERR_INVALID_ARG, "embed_t and embed_t_tiled must be 16-byte aligned");
  if (dims->dtype != DG_BF16 || dims->d_model % 256)
    return fail(DG_ERR_UNSUPPORTED, "the blocked embed^T needs bf16 and d_model %% 256 == 0");
  // embed^T is [d_model, vocab]: blocks of 256 of its rows x 32 of its columns
  DG_TRY_HIP(dg::launch_tile_lm(embed_t, embed_t_tiled, dims->d_model, dims->vocab,
                                static_cast<hipStream_t>(stream)),
             "embed^T tiling launch");
  return ok();
}

}  // extern "C"
