// Internal launch interface between the C-ABI layer and the kernels.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "dg.h"

namespace dg {

// Vocabulary tile of the LM-head statistics (and of the p~ rescale factors).
constexpr int VTILE = 256;
// Self-conditioning GEMM: d columns per workgroup (bf16), and whether a
// vocabulary range's workgroups are kept on one XCD
constexpr int kScTileD = 256;
constexpr bool kScGroup = false;

struct QkvArgs {
  const int32_t *ids;      // [M] token ids
  const void *embed;       // [V, d]
  const void *sc_in;       // [M, d] or null
  const void *wq, *wk, *wv;
  void *q, *k, *v;         // [M, nq], [M, nkv], [M, nkv]
  const int32_t *active;   // per-canvas flag or null (rows of inactive canvases skipped)
  int32_t *flags;          // device flag word or null
  float q_scale;            // q is written as (x Wq^T) * q_scale
  int64_t M;
  int d, nq, nkv, vocab, C;
  int col0, col1;          // output columns [col0, col1) of [q | k | v]
  // row of k and v that input row m writes (-1: none), or null (row m)
  const int32_t *kv_row;
  // split-K partials [proj_ksplit][M][col1 - col0] fp32, or null (no split)
  float *part;
  int ksplit, kchunk;      // set by the launcher
  // each k, v row written is also written kv_copies more times, C, 2C, ...
  // rows further on (the canvases that follow, holding copies of it)
  int kv_copies;
  // rows past *m_dev (a count on the device, at most M) are skipped, or null
  const int32_t *m_dev;
  // with no kv_row map and kv_cmul > 1: input row m of canvas m / C writes
  // k, v row (m / C) * kv_cmul * C + m % C (canvas c's k, v land in canvas slot
  // c * kv_cmul, the first of kv_cmul canvases that will hold copies of it)
  int kv_cmul;
  int rchunks;             // runs of row tiles per weight tile (set by the launcher)
};

struct OprojArgs {
  const void *o;           // [M, kdim]
  const void *wo;          // [d, kdim]
  const int32_t *ids;
  const void *embed, *sc_in;
  void *h;                 // [M, d]
  const int32_t *active;
  int64_t M;
  int d, kdim, vocab, C;
  // split-K partials [proj_ksplit][M][d] fp32, or null (no split)
  float *part;
  int ksplit, kchunk;      // set by the launcher
  // bf16 only: o is fp32 [M, kdim], taken as bf16 hi and lo halves (the
  // product runs over 2 kdim columns, Wo read twice), and h is written as bf16
  // [M, 2d] rows: hi = bf16(h) in columns [0, d), lo = bf16(h - hi) in [d, 2d)
  int prec;
  int rchunks;             // runs of row tiles per weight tile (set by the launcher)
};

struct LmheadArgs {
  const void *head;        // [V, d]
  const void *head_tiled;  // the same in 256 x 32 blocks (bf16), or null
  const uint8_t *head_fp8;  // e4m3 codes [V, d] (bf16 storage only), or null
  const int32_t *head_exp;  // [V]: head row v = decode(codes[v]) * 2^head_exp[v]
  const void *h;           // [*, d]
  const int32_t *row_index;  // [nrows] rows of h to use (-1 = none) or null (identity)
  const int32_t *active_rows;  // per-group flag (groups of rows_per_flag rows) or null
  int rows_per_flag;
  float logit_scale;
  const float *row_scale;  // [nrows] or null
  // per (row, tile): (m = max l, sum e, sum e*(l - r ln2), argmax bits) with
  // e = e^(l - r ln2), r = tile_ref(m)
  float4 *stats;           // [nrows, nvt]
  void *ptilde;            // T or null: e^(l - r ln2) of the row's tile, [nrows, V]
  // row-major, or (ptilde_blocked) in blocks of 256 rows x 32 vocabulary
  // entries: (n, v) at ((n / 256) * (V / 32) + v / 32) * 8192 + (n % 256) * 32 + v % 32
  int ptilde_blocked;
  float *logits;           // [nrows, V] or null
  // label logits of slot rows (optional): row n belongs to slot
  // bs = (n / lab_span) * lab_S + n % lab_S, whose lab_n[bs] label ids are
  // lab_ids[bs * 26 + q]; the scaled logit of label q goes to lab_logit[n * 26 + q]
  const int32_t *lab_ids;
  const int32_t *lab_n;
  float *lab_logit;
  int lab_span, lab_S;
  int64_t nrows;
  int d, vocab, nvt;
  // 1 + an id removed from the softmax (its logit is -inf), or 0 for none
  int exclude_id1;
  // bf16 only: h rows are [*, 2d], bf16 hi = bf16(h) then lo = bf16(h - hi);
  // the logits are those of hi + lo
  int hl;
  // e4m3 activations (with head_fp8; d a multiple of 128), or null: h row n
  // = decode(h_fp8[n]) * 2^h_exp[n] (rows as in h, through row_index)
  const uint8_t *h_fp8;
  const int32_t *h_exp;
};

struct ScArgs {
  const void *ptilde;      // [M, V], row-major or blocked as in LmheadArgs
  int ptilde_blocked;
  const void *embed_t_tiled;  // E^T in 256 x 32 blocks (d % 256 == 0), or null
  const int32_t *shift;    // [M, nvt] p = p~ * 2^-shift / Z
  const float *inv_z;      // [M] 1/Z
  const void *embed_t;     // [d, V]
  float *part;             // [ksplit, M, d]
  void *out;               // [M, d] T
  const int32_t *active;   // per-canvas flag (canvases of C rows) or null
  int64_t M;
  int d, vocab, nvt, ksplit, C;
};

struct VocabMergeArgs {
  const float4 *stats;     // [nrows, nvt]
  int64_t nrows;
  int nvt;
  float *conf, *entropy;   // [nrows] or null
  int32_t *argmax;         // [nrows] or null
  float2 *rowstat;         // [nrows] (m, lse) or null
  int32_t *shift;          // [nrows, nvt] R - r_t (R = max_t r_t) or null
  float *inv_z;            // [nrows] 1/Z, Z = sum_v e^(l_v - R ln2) (with shift)
};

struct AttnArgs {
  const void *q, *k, *v;       // canvas [nc, C, Hq, hd], [nc, C, Hkv, hd]
  const void *kp, *vp;         // prompt [total, Hkv, hd]
  const int32_t *cu;           // [nprompt + 1]
  const int32_t *active;       // per-canvas flag or null
  int32_t *flags;
  // Queries: with qpos null, every canvas position (qn = C); otherwise canvas
  // cb's queries are rows cb*qn + i (i < qn) at canvas positions
  // qpos[cb*qn + i], where a position outside [0, C) names no query (its
  // output row is written and meaningless).  Outputs are laid out by query row.
  const int32_t *qpos;
  int qn;
  void *o;                     // [nc, qn, Hq, hd]
  void *part_o;                // [nsplit, nc*Hq*qn, hd] storage type
  float2 *part_ml;             // [nsplit, nc*Hq*qn]
  int64_t total_len;
  int nc, C, Hq, Hkv, W, max_len, nsplit, chunk, canvas_per_prompt;
  // gathered queries only: one workgroup serves every query head of its kv head
  // (query column c: head kv*G + c / qn, query c % qn); set by the launcher
  int packed;
  // bf16 only: probabilities enter PV as bf16 hi + lo terms; o and the split
  // partials are fp32 (o: [nc, qn, Hq, hd] float)
  int prec;
  // canvas cb's keys and values are canvas cb * kv_cmul of k and v (0 or 1: cb)
  int kv_cmul;
  // gathered queries of cpack consecutive canvases share a tile (set by the
  // launcher; they share their prompt)
  int cpack;
  // Draws read from their base canvas (see attn_patch_supported):
  // with kpatch set, canvas cb's canvas keys are those of canvas
  // cb / canvas_per_prompt of k, v, except, for canvases with
  // cb % canvas_per_prompt >= patch_from, at the positions qpos[cb*qn + s]
  // (shared by the canvases of a base), where they are row cb*qn + s of
  // kpatch / vpatch ([nc*qn, Hkv*hd]).
  const void *kpatch, *vpatch;
  int patch_from;
  // patched tiles: with win_cnt set, the base canvas c's rows a tile reads are
  // its win_cnt[c] positions win_pos[c*C + k] (ascending: the union of the
  // windows of its queries); else every position from the lowest window start
  // to the highest window end
  const int32_t *win_pos, *win_cnt;
  // Encoder mode (causal attention over prompts cut into chunks of C tokens),
  // or null: canvas cb is a chunk, and chunks[cb] = {x: first cache row of its
  // sequence, y: tokens of the sequence before the chunk (its prompt keys are
  // rows [x, x + y) of kp, vp), z: tokens in the chunk (<= C; queries and
  // canvas keys at positions >= z are absent), w: unused}.  A canvas key is
  // visible to the queries at or after it (no window).
  const int4 *chunks;
  // q arrives pre-scaled by log2(e) / sqrt(hd): q.k is the score in log2 units
};

// Encoder-mode layout (encode.hip): B sequences cut into J chunks of C tokens
struct EncodeArgs {
  const int32_t *cu;           // [B + 1] sequence offsets in the cache rows
  const int32_t *prompt_ids;   // [total_len]
  int32_t *flags;
  int32_t *ids_pad;            // [B * J, C] token ids of each chunk (0 past its end)
  int4 *chunks;                // [B * J] AttnArgs::chunks
  int32_t *active;             // [B * J] 1 for a chunk holding tokens
  const void *h_pad, *o_pad;   // [B * J, C, *] rows of the chunks
  void *hidden_out, *attn_out; // [total_len, *] token rows (attn_out may be null)
  int64_t total_len, h_row_bytes, o_row_bytes;
  int B, J, C, max_len;
};

struct CommitArgs {
  const int32_t *ids;
  const float *conf, *entropy;
  const int32_t *argmax;
  uint8_t *mask;
  int32_t *out_ids;
  int32_t *n_committed;
  int B, C, mask_id;
  float tau;
};

// K splits of a projection of M rows x ncols outputs over K (1: none); the
// partial buffer of a split launch holds ksplit * M * ncols floats
int proj_ksplit(int64_t M, int64_t ncols, int K, bool bf);
// K split of a projection: ks splits of kchunk columns each (ks = 1: none)
void proj_split(int64_t M, int64_t ncols, int K, bool bf, int *ks, int *kchunk);
hipError_t launch_qkv(const QkvArgs &a, bool bf, hipStream_t st);
hipError_t launch_oproj(const OprojArgs &a, bool bf, hipStream_t st);
hipError_t launch_lmhead(const LmheadArgs &a, bool bf, hipStream_t st);
hipError_t launch_scgemm(const ScArgs &a, bool bf, hipStream_t st);
int sc_ksplit(int64_t M, int d, int vocab, bool bf);
hipError_t launch_vocab_merge(const VocabMergeArgs &a, hipStream_t st);

// attention: query rows per workgroup, split-KV planning, launch (+ merge)
int attn_query_tile(int head_dim);
// canvases whose gathered queries share one tile: cpp (the canvases that
// share a prompt) when all their queries of a kv group fit a query tile, else 1
int attn_cpack(int qn, bool gathered, int Hq, int Hkv, int head_dim, int cpp);
// whether gathered queries pack the G query heads of a kv head (and the
// cpack canvases) into one tile
bool attn_packed(int qn, bool gathered, int Hq, int Hkv, int head_dim, int cpp);
// qn queries per canvas; gathered: queries at arbitrary positions (every
// canvas key is a candidate) instead of consecutive ones.  nsplit_bound (may
// be null) receives a split count that is >= nsplit for every prompt length
// up to max_len and non-decreasing in max_len: partial buffers sized with it
// fit any shorter prompt.
void attn_plan(int nc, int C, int qn, bool gathered, int Hq, int Hkv, int W, int head_dim,
               int max_len, int cpp, int *nsplit, int *chunk, int *nsplit_bound);
hipError_t launch_attention(const AttnArgs &a, int head_dim, bool bf, hipStream_t st);
// whether draws can read their base canvas's k, v with patched slot rows
// (the bf16 read's precise attention at head_dim 64)
bool attn_patch_supported(int head_dim, bool bf, int n_slots);

hipError_t launch_commit(const CommitArgs &a, hipStream_t st);
// Multi-step loop bookkeeping (one workgroup per canvas).  loop_init: commit
// step -1 everywhere, steps 0, active = the canvas holds a mask id.
// loop_update after the commit of step t: for each active canvas, the
// committed positions take their new ids and commit step t, its step count
// becomes t + 1, it stays active while a mask id remains, and *n_active
// counts the canvases still active (cleared by the caller first).
hipError_t launch_loop_init(const int32_t *ids, int B, int C, int mask_id, int32_t *commit_step,
                            int32_t *steps, int32_t *active, hipStream_t st);
hipError_t launch_loop_update(int32_t *ids, const int32_t *out_ids, const uint8_t *mask, int B,
                              int C, int mask_id, int t, int32_t *commit_step, int32_t *steps,
                              int32_t *active, int32_t *n_active, hipStream_t st);
// bf16 [rows, cols] -> blocks of 256 rows x 32 columns (rows % 256 == 0, cols % 32 == 0)
hipError_t launch_tile_lm(const void *src, void *dst, int rows, int cols, hipStream_t st);
// e4m3 copy of a bf16 [rows, cols] head: per-row exponents and codes
hipError_t launch_quantize_e4m3(const void *head, uint8_t *codes, int32_t *exps, int rows, int cols,
                                hipStream_t st);
hipError_t launch_transpose(const void *src, void *dst, int rows, int cols, bool bf,
                            hipStream_t st);
hipError_t launch_clear_i32(int32_t *p, int64_t n, hipStream_t st);
hipError_t launch_encode_plan(const EncodeArgs &a, hipStream_t st);
hipError_t launch_encode_scatter(const EncodeArgs &a, hipStream_t st);

// slot read pieces
struct SlotArgs {
  const int32_t *slot_pos;     // [B, S]
  const int32_t *label_ids;    // [B, S, 26]
  const int32_t *n_labels;     // [B, S]
  const int32_t *noise_ids;    // [n_draws, B, S]
  // Slot rows of an LM-head pass are laid out as n = (b * grp + j) * S + s:
  // pass j of canvas b (the first read, or draw d), slot s.  The first read is
  // j = 0 with grp_first; draw d is j = off_draw + d with grp_draw.
  const float2 *rowstat;       // per row n: (m, lse)
  const float *lab_logit;      // per row n: scaled label logits [26]
  int grp_first, grp_draw, off_draw;
  const float *row_scale;      // [B, S] or null
  float logit_scale;
  float threshold;
  int B, S, C, V, d, n_draws;
  // Per slot row n (out of the build kernels): its row of the LM-head pass
  // (n itself, or -1 = not read), and for the forward pass its canvas
  // position (-1 = none) and token id there
  int32_t *rows, *qpos, *qids;
  // one-pass reads: k/v row written by base-canvas row b*C + i ([B*C]) and by
  // slot row n ([B*(1+nd)*S], -1 = none: the base canvas already holds it)
  int32_t *kv_row_base, *kv_row_slot;
  int32_t *status;             // [B, S]
  float *logprobs, *probs, *entropy, *first_entropy;
  int32_t *best, *draws_used;
  int32_t *canvas_flag;        // [B + B*S]: canvas has a slot to re-read, then per-slot flags
  int32_t *draw_active;        // [B*nd]
  const int32_t *canvas_ids;   // [B, C]
  int32_t *draw_ids;           // [B*nd, C]
  int mask_id;
  // whole-canvas order: the hidden state has every canvas row, and a slot
  // row's LM-head row is its canvas row (canvas * C + position)
  int full_canvas;
  // one-pass patched reads (win_pos set): the union of the windows (+-W) of
  // base canvas b's slots, as win_cnt[b] ascending positions win_pos[b*C + k],
  // and the same rows of every base canvas in one list for the k/v projection
  // (win_ids: token ids, win_rows: canvas rows b*C + position; win_total counts
  // them, zeroed before the build)
  int W;
  int32_t *win_pos, *win_cnt, *win_ids, *win_rows, *win_total;
};

hipError_t launch_slot_rows(const SlotArgs &a, hipStream_t st);
hipError_t launch_slot_first(const SlotArgs &a, hipStream_t st);
hipError_t launch_slot_build_draws(const SlotArgs &a, hipStream_t st);
hipError_t launch_slot_draw_rows2(const SlotArgs &a, int32_t *row_active, float *rs_draw,
                                  hipStream_t st);
hipError_t launch_slot_average(const SlotArgs &a, hipStream_t st);
// Two-pass draws: for each flagged canvas b, its k and v rows (kv_row_bytes
// bytes per canvas row, stored at canvas slot b * n_draws) are copied to the
// canvas slots b * n_draws + 1 .. b * n_draws + n_draws - 1 of its other draws
hipError_t launch_slot_copy_kv(const SlotArgs &a, void *k, void *v, int64_t kv_row_bytes,
                               hipStream_t st);
// one pass over the first read and every draw: ids of the B*(1+nd) canvases,
// hidden-row indices of their slot rows, and the status of draws with bad noise
hipError_t launch_slot_spec_build(const SlotArgs &a, int32_t *ids, float *rs, hipStream_t st);
// the rest of a one-pass read, one workgroup per canvas: first read, re-read
// flags, noise-id status and draw average
hipError_t launch_slot_finish(const SlotArgs &a, hipStream_t st);
// Two-stage reads: the slots of one stage (idx, by value), gathered from and
// scattered back to the [B, S] arrays of the call.
constexpr int kMaxStagedSlots = 64;
struct StagedArgs {
  int idx[kMaxStagedSlots];        // the stage's slots, in order
  int ask_slot[kMaxStagedSlots];   // per stage slot: condition slot (-1: none)
  int ask_label[kMaxStagedSlots];  // per stage slot: required best label index
  int n, S, B, C, nd;
  const int32_t *slot_pos, *label_ids, *n_labels, *noise_ids;   // [B,S], [B,S,26], [B,S], [nd,B,S]
  const float *row_scale;                                        // [B,S] or null
  int32_t *pos_s, *lab_s, *nlab_s, *noise_s;                     // the stage's copies, n slots
  float *rs_s;
  const float *lp_s, *pr_s, *ent_s, *fent_s;                     // the stage's outputs
  const int32_t *best_s, *draws_s, *status_s;
  float *logprobs, *probs, *entropy, *first_entropy;             // the call's outputs
  int32_t *best, *draws_used, *status;
  const int32_t *canvas;                                         // [B,C]
  int32_t *pinned;                                               // [B,C]
};
// stage copies of slot arrays; slots whose ask_if fails get one label
hipError_t launch_staged_gather(const StagedArgs &a, hipStream_t st);
// stage outputs into the call's outputs; slots whose ask_if fails: not asked
hipError_t launch_staged_scatter(const StagedArgs &a, hipStream_t st);
// pinned = canvas with each stage slot read without error holding its best label
hipError_t launch_staged_pin(const StagedArgs &a, hipStream_t st);

}  // namespace dg
