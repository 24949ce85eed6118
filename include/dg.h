/*
 * dg.h -- C-ABI of the MI355X (gfx950) denoise step, entropy-bounded commit and
 * structured slot read of a DiffusionGemma-style decoder.
 *
 * What the calls compute (pages cited by title and section):
 *   dg_denoise_step  one decoder-mode denoise forward over every canvas position
 *                    (24-ai.news "vLLM integrates DiffusionGemma", section "How is
 *                    diffusion text generation different?": canvas refined in
 *                    parallel, bidirectional attention with a +-W window; thakicloud
 *                    "DiffusionGemma-as-Jev", section "What is DiffusionGemma":
 *                    decoder mode reads the encoder KV), followed by the LM head, the
 *                    vocabulary softmax giving confidence and entropy, and the
 *                    self-conditioning vector (24-ai.news, section "Mechanism for
 *                    deciding completed tokens").
 *   dg_commit        the commit stage (24-ai.news, sections "Mechanism for deciding
 *                    completed tokens" and "Integration into vLLM": denoise and
 *                    commit are separate sampler stages): accept masked positions in
 *                    confidence order until the cumulative entropy exceeds a
 *                    threshold.
 *   dg_slot_read     a read-only denoise forward on a caller-prefilled canvas that
 *                    reports, at each decision slot, the logprobs of the allowed
 *                    single-token labels, their renormalised distribution and its
 *                    entropy (tau-home "DiffusionGemma like Jev", section "Refusing
 *                    JSON token generation"); at most 26 labels (sotaaz "DiffusionGemma
 *                    vLLM example server", section "The server takes at most 26
 *                    alternatives"); a slot whose first-read entropy exceeds a
 *                    threshold (0.1 on that page) is re-read with noise draws (4)
 *                    whose distributions are averaged, n_draws = 1 being "samples: 1".
 *
 * The model is one attention block standing in for the backbone:
 *   x = E[ids] + sc_in;  q,k,v = x Wq^T, x Wk^T, x Wv^T;
 *   o = softmax(q k^T / sqrt(hd)) v over {all prompt keys} U {canvas j : |i-j| <= W},
 *       query head h reading KV head h / (Hq/Hkv);
 *   h = x + o Wo^T;  l = s_i * (h . LM_v);  p = softmax(l);
 *   conf = max p;  entropy = -sum p ln p (nats);  argmax = lowest id of max l;
 *   sc_out = sum_v p_v E_v.
 *
 * Conventions for every call:
 *   - All array pointers are DEVICE pointers unless stated otherwise; the caller
 *     owns every buffer (inputs, outputs and the workspace) and keeps it alive
 *     until the work queued on `stream` has finished.
 *   - Row-major layouts; "T" is the storage type named by dg_dims.dtype (float or
 *     bfloat16).  Accumulation is always fp32.
 *   - Calls are asynchronous on `stream` (a hipStream_t; NULL = the null stream)
 *     and never synchronise the host.  They are safe to call concurrently from
 *     several threads when each uses its own stream and workspace.
 *   - The library never allocates device memory.  Scratch memory is the
 *     caller-provided workspace, sized by the *_workspace queries (except for
 *     dg_slot_read_noalloc, whose workspace is a static device array).
 *   - Host-visible arguments are checked before anything is launched; a failed
 *     check returns a non-zero dg_status, launches nothing and leaves a message
 *     for dg_last_error().  Index data that lives in device memory (token ids,
 *     prompt offsets, slot positions, label ids) is checked inside the kernels,
 *     which never read out of bounds; problems are reported through the
 *     device-side flag / status outputs described below.
 *   - A HIP launch failure returns DG_ERR_HIP.
 */
#ifndef DG_H
#define DG_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define DG_MAX_LABELS 26   /* labels A..Z, one token each */
#define DG_MAX_CANVAS 1024 /* canvas positions per sequence handled by dg_commit */

typedef enum {
    DG_OK = 0,
    DG_ERR_INVALID_ARG = 1,
    DG_ERR_TOO_MANY_LABELS = 2,
    DG_ERR_UNSUPPORTED = 3,
    DG_ERR_WORKSPACE = 4,
    DG_ERR_HIP = 5
} dg_status;

typedef enum { DG_F32 = 0, DG_BF16 = 1 } dg_dtype;

/* Model and canvas dimensions.
 *   d_model    multiple of 32 (of 64 with bf16 storage)
 *   head_dim   64 or 512
 *   n_q_heads  multiple of n_kv_heads (GQA group G = n_q_heads / n_kv_heads)
 *   vocab      multiple of 256
 *   canvas     1 .. DG_MAX_CANVAS positions per sequence
 *   window     W >= 0: canvas query i sees canvas keys j with |i - j| <= W
 *   mask_id    token id of an undecided position, in [0, vocab)
 *   dtype      a dg_dtype: storage type T of weights, prompt KV, sc vectors */
typedef struct {
    int32_t d_model, n_q_heads, n_kv_heads, head_dim, vocab, canvas, window, mask_id;
    int32_t dtype;
} dg_dims;

/* Weights, all T, row-major, device.
 *   embed    [vocab, d_model]  token embedding; also the LM head when lm_head is NULL
 *   embed_t  [d_model, vocab]  the same matrix transposed (see dg_prepare_embed_t);
 *                              required when sc_out is requested, unless
 *                              embed_t_tiled is set
 *   lm_head  [vocab, d_model]  separate LM head, or NULL for a tied head
 *   wq       [n_q_heads*head_dim, d_model]
 *   wk, wv   [n_kv_heads*head_dim, d_model]
 *   wo       [d_model, n_q_heads*head_dim]
 *   lm_tiled the LM head (lm_head, else embed) in the blocked layout written by
 *            dg_prepare_lm_tiled, or NULL.  Optional and bf16 only (ignored for
 *            fp32); the results are the same either way, the blocked layout is
 *            read faster.  Appended after the first seven fields, so a struct
 *            initialised with those seven leaves it NULL.
 *   embed_t_tiled  embed_t in the blocked layout written by dg_prepare_embed_t_tiled,
 *            or NULL.  Optional and bf16 only, for d_model a multiple of 256; when
 *            set, the self-conditioning contraction streams it instead of embed_t
 *            (same results, contiguous 16 KB reads per K step) and sc_out may be
 *            requested without embed_t.
 *   lm_fp8, lm_fp8_exp  an FP8 copy of the LM head written by dg_prepare_lm_fp8, or
 *            NULL: codes [vocab, d_model] uint8 (e4m3) and per-row exponents [vocab]
 *            int32; head row v = decode(codes[v]) * 2^lm_fp8_exp[v].  bf16 only;
 *            when set, every LM-head pass (denoise step, slot read, loop) uses this
 *            head instead of lm_head / embed, with bf16 activations and fp32
 *            accumulation (weight-only FP8: half the bytes per vocabulary pass).
 *            The embedding and p.E keep the bf16 embed.
 *   lm_fp8_act  nonzero, with lm_fp8 set: the denoise step (and the loop) also
 *            quantise each hidden row h[n] to e4m3 by the same rule as the head's
 *            rows (its own power-of-two exponent e_n, the smallest with max |h[n]|
 *            <= 448 * 2^e_n) and run the LM head on the FP8 matrix cores, both
 *            operands e4m3, fp32 accumulation, logits scaled by 2^(e_v + e_n).
 *            Needs d_model a multiple of 128 (DG_ERR_UNSUPPORTED otherwise).  Slot
 *            reads keep bf16 activations.  0 (the default) is weight-only FP8. */
typedef struct {
    const void *embed, *embed_t, *lm_head, *wq, *wk, *wv, *wo;
    const void *lm_tiled;
    const void *embed_t_tiled;
    const void *lm_fp8;
    const int32_t *lm_fp8_exp;
    int32_t lm_fp8_act;
} dg_weights;

/* Cached prompt (encoder-mode) keys and values of every sequence, packed.
 *   k, v        [total_len, n_kv_heads, head_dim] T, device
 *   cu_seqlens  [batch+1] int32, device: sequence b owns rows cu[b] .. cu[b+1]-1;
 *               must be non-decreasing with cu[batch] <= total_len
 *   max_len     host: an upper bound on every cu[b+1]-cu[b] (sizes the split-KV grid)
 *   total_len   host: number of rows allocated in k and v
 * A sequence of length 0 attends to its canvas window only. */
typedef struct {
    const void *k, *v;
    const int32_t *cu_seqlens;
    int32_t max_len;
    int64_t total_len;
} dg_prompt_kv;

/* Stages of dg_denoise_step, in launch order. */
enum {
    DG_STAGE_QKV = 0,         /* embedding gather + q/k/v projection */
    DG_STAGE_ATTENTION = 1,   /* prompt + windowed canvas attention (and split merge) */
    DG_STAGE_OPROJ = 2,       /* output projection + residual */
    DG_STAGE_LMHEAD = 3,      /* LM head with per-tile softmax statistics */
    DG_STAGE_VOCAB_MERGE = 4, /* confidence / entropy / argmax per row */
    DG_STAGE_SELFCOND = 5,    /* p.E self-conditioning (and split-K reduce) */
    DG_N_STAGES = 6
};

/* Optional intermediate outputs and instrumentation (each member may be NULL;
 * pass NULL for the struct to skip them all).  Written in addition to the
 * regular outputs.
 *   attn_out     [batch, canvas, n_q_heads*head_dim] T   attention output o
 *   hidden_out   [batch, canvas, d_model] T              block output h
 *   logits_out   [batch, canvas, vocab] fp32             scaled logits l
 *   stage_events 2*DG_N_STAGES hipEvent_t handles created by the caller, or NULL:
 *                event 2i is recorded on the call's stream just before stage i
 *                and event 2i+1 just after it (a stage that is skipped records
 *                both back to back) */
typedef struct {
    void *attn_out;
    void *hidden_out;
    float *logits_out;
    void **stage_events;
} dg_debug;

/* Device-side input problems reported through *dev_flags (bitwise OR). */
#define DG_FLAG_BAD_TOKEN   1  /* a canvas id outside [0, vocab): embedded as a zero row */
#define DG_FLAG_BAD_SEQLENS 2  /* cu_seqlens not monotone / beyond total_len / longer than
                                  max_len: the prompt range was clamped */

/* Per-slot status codes of dg_slot_read (status[b*n_slots+s]). */
#define DG_SLOT_OK        0
#define DG_SLOT_BAD_POS   1  /* slot position outside [0, canvas): slot skipped */
#define DG_SLOT_BAD_COUNT 2  /* n_labels outside [1, 26]: slot skipped */
#define DG_SLOT_BAD_LABEL 3  /* a label id outside [0, vocab): slot skipped */
#define DG_SLOT_BAD_NOISE 4  /* a noise id outside [0, vocab): the mask id was used instead */
#define DG_SLOT_NOT_ASKED 5  /* dg_slot_read_staged: the slot's ask_if condition did not hold */
#define DG_MAX_STAGED_SLOTS 64 /* slots of one dg_slot_read_staged call */

/* Bytes of workspace dg_denoise_step needs for `batch` sequences whose prompts
 * are at most `max_prompt` long.  Returns 0 for invalid dims. */
size_t dg_denoise_step_workspace(const dg_dims *dims, int32_t batch, int32_t max_prompt);

/* One denoise step over `batch` canvases.
 *   canvas_ids   [batch, canvas] int32   token ids (mask_id at undecided positions)
 *   sc_in        [batch, canvas, d_model] T or NULL (= zero) self-conditioning input
 *   logit_scale  logits are multiplied by logit_scale * row_scale[b, i]
 *   row_scale    [batch, canvas] fp32 or NULL (= 1)
 *   conf         [batch, canvas] fp32  out: max probability
 *   entropy      [batch, canvas] fp32  out: softmax entropy in nats
 *   argmax       [batch, canvas] int32 out: most probable id (lowest on ties)
 *   sc_out       [batch, canvas, d_model] T or NULL: out: sum_v p_v E_v
 *   debug        optional intermediates (may be NULL)
 *   dev_flags    [1] int32 device or NULL: OR of DG_FLAG_* (the call clears it first)
 *   workspace    device buffer of at least dg_denoise_step_workspace(...) bytes,
 *                256-byte aligned
 * Errors: DG_ERR_INVALID_ARG (bad dims/pointers/sizes), DG_ERR_UNSUPPORTED
 * (head_dim not 64/512, dtype unknown), DG_ERR_WORKSPACE (ws_bytes too small),
 * DG_ERR_HIP. */
dg_status dg_denoise_step(const dg_dims *dims, const dg_weights *w, const dg_prompt_kv *kv,
                          int32_t batch, const int32_t *canvas_ids, const void *sc_in,
                          float logit_scale, const float *row_scale,
                          float *conf, float *entropy, int32_t *argmax, void *sc_out,
                          const dg_debug *debug, int32_t *dev_flags,
                          void *workspace, size_t ws_bytes, void *stream);

/* Repeated denoise steps until no canvas holds a mask id: the generation loop
 * of 24-ai.news, "How is diffusion text generation different?" (the canvas is
 * refined over several steps) and "Mechanism for deciding completed tokens"
 * (each step commits the most confident positions until the cumulative
 * entropy exceeds the threshold, and the step's self-conditioning vector
 * p.E is an additional input of the next step).
 * Step t runs dg_denoise_step on the current canvas with sc_in = the previous
 * step's sc_out (the caller's sc_in, or none, at t = 0), then dg_commit with
 * threshold_nats, and writes the committed ids into the canvas.  In the loop
 * the mask id is removed from the vocabulary softmax (its logit is -inf), so
 * confidence, entropy, argmax and p.E cover the other ids and every commit
 * writes a real token: committing the mask id would leave the position
 * undecided and could stall the loop.  A canvas with no mask id left is
 * finished: later steps skip it.
 *   canvas_ids    [batch, canvas] int32, device, in/out: the start canvas; on
 *                 return the final canvas
 *   sc_in         [batch, canvas, d_model] T or NULL (first step only)
 *   logit_scale, row_scale  as in dg_denoise_step (row_scale applies at every step)
 *   threshold_nats  commit threshold, >= 0 (DG_ERR_INVALID_ARG otherwise: the
 *                 loop progresses only if every step commits)
 *   max_steps     at most this many steps (>= 0)
 *   check_every   the host reads back the number of unfinished canvases
 *                 every check_every steps (>= 1) and stops at 0; steps launched
 *                 after the last canvas finished change nothing
 *   commit_step   [batch, canvas] int32, device, out: the step at which each
 *                 position was committed, -1 for positions never committed
 *   steps_taken   [batch] int32, device, out: steps until the canvas finished
 *                 (or max_steps)
 *   steps_launched  host int32 out (may be NULL): steps the call launched
 *   dev_flags     as in dg_denoise_step, accumulated over the steps (may be NULL)
 * Requires weights.embed_t or embed_t_tiled.  The workspace holds a step's
 * workspace plus the loop state; size it with dg_denoise_loop_workspace.
 * The call synchronises the stream every check_every steps (the only host
 * synchronisation of the library); it allocates nothing.
 * Errors: as dg_denoise_step and dg_commit. */
size_t dg_denoise_loop_workspace(const dg_dims *dims, int32_t batch, int32_t max_prompt);
dg_status dg_denoise_loop(const dg_dims *dims, const dg_weights *w, const dg_prompt_kv *kv,
                          int32_t batch, int32_t *canvas_ids, const void *sc_in,
                          float logit_scale, const float *row_scale, float threshold_nats,
                          int32_t max_steps, int32_t check_every, int32_t *commit_step,
                          int32_t *steps_taken, int32_t *steps_launched, int32_t *dev_flags,
                          void *workspace, size_t ws_bytes, void *stream);

/* Encoder-mode prefill of the cached prompt keys and values: the encoder mode
 * fills the KV cache that the decoder-mode denoise step reads (thakicloud,
 * "What is DiffusionGemma"; prefill is a stage of its own in 24-ai.news,
 * "Integration into vLLM infrastructure").  With the single attention block
 * that stands in for the backbone, the cache entry of prompt token t is that
 * block's key and value projection of its embedding:
 *   k_t = E[id_t] Wk^T,  v_t = E[id_t] Wv^T  (no self-conditioning input)
 *   n_tokens    tokens to prefill (>= 0)
 *   prompt_ids  [n_tokens] int32, device; ids outside [0, vocab) embed as zero
 *               rows and set DG_FLAG_BAD_TOKEN in *dev_flags
 *   k_out, v_out  [n_tokens, n_kv_heads, head_dim] T, device (e.g. rows
 *               cu[b] .. cu[b+1]-1 of a packed dg_prompt_kv cache)
 *   dev_flags   device int32 or NULL: cleared, then set as described
 * Uses weights.embed, wk, wv.  Allocates nothing; asynchronous on stream.
 * Errors: DG_ERR_INVALID_ARG, DG_ERR_UNSUPPORTED, DG_ERR_HIP. */
dg_status dg_prefill_kv(const dg_dims *dims, const dg_weights *w, int64_t n_tokens,
                        const int32_t *prompt_ids, void *k_out, void *v_out,
                        int32_t *dev_flags, void *stream);

/* Entropy-bounded commit of `batch` canvases of `canvas` positions each
 * (1 <= canvas <= DG_MAX_CANVAS).  Candidates are positions whose id equals
 * mask_id; they are ranked by (conf descending, position ascending); the
 * candidate at rank k is accepted iff the fp32 sum of the entropies at ranks
 * < k is <= threshold_nats (the candidate that crosses the threshold is
 * accepted; at least one is accepted whenever a candidate exists and the
 * threshold is >= 0).
 *   canvas_ids, argmax [batch, canvas] int32; conf, entropy [batch, canvas] fp32
 *   commit_mask  [batch, canvas] uint8 out: 1 where accepted
 *   out_ids      [batch, canvas] int32 out: argmax where accepted, else canvas_ids
 *   n_committed  [batch] int32 out (may be NULL)
 * out_ids may alias canvas_ids (in-place commit).
 * Errors: DG_ERR_INVALID_ARG, DG_ERR_HIP. */
dg_status dg_commit(int32_t batch, int32_t canvas, int32_t mask_id,
                    const int32_t *canvas_ids, const float *conf, const float *entropy,
                    const int32_t *argmax, float threshold_nats,
                    uint8_t *commit_mask, int32_t *out_ids, int32_t *n_committed,
                    void *stream);

/* Bytes of workspace dg_slot_read needs. */
size_t dg_slot_read_workspace(const dg_dims *dims, int32_t batch, int32_t n_slots,
                              int32_t max_prompt, int32_t n_draws);

/* Encoder-mode forward over the prompts: the encoder mode runs the model over
 * the prompt with left-to-right (causal) attention and fills the KV cache that
 * the decoder-mode denoise step reads (thakicloud, "What is DiffusionGemma").
 * With one block standing in for the backbone:
 *   k_out, v_out  the cache rows, exactly as dg_prefill_kv writes them (every
 *                 row of [0, total_len), k_t = E[id_t] Wk^T, v_t = E[id_t] Wv^T);
 *   attn_out      [total_len, n_q_heads*head_dim] T or NULL: for token t of
 *                 sequence b, softmax(q_t . k_s / sqrt(head_dim)) v_s over the
 *                 tokens s <= t of its own sequence (GQA as in the step), with
 *                 q_t = E[id_t] Wq^T;
 *   hidden_out    [total_len, d_model] T or NULL: the block output
 *                 E[id_t] + attn_t Wo^T, the encoder's hidden state that a
 *                 following block would read.
 * Sequence b owns rows cu_seqlens[b] .. cu_seqlens[b+1]-1 (device int32
 * [batch+1], non-decreasing, <= total_len; offsets outside that are clamped as
 * the step clamps them and set DG_FLAG_BAD_SEQLENS), at most max_len tokens
 * each (host; a longer sequence is cut to its first max_len tokens).  Rows of
 * attn_out / hidden_out outside every sequence are left untouched; rows that
 * clamped sequences share hold the result of one of them.
 *   prompt_ids    [total_len] int32, device; ids outside [0, vocab) embed as zero
 *                 rows and set DG_FLAG_BAD_TOKEN
 *   dev_flags     device int32 or NULL: cleared, then set as described
 * The prompts run in chunks of `canvas` tokens, each chunk attending to the
 * cache rows of its sequence before it and causally within itself.  With
 * hidden_out and attn_out both NULL the call equals dg_prefill_kv over
 * total_len rows (no workspace needed).  Workspace: dg_prefill_encode_workspace
 * bytes (monotone in batch and max_len).  Allocates nothing; asynchronous on
 * stream.  Errors: DG_ERR_INVALID_ARG, DG_ERR_UNSUPPORTED, DG_ERR_WORKSPACE,
 * DG_ERR_HIP. */
size_t dg_prefill_encode_workspace(const dg_dims *dims, int32_t batch, int32_t max_len);
dg_status dg_prefill_encode(const dg_dims *dims, const dg_weights *w, int32_t batch,
                            const int32_t *cu_seqlens, int32_t max_len, int64_t total_len,
                            const int32_t *prompt_ids, void *k_out, void *v_out,
                            void *hidden_out, void *attn_out, int32_t *dev_flags,
                            void *workspace, size_t ws_bytes, void *stream);

/* Structured read of `n_slots` slots in each of `batch` caller-prefilled canvases.
 * The canvas is never modified and nothing is committed.
 *   canvas_ids   [batch, canvas] int32   prefilled skeleton (slots usually mask_id)
 *   slot_pos     [batch, n_slots] int32  slot positions
 *   label_ids    [batch, n_slots, 26] int32 allowed label ids, first n_labels used
 *   n_labels     [batch, n_slots] int32  1..26
 *   noise_ids    [n_draws, batch, n_slots] int32: token that draw d writes at slot s
 *                of canvas b (ignored when n_draws == 1; may then be NULL)
 *   logit_scale, row_scale ([batch, n_slots] fp32 or NULL) scale the slot logits
 *   entropy_threshold  a slot is re-read iff n_draws > 1 and its first-read
 *                entropy is > this
 *   n_draws      1 .. 16; 1 = never re-read
 * Outputs (fp32 unless noted; entries j >= n_labels are 0):
 *   logprobs [batch, n_slots, 26]  ln p(label_j) under the full-vocabulary softmax
 *                                  (draw-averaged in probability space if re-read)
 *   probs    [batch, n_slots, 26]  distribution renormalised over the labels
 *   entropy, first_entropy [batch, n_slots]  entropy of probs; of the first read
 *   best     [batch, n_slots] int32  index j of the most probable label (lowest on ties)
 *   draws_used [batch, n_slots] int32  1, or n_draws if re-read (0 if skipped)
 *   status   [batch, n_slots] int32  DG_SLOT_* code
 * A re-read replaces every slot token of its canvas by that draw's noise id and
 * runs the whole step again; the draws (not the first read) are averaged.
 * Errors: DG_ERR_TOO_MANY_LABELS never arises here (label arrays are fixed at 26;
 * counts are checked per slot); DG_ERR_INVALID_ARG, DG_ERR_UNSUPPORTED,
 * DG_ERR_WORKSPACE, DG_ERR_HIP. */
dg_status dg_slot_read(const dg_dims *dims, const dg_weights *w, const dg_prompt_kv *kv,
                       int32_t batch, const int32_t *canvas_ids, int32_t n_slots,
                       const int32_t *slot_pos, const int32_t *label_ids,
                       const int32_t *n_labels, const int32_t *noise_ids,
                       float logit_scale, const float *row_scale,
                       float entropy_threshold, int32_t n_draws,
                       float *logprobs, float *probs, float *entropy, float *first_entropy,
                       int32_t *best, int32_t *draws_used, int32_t *status,
                       void *workspace, size_t ws_bytes, void *stream);

/* The same read in the whole-canvas order: q, attention and the output
 * projection run over every canvas row of the first read and of the draws,
 * as the layers below the last one of a multi-layer model need every
 * position's hidden state for one denoise forward (tau-home "DiffusionGemma
 * like Jev", section "Refusing JSON token generation": one denoise forward
 * over the prefilled canvas), and the LM head runs at the slot rows.  With
 * the single block standing in for the backbone, the slot rows' results
 * equal dg_slot_read's up to fp32 summation order (dg_slot_read computes q,
 * attention and the output projection at the slot rows only, which is exact
 * for a last block).  Arguments, outputs and errors as dg_slot_read; size the
 * workspace with dg_slot_read_full_canvas_workspace. */
size_t dg_slot_read_full_canvas_workspace(const dg_dims *dims, int32_t batch, int32_t n_slots,
                                          int32_t max_prompt, int32_t n_draws);
dg_status dg_slot_read_full_canvas(const dg_dims *dims, const dg_weights *w,
                                   const dg_prompt_kv *kv, int32_t batch,
                                   const int32_t *canvas_ids, int32_t n_slots,
                                   const int32_t *slot_pos, const int32_t *label_ids,
                                   const int32_t *n_labels, const int32_t *noise_ids,
                                   float logit_scale, const float *row_scale,
                                   float entropy_threshold, int32_t n_draws, float *logprobs,
                                   float *probs, float *entropy, float *first_entropy,
                                   int32_t *best, int32_t *draws_used, int32_t *status,
                                   void *workspace, size_t ws_bytes, void *stream);

/* dg_slot_read without a workspace argument, for callers that cannot allocate
 * device memory (code under graph capture, tight serving loops, harnesses that
 * forbid allocation).  Same arguments, outputs and errors as dg_slot_read; the
 * workspace is a static device array of DG_NOALLOC_SCRATCH_BYTES in the
 * library, one per GPU, held until the process ends, whose address is looked up
 * on the first call on each device.  The call allocates nothing.
 *   - DG_ERR_WORKSPACE when dg_slot_read_workspace(dims, batch, n_slots,
 *     kv->max_len, n_draws) exceeds DG_NOALLOC_SCRATCH_BYTES (the headline
 *     read, 8 slots at d 2816 / V 262,144, needs about 26 MiB).
 *   - Every call on a GPU uses that GPU's one array: calls on the same GPU must
 *     not overlap in time (different streams or threads race on it).  Nothing
 *     in it needs clearing between calls.
 *   - Runs on the device current at the call, which must own `stream`. */
#define DG_NOALLOC_SCRATCH_BYTES (64u << 20)
dg_status dg_slot_read_noalloc(const dg_dims *dims, const dg_weights *w, const dg_prompt_kv *kv,
                               int32_t batch, const int32_t *canvas_ids, int32_t n_slots,
                               const int32_t *slot_pos, const int32_t *label_ids,
                               const int32_t *n_labels, const int32_t *noise_ids,
                               float logit_scale, const float *row_scale,
                               float entropy_threshold, int32_t n_draws,
                               float *logprobs, float *probs, float *entropy, float *first_entropy,
                               int32_t *best, int32_t *draws_used, int32_t *status, void *stream);

/* Two-stage structured read (sotaaz, "The server takes at most 26
 * alternatives per question": a question with ask_if is read only when the
 * answer of an earlier question meets the condition, the draws are taken per
 * stage, and the first answer is written back into the canvas before the
 * second read).  Arguments as dg_slot_read, plus three host arrays of n_slots
 * entries (n_slots <= DG_MAX_STAGED_SLOTS):
 *   slot_stage    0 or 1: the stage that reads the slot
 *   ask_if_slot   -1, or a stage-0 slot c: this stage-1 slot is asked only if
 *                 slot c was read without error (DG_SLOT_OK) with best label
 *                 index ask_if_label[s]
 *   ask_if_label  label index in [0, 26) (used when ask_if_slot >= 0)
 * Stage 0 reads its slots with dg_slot_read (draws put noise at stage-0 slots;
 * stage-1 slots keep the mask id).  The best label of every stage-0 slot read
 * without error is then written at its position in a copy of the canvas, in
 * slot order, and stage 1 reads its slots on that copy (draws put noise at
 * every stage-1 slot).  A slot not asked is read with its first label only (it
 * never asks for draws) and reports zeros, best -1, draws_used 0 and status
 * DG_SLOT_NOT_ASKED.  canvas_ids is never modified.  The workspace holds
 * dg_slot_read's for n_slots slots plus the stage copies; size it with
 * dg_slot_read_staged_workspace.
 * Errors: as dg_slot_read; DG_ERR_INVALID_ARG for a bad stage array. */
size_t dg_slot_read_staged_workspace(const dg_dims *dims, int32_t batch, int32_t n_slots,
                                     int32_t max_prompt, int32_t n_draws);
dg_status dg_slot_read_staged(const dg_dims *dims, const dg_weights *w, const dg_prompt_kv *kv,
                              int32_t batch, const int32_t *canvas_ids, int32_t n_slots,
                              const int32_t *slot_pos, const int32_t *label_ids,
                              const int32_t *n_labels, const int32_t *noise_ids,
                              const int32_t *slot_stage, const int32_t *ask_if_slot,
                              const int32_t *ask_if_label, float logit_scale,
                              const float *row_scale, float entropy_threshold, int32_t n_draws,
                              float *logprobs, float *probs, float *entropy, float *first_entropy,
                              int32_t *best, int32_t *draws_used, int32_t *status,
                              void *workspace, size_t ws_bytes, void *stream);

/* Writes embed_t = embed^T ([d_model, vocab] from [vocab, d_model]), the layout
 * the self-conditioning contraction streams.  Weight preparation, done once. */
dg_status dg_prepare_embed_t(const dg_dims *dims, const void *embed, void *embed_t,
                             void *stream);

/* Writes lm_tiled, the LM head [vocab, d_model] (bf16) in blocks of 256 vocabulary
 * rows x 32 columns: element (v, k) sits at
 *   ((v / 256) * (d_model / 32) + k / 32) * 8192 + (v % 256) * 32 + k % 32,
 * so one K step of a 256-row vocabulary tile is 16 KB of contiguous memory.
 * lm_tiled holds vocab * d_model elements.  Requires dtype DG_BF16 and d_model a
 * multiple of 32 (DG_ERR_UNSUPPORTED otherwise).  Weight preparation, done once;
 * head and lm_tiled are device pointers, 16-byte aligned. */
dg_status dg_prepare_lm_tiled(const dg_dims *dims, const void *head, void *lm_tiled,
                              void *stream);

/* Writes embed_t_tiled, embed^T [d_model, vocab] (bf16) in blocks of 256 rows of
 * d_model x 32 vocabulary columns: element (c, v) of embed^T (= embed[v][c]) sits at
 *   ((c / 256) * (vocab / 32) + v / 32) * 8192 + (c % 256) * 32 + v % 32,
 * so one K step (32 vocabulary entries) of a 256-wide d tile of the
 * self-conditioning contraction is 16 KB of contiguous memory.  Reads embed_t
 * (row-major, from dg_prepare_embed_t); embed_t_tiled holds vocab * d_model
 * elements.  Requires dtype DG_BF16 and d_model a multiple of 256
 * (DG_ERR_UNSUPPORTED otherwise).  Weight preparation, done once; both pointers
 * are device pointers, 16-byte aligned. */
dg_status dg_prepare_embed_t_tiled(const dg_dims *dims, const void *embed_t,
                                   void *embed_t_tiled, void *stream);

/* Writes the FP8 (e4m3) copy of the LM head [vocab, d_model] (bf16): for each
 * vocabulary row v, exps[v] = the smallest integer e with max_k |head[v][k]| <=
 * 448 * 2^e (0 for a zero row), and codes[v][k] = head[v][k] / 2^e rounded to the
 * nearest e4m3 value, ties to even (e4m3: sign, 4 exponent bits with bias 7, 3
 * mantissa bits, subnormals, largest finite 448).  The FP8 variant of the
 * checkpoints the pages measure (24-ai.news, performance section), here as a
 * weight-only format.  codes holds vocab * d_model bytes, exps vocab int32; all
 * device pointers, 16-byte aligned.  Requires dtype DG_BF16 (DG_ERR_UNSUPPORTED
 * otherwise).  Weight preparation, done once. */
dg_status dg_prepare_lm_fp8(const dg_dims *dims, const void *head, void *codes, int32_t *exps,
                            void *stream);

/* Host-only validation (no HIP calls; usable without a GPU).  Same checks the
 * calls above make before launching anything. */
dg_status dg_denoise_step_validate(const dg_dims *dims, int32_t batch, int32_t max_prompt,
                                   const dg_weights *w, const dg_prompt_kv *kv);
dg_status dg_slot_read_validate(const dg_dims *dims, int32_t batch, int32_t n_slots,
                                int32_t n_draws, float entropy_threshold);
dg_status dg_commit_validate(int32_t batch, int32_t canvas);

/* Checks a question's alternative count before a slot is built: more than
 * DG_MAX_LABELS alternatives cannot be given single-token labels A..Z. */
dg_status dg_check_label_count(int32_t n_alternatives);

const char *dg_status_string(dg_status s);
/* Detail message of the last non-OK return on the calling thread ("" if none). */
const char *dg_last_error(void);
/* Library version string. */
const char *dg_version(void);

#ifdef __cplusplus
}
#endif
#endif /* DG_H */
