"""Plain float64 oracle of one decoder-mode denoise step, the entropy-bounded
commit and the structured slot read.

TEST INFRASTRUCTURE ONLY: imported by tests/, the smoke check and the bench's
CPU-baseline leg; never by the HIP library, with which it shares no code.

Sources (the pages this method is described on; cited by page and section):

* 24-ai.news, "vLLM integrates DiffusionGemma" -- section "How is diffusion text
  generation different?": a canvas of 256 tokens refined in parallel; the
  decoder mode uses bidirectional attention with a +-W sliding window.
  Section "Mechanism for deciding completed tokens": per-token confidence,
  accept the most confident tokens until the cumulative entropy exceeds a
  preset threshold; self-conditioning turns the full softmax into a
  probability-weighted embedding mean.  Section "Integration into vLLM":
  prefill / denoise / commit are separate stages.
* thakicloud, "DiffusionGemma-as-Jev" -- section "What is DiffusionGemma": the
  decoder mode reads the encoder-mode KV cache with bidirectional attention.
* tau-home, "DiffusionGemma like Jev" -- section "Refusing JSON token
  generation": the canvas skeleton is prefilled, only decision slots are left
  open, and one denoise forward reads the logprob and entropy of the allowed
  label token ids at each slot.
* sotaaz, "DiffusionGemma vLLM example server" -- section "The server takes at
  most 26 alternatives per question": labels A-Z, one token each, more are
  rejected; when the first read's entropy exceeds 0.1 each stage is read with
  4 draws that are averaged, and "samples: 1" forces a single draw.
* agentlenshq, "DiffusionGemma: 4x faster text generation" -- section
  "Technical architecture": a canvas of random placeholder tokens; every token
  in the 256-block can see every other (the W >= C-1 case).

Readings where the pages are silent (each also listed in the design notes):
one attention block stands in for the backbone (q/k/v/o projections with a
residual, no norm, RoPE or MLP); attention scale 1/sqrt(head_dim); the window
is inclusive |i-j| <= W and every canvas position, masked or not, is a key;
all prompt keys are visible; GQA head h reads KV head floor(h/G); the LM head
is tied to the embedding unless a separate one is given; logits are multiplied
by logit_scale (and an optional per-row scale) before the softmax;
confidence = max probability, committed token = argmax with the lowest id on
ties; entropies in nats with 0 ln 0 = 0; commit acceptance uses the exclusive
prefix of entropies in confidence order (ties to the lower position); the
slot re-read trigger is the entropy of the distribution renormalised over the
allowed labels, strict >, decided per slot; a draw writes its own noise token
at every slot of the canvas and the draws (not the first read) are averaged in
probability space.

Parity status of the whole step against the real DiffusionGemma model:
parity unpinned (the pages print no worked example and ship no weights); each
function below is pinned by the closed forms, library special cases,
invariants and brute force in tests/test_oracle_*.py.
"""
from dataclasses import dataclass
import math

import numpy as np

F64 = np.float64
MAX_LABELS = 26            # sotaaz, "at most 26 alternatives": labels A..Z

# per-slot status codes (shared meaning with the C-ABI's per-slot status)
SLOT_OK = 0
SLOT_BAD_POS = 1           # slot position outside [0, C)
SLOT_BAD_COUNT = 2         # label count outside [1, 26]
SLOT_BAD_LABEL = 3         # a label id outside [0, V)
SLOT_BAD_NOISE = 4         # a noise-draw token id outside [0, V) (replaced by the mask id)
SLOT_NOT_ASKED = 5         # staged read: the slot's ask_if condition did not hold


# --------------------------------------------------------------------------
# S0  input assembly
# --------------------------------------------------------------------------
def embed_input(E, ids, sc_in=None):
    """x_i = E[ids_i] + sc_in_i.

    24-ai.news, "Mechanism for deciding completed tokens": the
    self-conditioning vector of the previous step is an additional model
    input; here it is added to the token embedding (absent = 0).
    An id outside [0, V) names no row; the pages are silent on such input,
    and the reading taken is that it embeds as a zero row (the library flags
    it and does the same).
    """
    E = np.asarray(E, dtype=F64)
    ids = np.asarray(ids)
    ok = (ids >= 0) & (ids < E.shape[0])
    x = np.zeros(ids.shape + (E.shape[1],), dtype=F64)
    x[ok] = E[ids[ok]]
    if sc_in is not None:
        x = x + np.asarray(sc_in, dtype=F64)
    return x


# --------------------------------------------------------------------------
# S1 / S3  projections of the one-block surrogate
# --------------------------------------------------------------------------
def qkv_project(x, Wq, Wk, Wv, n_q_heads, n_kv_heads, head_dim):
    """q = x Wq^T, k = x Wk^T, v = x Wv^T, split into heads.

    W matrices are [out, in] row-major.  Returns q [n, Hq, hd], k and v
    [n, Hkv, hd].
    """
    n = x.shape[0]
    q = x @ np.asarray(Wq, F64).T
    k = x @ np.asarray(Wk, F64).T
    v = x @ np.asarray(Wv, F64).T
    return (q.reshape(n, n_q_heads, head_dim), k.reshape(n, n_kv_heads, head_dim),
            v.reshape(n, n_kv_heads, head_dim))


def prefill_kv(E, Wk, Wv, ids, n_kv_heads, head_dim):
    """Encoder-mode prefill of the prompt KV cache (thakicloud, "What is
    DiffusionGemma": the encoder mode writes the KV cache the decoder reads).
    With one attention block standing in for the backbone, prompt token t's
    cache entry is that block's key/value projection of its embedding:
    k_t = E[id_t] Wk^T, v_t = E[id_t] Wv^T, shaped [n, n_kv_heads, head_dim].
    Ids outside [0, V) embed as zero rows.
    """
    ids = np.asarray(ids)
    ok = (ids >= 0) & (ids < E.shape[0])
    x = np.zeros((len(ids), E.shape[1]), dtype=F64)
    x[ok] = embed_input(E, ids[ok])
    k = x @ np.asarray(Wk, F64).T
    v = x @ np.asarray(Wv, F64).T
    n = x.shape[0]
    return k.reshape(n, n_kv_heads, head_dim), v.reshape(n, n_kv_heads, head_dim)


def causal_attention(q, k, v, rows=None):
    """Causal self-attention over one prompt sequence (encoder mode).

    thakicloud, "What is DiffusionGemma": the encoder mode runs the model over
    the prompt and fills the KV cache that decoder mode reads; encoder-mode
    attention is the ordinary left-to-right (causal) kind.  Query t sees keys
    s <= t of its own sequence.  q: [P, Hq, hd], k, v: [P, Hkv, hd] (GQA head
    h reads kv head h // (Hq / Hkv)); ``rows`` selects the query positions
    (default all).  Returns o: [len(rows), Hq, hd].
    """
    q = np.asarray(q, F64)
    k = np.asarray(k, F64)
    v = np.asarray(v, F64)
    P, Hq, hd = q.shape
    G = Hq // k.shape[1]
    rows = np.arange(P) if rows is None else np.asarray(rows)
    out = np.empty((len(rows), Hq, hd))
    scale = 1.0 / math.sqrt(hd)
    visible = np.arange(P)[None, :] <= rows[:, None]                  # [R, P]
    for h in range(Hq):
        g = h // G
        s = (q[rows, h, :] @ k[:, g, :].T) * scale
        s = np.where(visible, s, -np.inf)
        m = s.max(axis=1, keepdims=True)
        w = np.exp(s - m)
        out[:, h, :] = (w / w.sum(axis=1, keepdims=True)) @ v[:, g, :]
    return out


def encode_prompt(E, Wq, Wk, Wv, Wo, ids, dims, rows=None):
    """Encoder-mode forward of the one-block surrogate over one prompt.

    The block's key and value projections of the prompt embeddings are the
    cache entries (prefill_kv); its queries attend causally (causal_attention)
    and the block output h = x + o Wo^T is the encoder's hidden state, which a
    following block would read.  Ids outside [0, V) embed as zero rows.
    ``rows`` restricts attention and output to those positions.  Returns a
    dict of float64 arrays: k, v [P, Hkv, hd]; attn_out [R, Hq*hd]; hidden_out
    [R, d].
    """
    x = embed_input(E, ids)
    q, k, v = qkv_project(x, Wq, Wk, Wv, dims.n_q_heads, dims.n_kv_heads, dims.head_dim)
    P = x.shape[0]
    rows = np.arange(P) if rows is None else np.asarray(rows)
    o = causal_attention(q, k, v, rows)
    return {"k": k, "v": v, "attn_out": o.reshape(len(rows), -1),
            "hidden_out": block_output(x[rows], o, Wo), "rows": rows}


def block_output(x, o, Wo):
    """h = x + concat_heads(o) Wo^T  (residual around the attention block)."""
    n = o.shape[0]
    return x + o.reshape(n, -1) @ np.asarray(Wo, F64).T


# --------------------------------------------------------------------------
# S2  decoder-mode attention: full prompt KV + +-W canvas window
# --------------------------------------------------------------------------
def window_attention(q, k, v, Kp, Vp, window, rows=None):
    """Bidirectional canvas attention with a +-W window plus the prompt KV.

    24-ai.news, "How is diffusion text generation different?": decoder mode
    attends in both directions within a +-W sliding window over the canvas;
    thakicloud, "What is DiffusionGemma": it reads the encoder (prompt) KV.

    q: [C, Hq, hd] canvas queries; k, v: [C, Hkv, hd] canvas keys/values;
    Kp, Vp: [P, Hkv, hd] prompt keys/values (P may be 0).  ``rows`` selects the
    query positions to compute (default all).  Key set of query i: every
    prompt token, and canvas positions j with |i - j| <= window.
    Returns o: [len(rows), Hq, hd].
    """
    q = np.asarray(q, F64)
    k = np.asarray(k, F64)
    v = np.asarray(v, F64)
    Kp = np.asarray(Kp, F64)
    Vp = np.asarray(Vp, F64)
    C, Hq, hd = q.shape
    Hkv = k.shape[1]
    G = Hq // Hkv
    P = Kp.shape[0]
    rows = np.arange(C) if rows is None else np.asarray(rows)
    jj = np.arange(C)
    canvas_visible = np.abs(rows[:, None] - jj[None, :]) <= window   # [R, C]
    out = np.empty((len(rows), Hq, hd))
    scale = 1.0 / math.sqrt(hd)
    for h in range(Hq):
        g = h // G
        qh = q[rows, h, :]                                            # [R, hd]
        s_prompt = (qh @ Kp[:, g, :].T) * scale                       # [R, P]
        s_canvas = (qh @ k[:, g, :].T) * scale                        # [R, C]
        s_canvas = np.where(canvas_visible, s_canvas, -np.inf)
        s = np.concatenate([s_prompt, s_canvas], axis=1)
        m = s.max(axis=1, keepdims=True)
        w = np.exp(s - m)
        a = w / w.sum(axis=1, keepdims=True)
        out[:, h, :] = a[:, :P] @ Vp[:, g, :] + a[:, P:] @ v[:, g, :]
    return out


# --------------------------------------------------------------------------
# S4  LM head
# --------------------------------------------------------------------------
def lm_logits(h, head, scale, chunk=32768):
    """l_{i,v} = s_i * (h_i . head_v) for every vocabulary row v.

    tau-home, "NVFP4 local run ...": probabilities are read at the engine's
    logit level.  ``head`` is [V, d] (the tied embedding unless a separate LM
    head is given); ``scale`` is a scalar or a per-row array.
    """
    h = np.asarray(h, F64)
    V = head.shape[0]
    out = np.empty((h.shape[0], V))
    for v0 in range(0, V, chunk):
        out[:, v0:v0 + chunk] = h @ np.asarray(head[v0:v0 + chunk], F64).T
    s = np.asarray(scale, F64)
    if s.ndim == 0:
        out *= s
    else:
        out *= s.reshape(-1, 1)
    return out


# --------------------------------------------------------------------------
# FP8 (e4m3) rows: the LM head's copy and, optionally, the hidden rows
# --------------------------------------------------------------------------
E4M3_MAX = 448.0   # largest finite e4m3 value (OCP 8-bit float, 4 exponent bits, bias 7)


def e4m3_row_exponent(amax):
    """Smallest integer e with amax <= 448 * 2^e (0 for an all-zero row).

    With amax = m 2^E, 1 <= m < 2, and 448 = 1.75 2^8: e = E - 8, plus 1 when
    m > 1.75.  Exact (no division).
    """
    amax = np.asarray(amax, dtype=np.float64)
    f, x = np.frexp(amax)                  # amax = f 2^x, 0.5 <= f < 1
    m = 2.0 * f                            # 1 <= m < 2, E = x - 1
    e = (x - 1) - 8 + (m > 1.75)
    return np.where(amax > 0, e, 0).astype(np.int64)


def e4m3_encode(q):
    """Round-to-nearest-even to e4m3 codes (uint8) of values |q| <= 448, taken
    in float64 (exact for float32 and bf16 inputs): subnormals (|q| < 2^-6) are
    multiples of 2^-9, normals have a 3-bit mantissa; a mantissa that rounds up
    to 8 carries into the exponent (for subnormals that carry is the code of
    2^-6 itself)."""
    q = np.asarray(q, dtype=np.float64)
    a = np.abs(q)
    sign = (np.signbit(q)).astype(np.uint8) << 7
    code = np.zeros(a.shape, dtype=np.int64)
    sub = a < 2.0 ** -6
    code[sub] = np.rint(a[sub] * 512.0).astype(np.int64)
    nrm = ~sub
    if nrm.any():
        _, x = np.frexp(a[nrm])
        E = x - 1                                           # a = (1 + f) 2^E
        frac = a[nrm] / np.ldexp(1.0, E) - 1.0              # exact
        m3 = np.rint(frac * 8.0).astype(np.int64)
        carry = m3 == 8
        E = E + carry
        m3 = np.where(carry, 0, m3)
        code[nrm] = ((E + 7) << 3) | m3
    return (code.astype(np.uint8) | sign).astype(np.uint8)


def e4m3_decode(codes):
    """Value of each e4m3 code: (-1)^s (1 + m/8) 2^(e-7), or (-1)^s m 2^-9 for
    e = 0.  (Code 0x7F / 0xFF, not a number, is never produced.)"""
    c = np.asarray(codes, dtype=np.int64)
    s = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = c & 0x7
    val = np.where(e == 0, m * 2.0 ** -9, (1.0 + m / 8.0) * np.exp2(e - 7.0))
    return s * val


def quantize_rows_e4m3(rows):
    """Per row: exponent e (e4m3_row_exponent of the row's largest magnitude)
    and the codes of row / 2^e, all in float64 (the division is exact: a power
    of two).  Returns (codes uint8 [n, d], exps int64 [n])."""
    x = np.asarray(rows, dtype=np.float64)
    e = e4m3_row_exponent(np.abs(x).max(axis=1))
    q = x * np.ldexp(1.0, -e)[:, None]
    return e4m3_encode(q), e


def quantize_head_e4m3(head):
    """quantize_rows_e4m3 of the LM head read as stored (bf16 values are exact
    in float32 and float64).  Returns (codes uint8 [V, d], exps int64 [V])."""
    return quantize_rows_e4m3(np.asarray(head, dtype=np.float32))


def dequantize_head_e4m3(codes, exps):
    """The rows an FP8 operand stands for: decode(code) 2^e, float64."""
    return e4m3_decode(codes) * np.exp2(np.asarray(exps, dtype=np.float64))[:, None]


def fp8_activations(h):
    """The hidden rows as the FP8 LM head sees them with FP8 activations: each
    row quantised to e4m3 by the head's own rule (its power-of-two exponent,
    round to nearest even) and decoded.  The pages name FP8 checkpoints
    (24-ai.news, performance section) without a scale granularity; the reading
    taken is one power-of-two scale per row for both operands."""
    codes, e = quantize_rows_e4m3(h)
    return dequantize_head_e4m3(codes, e)


# --------------------------------------------------------------------------
# S5  vocabulary softmax: confidence, entropy, argmax
# --------------------------------------------------------------------------
@dataclass
class VocabStats:
    m: np.ndarray        # row max of the logits
    Z: np.ndarray        # sum exp(l - m)
    p: np.ndarray        # probabilities [n, V]
    conf: np.ndarray     # max probability = 1 / Z
    entropy: np.ndarray  # nats
    argmax: np.ndarray   # lowest id among the maxima
    lse: np.ndarray      # m + ln Z


def vocab_softmax(l):
    """Per row: m = max l, Z = sum e^(l-m), p = e^(l-m)/Z, conf = 1/Z,
    H = ln Z - sum p (l - m), argmax = lowest id attaining m.

    24-ai.news, "Mechanism for deciding completed tokens": each position gets
    a confidence and an entropy.  The entropy is written in the form that can
    be accumulated over vocabulary tiles; it equals -sum p ln p.
    """
    l = np.asarray(l, F64)
    m = l.max(axis=1)
    e = np.exp(l - m[:, None])
    Z = e.sum(axis=1)
    p = e / Z[:, None]
    # an entry with p = 0 adds 0 (0 ln 0 = 0), also where its logit is -inf
    with np.errstate(invalid="ignore"):
        H = np.log(Z) - np.where(p > 0, p * (l - m[:, None]), 0.0).sum(axis=1)
    am = np.argmax(l, axis=1)          # numpy returns the first maximum
    return VocabStats(m=m, Z=Z, p=p, conf=1.0 / Z, entropy=H, argmax=am.astype(np.int64),
                      lse=m + np.log(Z))


# --------------------------------------------------------------------------
# S6  self-conditioning
# --------------------------------------------------------------------------
def self_condition(p, E):
    """sc_i = sum_v p_{i,v} E_v: the probability-weighted mean of the
    embedding rows over the full vocabulary.

    24-ai.news, "Mechanism for deciding completed tokens": the previous
    step's full softmax becomes a probability-weighted embedding average fed
    back as an extra input.
    """
    return np.asarray(p, F64) @ np.asarray(E, F64)


# --------------------------------------------------------------------------
# Whole denoise step (S0..S6) for one canvas, then for a batch
# --------------------------------------------------------------------------
def denoise_canvas(E, Wq, Wk, Wv, Wo, Kp, Vp, ids, dims, sc_in=None, lm_head=None,
                   logit_scale=1.0, row_scale=None, rows=None, need_sc=True,
                   need_logits=False, exclude_id=None, act_fp8=False):
    """One decoder-mode denoise step over one canvas (24-ai.news, "How is
    diffusion text generation different?": every canvas position is refined
    in parallel in one forward pass).

    ``rows`` restricts S2..S6 to those positions (S0/S1 keys and values are
    always computed for the whole canvas).  ``exclude_id`` removes one id from
    the vocabulary softmax (its logit becomes -inf): the multi-step loop
    removes the mask id.  ``act_fp8``: the LM head reads fp8_activations(h)
    (hidden_out stays h).  Returns a dict of float64 arrays.
    """
    x = embed_input(E, ids, sc_in)
    q, k, v = qkv_project(x, Wq, Wk, Wv, dims.n_q_heads, dims.n_kv_heads, dims.head_dim)
    C = x.shape[0]
    rows = np.arange(C) if rows is None else np.asarray(rows)
    o = window_attention(q, k, v, Kp, Vp, dims.window, rows)
    h = block_output(x[rows], o, Wo)
    s = logit_scale if row_scale is None else logit_scale * np.asarray(row_scale, F64)[rows]
    head = E if lm_head is None else lm_head
    l = lm_logits(fp8_activations(h) if act_fp8 else h, head, s)
    if exclude_id is not None:
        l[:, exclude_id] = -np.inf
    st = vocab_softmax(l)
    out = {"rows": rows, "x": x[rows], "attn_out": o.reshape(len(rows), -1),
           "hidden_out": h, "conf": st.conf, "entropy": st.entropy,
           "argmax": st.argmax, "m": st.m, "lse": st.lse}
    if need_logits:
        out["logits"] = l
    if need_sc:
        out["sc_out"] = self_condition(st.p, E)
    return out


def denoise_step(inp, sc_in=None, row_scale=None, rows=None, canvases=None,
                 need_sc=True, need_logits=False, act_fp8=False):
    """Run :func:`denoise_canvas` for each canvas of an input dict.

    Returns a list (one entry per canvas in ``canvases``).
    """
    dims = inp["dims"]
    cu = inp["cu_seqlens"]
    B = inp["batch"]
    canvases = range(B) if canvases is None else canvases
    res = []
    for b in canvases:
        p0, p1 = int(cu[b]), int(cu[b + 1])
        res.append(denoise_canvas(
            inp["embed"], inp["wq"], inp["wk"], inp["wv"], inp["wo"],
            inp["prompt_k"][p0:p1], inp["prompt_v"][p0:p1], inp["canvas_ids"][b], dims,
            sc_in=None if sc_in is None else sc_in[b], lm_head=inp.get("lm_head"),
            logit_scale=inp["logit_scale"],
            row_scale=None if row_scale is None else row_scale[b],
            rows=rows, need_sc=need_sc, need_logits=need_logits, act_fp8=act_fp8))
    return res


# --------------------------------------------------------------------------
# S7  entropy-bounded commit
# --------------------------------------------------------------------------
def commit_canvas(ids, conf, entropy, argmax, mask_id, tau):
    """Entropy-bounded commit of one canvas.

    24-ai.news, "Mechanism for deciding completed tokens": rank positions by
    confidence and accept from the most confident one until the cumulative
    entropy exceeds a preset threshold.  Reading: candidates are the masked
    positions; order is (confidence descending, position ascending); the
    candidate at rank k is accepted iff the sum of the entropies of ranks
    < k is <= tau (so the candidate that crosses tau is still accepted).
    Returns (commit_mask uint8 [C], out_ids int64 [C], n_committed).
    """
    ids = np.asarray(ids)
    C = len(ids)
    cand = [i for i in range(C) if ids[i] == mask_id]
    order = sorted(cand, key=lambda i: (-float(conf[i]), i))
    mask = np.zeros(C, dtype=np.uint8)
    out = ids.astype(np.int64).copy()
    prefix = 0.0
    for i in order:
        if prefix <= tau:
            mask[i] = 1
            out[i] = int(argmax[i])
        prefix += float(entropy[i])
    return mask, out, int(mask.sum())


def commit(ids, conf, entropy, argmax, mask_id, tau):
    """Batched :func:`commit_canvas` over [B, C] arrays."""
    B = ids.shape[0]
    masks, outs, ns = [], [], []
    for b in range(B):
        m, o, n = commit_canvas(ids[b], conf[b], entropy[b], argmax[b], mask_id, tau)
        masks.append(m)
        outs.append(o)
        ns.append(n)
    return np.stack(masks), np.stack(outs), np.array(ns, dtype=np.int64)


# --------------------------------------------------------------------------
# Multi-step loop: denoise, commit, self-conditioning feedback
# --------------------------------------------------------------------------
def denoise_loop(inp, tau, max_steps=None, row_scale=None, sc_in=None, tie_eps=None):
    """Repeat denoise step + commit on each canvas until it holds no mask id.

    24-ai.news, "How is diffusion text generation different?": the canvas is
    refined over several steps; "Mechanism for deciding completed tokens":
    each step commits the most confident positions until the cumulative
    entropy exceeds the threshold, and the self-conditioning vector of a step
    is an additional input of the next one.  Readings: step t of a canvas uses
    sc_in = sc_out of step t-1 (the given sc_in, or none, at t = 0); the mask
    id is removed from the vocabulary softmax of every loop step (committing
    the mask token would leave the position undecided, and with tied
    embeddings a masked position's own input makes the mask id its argmax, so
    the loop would stall); a canvas with no mask id left takes no more steps;
    at most max_steps steps (default: the canvas length, enough for any
    tau >= 0 since each step then commits at least one real token).

    With tie_eps, the first step at which the oracle itself declares a near-tie
    (commit_near_ties on the step's candidates, or argmax_near_ties on a
    position it commits) is recorded per canvas (-1: none): trajectories that
    differ only by rounding can part there.

    Returns ids [B, C] (final canvas), commit_step [B, C] (step at which each
    position was committed, -1 if never), steps [B], first_tie [B].
    """
    dims = inp["dims"]
    B, C, mask_id = inp["batch"], dims.canvas, dims.mask_id
    cu = inp["cu_seqlens"]
    max_steps = C if max_steps is None else max_steps
    ids = np.asarray(inp["canvas_ids"]).astype(np.int64).copy()
    commit_step = np.full((B, C), -1, dtype=np.int64)
    steps = np.zeros(B, dtype=np.int64)
    first_tie = np.full(B, -1, dtype=np.int64)
    for b in range(B):
        p0, p1 = int(cu[b]), int(cu[b + 1])
        sc = None if sc_in is None else sc_in[b]
        for t in range(max_steps):
            if not (ids[b] == mask_id).any():
                break
            st = denoise_canvas(
                inp["embed"], inp["wq"], inp["wk"], inp["wv"], inp["wo"],
                inp["prompt_k"][p0:p1], inp["prompt_v"][p0:p1], ids[b], dims, sc_in=sc,
                lm_head=inp.get("lm_head"), logit_scale=inp["logit_scale"],
                row_scale=None if row_scale is None else row_scale[b],
                need_sc=True, need_logits=tie_eps is not None, exclude_id=mask_id)
            mask, out, _ = commit_canvas(ids[b], st["conf"], st["entropy"], st["argmax"],
                                         mask_id, tau)
            if tie_eps is not None and first_tie[b] < 0:
                near = commit_near_ties(ids[b], st["conf"], st["entropy"], mask_id, tau, tie_eps)
                am = argmax_near_ties(st["logits"], tie_eps).mask
                if near.any() or (am & (mask == 1)).any():
                    first_tie[b] = t
            commit_step[b][mask == 1] = t
            ids[b] = out
            sc = st["sc_out"]
            steps[b] = t + 1
    return {"ids": ids, "commit_step": commit_step, "steps": steps, "first_tie": first_tie}


# --------------------------------------------------------------------------
# S8  structured slot read
# --------------------------------------------------------------------------
def label_read(l_row, lse, labels):
    """Read one slot from its full-vocabulary logit row.

    tau-home, "Refusing JSON token generation": the logprobs and the entropy
    of the allowed label ids are read at the slot.  lp_j = l[label_j] - lse;
    r = lp renormalised over the allowed labels; H = -sum r ln r (nats,
    0 ln 0 = 0); best = lowest index attaining max r.
    """
    lp = np.asarray(l_row, F64)[np.asarray(labels)] - lse
    mx = lp.max()
    w = np.exp(lp - mx)
    r = w / w.sum()
    return lp, r


def _entropy(r):
    r = np.asarray(r, F64)
    nz = r > 0
    return float(-(r[nz] * np.log(r[nz])).sum())


def slot_read_canvas(E, Wq, Wk, Wv, Wo, Kp, Vp, ids, dims, slot_pos, label_ids,
                     n_labels, noise_ids, logit_scale=1.0, row_scale=None,
                     entropy_threshold=0.1, n_draws=4, lm_head=None):
    """Structured read of every slot of one caller-seeded canvas.

    tau-home, "Refusing JSON token generation": one denoise forward on the
    prefilled canvas, never committing.  sotaaz, "The server takes at most 26
    alternatives": if the first read's entropy exceeds 0.1 the slot is read
    with 4 draws whose distributions are averaged; n_draws = 1 ("samples: 1")
    never re-reads.  Draw d writes noise_ids[d, s] at every slot s of the
    canvas (agentlenshq, "Technical architecture": random placeholder tokens)
    and reruns the step.  Averages: r = mean_d r_d, lp = ln mean_d e^(lp_d);
    entropy and best are recomputed from the averaged r.
    """
    C, V = dims.canvas, dims.vocab
    S = len(slot_pos)
    out = {
        "logprobs": np.zeros((S, MAX_LABELS)), "probs": np.zeros((S, MAX_LABELS)),
        "entropy": np.zeros(S), "first_entropy": np.zeros(S),
        "best": np.full(S, -1, dtype=np.int64), "draws_used": np.zeros(S, dtype=np.int64),
        "status": np.zeros(S, dtype=np.int64),
    }
    valid = np.ones(S, dtype=bool)
    for s in range(S):
        k = int(n_labels[s])
        if not (0 <= int(slot_pos[s]) < C):
            out["status"][s] = SLOT_BAD_POS
        elif not (1 <= k <= MAX_LABELS):
            out["status"][s] = SLOT_BAD_COUNT
        elif np.any((label_ids[s, :k] < 0) | (label_ids[s, :k] >= V)):
            out["status"][s] = SLOT_BAD_LABEL
        valid[s] = out["status"][s] == SLOT_OK
    vs = [s for s in range(S) if valid[s]]
    if not vs:
        return out
    head = E if lm_head is None else lm_head
    scale = np.full(S, float(logit_scale))
    if row_scale is not None:
        scale = scale * np.asarray(row_scale, F64)

    def read(canvas_ids):
        rows = np.array([int(slot_pos[s]) for s in vs])
        r = denoise_canvas(E, Wq, Wk, Wv, Wo, Kp, Vp, canvas_ids, dims, lm_head=lm_head,
                           logit_scale=1.0, rows=rows, need_sc=False, need_logits=True)
        res = {}
        for t, s in enumerate(vs):
            l_row = r["logits"][t] * scale[s]
            st = vocab_softmax(l_row[None, :])
            k = int(n_labels[s])
            res[s] = label_read(l_row, st.lse[0], label_ids[s, :k])
        return res

    first = read(np.asarray(ids))
    flagged = []
    for s in vs:
        lp, r = first[s]
        k = len(lp)
        H = _entropy(r)
        out["logprobs"][s, :k] = lp
        out["probs"][s, :k] = r
        out["entropy"][s] = H
        out["first_entropy"][s] = H
        out["best"][s] = int(np.argmax(r))
        out["draws_used"][s] = 1
        if n_draws > 1 and H > entropy_threshold:
            flagged.append(s)
    if flagged:
        acc_r = {s: 0.0 for s in flagged}
        acc_e = {s: 0.0 for s in flagged}
        for d in range(n_draws):
            cid = np.array(ids, copy=True)
            for s in range(S):
                if 0 <= int(slot_pos[s]) < C:
                    nid = int(noise_ids[d, s])
                    if not (0 <= nid < V):
                        nid = dims.mask_id
                        if out["status"][s] == SLOT_OK:
                            out["status"][s] = SLOT_BAD_NOISE
                    cid[int(slot_pos[s])] = nid
            rd = read(cid)
            for s in flagged:
                lp_d, r_d = rd[s]
                acc_r[s] = acc_r[s] + r_d
                acc_e[s] = acc_e[s] + np.exp(lp_d)
        for s in flagged:
            k = int(n_labels[s])
            r = acc_r[s] / n_draws
            out["probs"][s, :k] = r
            out["logprobs"][s, :k] = np.log(acc_e[s] / n_draws)
            out["entropy"][s] = _entropy(r)
            out["best"][s] = int(np.argmax(r))
            out["draws_used"][s] = n_draws
    return out


def slot_read(inp, row_scale=None, canvases=None, n_draws=None):
    """Batched :func:`slot_read_canvas` over an input dict; returns stacked arrays."""
    dims = inp["dims"]
    cu = inp["cu_seqlens"]
    B = inp["batch"]
    canvases = list(range(B)) if canvases is None else list(canvases)
    nd = inp["n_draws"] if n_draws is None else n_draws
    outs = []
    for b in canvases:
        p0, p1 = int(cu[b]), int(cu[b + 1])
        outs.append(slot_read_canvas(
            inp["embed"], inp["wq"], inp["wk"], inp["wv"], inp["wo"],
            inp["prompt_k"][p0:p1], inp["prompt_v"][p0:p1], inp["canvas_ids"][b], dims,
            inp["slot_pos"][b], inp["label_ids"][b], inp["n_labels"][b],
            inp["noise_ids"][:, b, :], logit_scale=inp["logit_scale"],
            row_scale=None if row_scale is None else row_scale[b],
            entropy_threshold=inp["entropy_threshold"], n_draws=nd,
            lm_head=inp.get("lm_head")))
    return {k: np.stack([o[k] for o in outs]) for k in outs[0]}


def slot_read_staged(inp, stage, ask_if_slot, ask_if_label, row_scale=None, n_draws=None):
    """Two-stage structured read of every canvas.

    sotaaz, "The server takes at most 26 alternatives": a question with ask_if
    is read only when the answer of an earlier question meets the condition,
    the entropy-triggered draws are taken per stage (two stages: up to 8
    reads), and the server writes the first answer back into the canvas before
    the second read.  Readings: stage[s] is 0 or 1; stage-0 slots are read
    first (their draws put noise at the stage-0 slots only; stage-1 slots keep
    the mask id); the best label of each stage-0 slot read without error is
    then pinned into the canvas at its position; stage-1 slots are read on that
    canvas (draws put noise at every stage-1 slot).  A stage-1 slot with
    ask_if_slot[s] = c >= 0 is asked only if slot c was read without error and
    its best label index equals ask_if_label[s]; otherwise its outputs are the
    zeros of a skipped slot with status SLOT_NOT_ASKED.  A slot not asked
    still holds the mask id and takes noise in the draws, but it is read with
    its first label only, so it never asks for draws itself.
    """
    dims = inp["dims"]
    cu = inp["cu_seqlens"]
    B = inp["batch"]
    nd = inp["n_draws"] if n_draws is None else n_draws
    stage = np.asarray(stage)
    ask_if_slot = np.asarray(ask_if_slot)
    ask_if_label = np.asarray(ask_if_label)
    S0 = np.nonzero(stage == 0)[0]
    S1 = np.nonzero(stage == 1)[0]
    outs = []
    for b in range(B):
        p0, p1 = int(cu[b]), int(cu[b + 1])
        args = (inp["embed"], inp["wq"], inp["wk"], inp["wv"], inp["wo"],
                inp["prompt_k"][p0:p1], inp["prompt_v"][p0:p1])
        kw = dict(logit_scale=inp["logit_scale"], entropy_threshold=inp["entropy_threshold"],
                  n_draws=nd, lm_head=inp.get("lm_head"))
        rs = None if row_scale is None else np.asarray(row_scale)[b]
        pos, labs, nlab = inp["slot_pos"][b], inp["label_ids"][b], inp["n_labels"][b]
        noise = inp["noise_ids"][:, b, :]
        S = len(pos)
        out = {"logprobs": np.zeros((S, MAX_LABELS)), "probs": np.zeros((S, MAX_LABELS)),
               "entropy": np.zeros(S), "first_entropy": np.zeros(S),
               "best": np.full(S, -1, dtype=np.int64), "draws_used": np.zeros(S, dtype=np.int64),
               "status": np.zeros(S, dtype=np.int64)}
        ids = np.asarray(inp["canvas_ids"][b]).copy()
        if len(S0):
            r0 = slot_read_canvas(*args, ids, dims, pos[S0], labs[S0], nlab[S0], noise[:, S0],
                                  row_scale=None if rs is None else rs[S0], **kw)
            for j, s in enumerate(S0):
                for k in out:
                    out[k][s] = r0[k][j]
            for j, s in enumerate(S0):
                if r0["status"][j] == SLOT_OK:
                    ids[int(pos[s])] = int(labs[s][int(r0["best"][j])])
        if len(S1):
            asked = np.array([ask_if_slot[s] < 0 or
                              (out["status"][ask_if_slot[s]] == SLOT_OK and
                               out["best"][ask_if_slot[s]] == ask_if_label[s]) for s in S1])
            n1 = np.where(asked, nlab[S1], 1)
            r1 = slot_read_canvas(*args, ids, dims, pos[S1], labs[S1], n1, noise[:, S1],
                                  row_scale=None if rs is None else rs[S1], **kw)
            for j, s in enumerate(S1):
                if asked[j]:
                    for k in out:
                        out[k][s] = r1[k][j]
                else:
                    out["status"][s] = SLOT_NOT_ASKED
        outs.append(out)
    return {k: np.stack([o[k] for o in outs]) for k in outs[0]}


# --------------------------------------------------------------------------
# Declared near-ties (decided from the oracle's own values, before any GPU run)
# --------------------------------------------------------------------------
@dataclass
class NearTies:
    mask: np.ndarray      # bool, True where the comparison is excused
    fraction: float


def argmax_near_ties(logits, eps):
    """Rows whose top-2 logit gap is below eps * max(1, |top1|)."""
    l = np.asarray(logits, F64)
    part = np.partition(l, -2, axis=1)
    top1, top2 = part[:, -1], part[:, -2]
    m = (top1 - top2) < eps * np.maximum(1.0, np.abs(top1))
    return NearTies(m, float(m.mean()) if m.size else 0.0)


def commit_near_ties(ids, conf, entropy, mask_id, tau, conf_eps, thr_eps=1e-3):
    """Positions of one canvas whose commit decision is within rounding reach.

    Excused (True) are:
    * candidates whose exclusive entropy prefix at their rank is within
      thr_eps of tau;
    * every member of the confidence cluster (a maximal run of two or more
      candidates, in rank order, whose neighbouring confidences differ by less
      than a relative conf_eps) that contains the last accepted rank.  Reordering
      inside any other cluster cannot change the accepted set: a cluster that
      ends two or more ranks before the boundary keeps every prefix at or
      below the prefix of the last accepted rank, and one that starts at or
      after the first rejected rank keeps every prefix above tau.
    """
    ids = np.asarray(ids)
    C = len(ids)
    cand = [i for i in range(C) if ids[i] == mask_id]
    order = sorted(cand, key=lambda i: (-float(conf[i]), i))
    near = np.zeros(C, dtype=bool)
    prefix = 0.0
    n_acc = 0
    for i in order:
        if abs(prefix - tau) < thr_eps:
            near[i] = True
        if prefix <= tau:
            n_acc += 1
        prefix += float(entropy[i])
    if n_acc == 0 or n_acc == len(order):
        return near
    # clusters in rank order
    cluster_id = np.zeros(len(order), dtype=np.int64)
    for r in range(1, len(order)):
        a, b = float(conf[order[r - 1]]), float(conf[order[r]])
        close = (a - b) < conf_eps * max(abs(a), abs(b))
        cluster_id[r] = cluster_id[r - 1] + (0 if close else 1)
    boundary = cluster_id[n_acc - 1]
    members = [i for r, i in enumerate(order) if cluster_id[r] == boundary]
    if len(members) > 1:          # a lone candidate cannot be reordered
        near[members] = True
    return near


def best_near_ties(probs, n_labels, eps):
    """Slots whose top-2 renormalised label probabilities differ by < eps."""
    pr = np.asarray(probs, F64)
    flat = pr.reshape(-1, pr.shape[-1])
    nl = np.asarray(n_labels).reshape(-1)
    out = np.zeros(flat.shape[0], dtype=bool)
    for i in range(flat.shape[0]):
        k = int(nl[i])
        if k >= 2:
            top = np.sort(flat[i, :k])[::-1]
            out[i] = (top[0] - top[1]) < eps
    return NearTies(out.reshape(pr.shape[:-1]), float(out.mean()) if out.size else 0.0)
