"""GPU parity of dg_slot_read against the CPU oracle, through the C-ABI."""
import numpy as np
import pytest

import oracle
from synth import config, make_inputs, companion_row_scale
from tests.helpers import TOL, TIE_EPS, to_np, assert_row_rel, assert_float

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def torch_cuda():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch


def _read(inp, row_scale=None, n_draws=None, **kw):
    """dg_slot_read (or, with full_canvas=True, dg_slot_read_full_canvas)."""
    import torch
    from slot_readout_amd.runtime import DeviceProblem
    dev = DeviceProblem(inp, with_embed_t=False)
    rs = None if row_scale is None else torch.from_numpy(row_scale).cuda()
    out = dev.slot_read(row_scale=rs, n_draws=n_draws, **kw)
    torch.cuda.synchronize()
    return {k: to_np(v) for k, v in out.items()}


def _check_slots(g, ref, inp, dtype, label="", max_excused=None):
    """Every slot output against the oracle's; with max_excused, the fraction
    of slots whose best label is excused as a declared near-tie must stay
    below it (companion inputs, where the decisions are meant to be real)."""
    tol = TOL[dtype]
    assert np.array_equal(g["status"], ref["status"]), f"{label} status"
    th = inp["entropy_threshold"]
    # a first entropy within the entropy bar of the threshold may decide the re-read
    # either way: such slots are excused (declared from the oracle's values)
    near = np.abs(ref["first_entropy"] - th) < tol["entropy_abs"]
    ok = (ref["status"] == oracle.SLOT_OK) & ~near
    assert np.array_equal(g["draws_used"][ok], ref["draws_used"][ok]), f"{label} draws_used"
    assert_float(g["first_entropy"][ok], ref["first_entropy"][ok], dtype, "entropy", f"{label} first_entropy")
    assert_float(g["entropy"][ok], ref["entropy"][ok], dtype, "entropy", f"{label} entropy")
    nl = inp["n_labels"]
    for b, s in zip(*np.nonzero(ok)):
        k = nl[b, s]
        assert_float(g["logprobs"][b, s, :k], ref["logprobs"][b, s, :k], dtype, "logprob",
                     f"{label} logprobs[{b},{s}]")
        assert_row_rel(g["probs"][b, s, :k][None], ref["probs"][b, s, :k][None], tol["probs"],
                       f"{label} probs[{b},{s}]")
        assert np.all(g["probs"][b, s, k:] == 0) and np.all(g["logprobs"][b, s, k:] == 0)
        assert abs(g["probs"][b, s, :k].sum() - 1) < 1e-5
    bnt = oracle.best_near_ties(ref["probs"], nl, TIE_EPS[dtype])
    bnear = bnt.mask
    if max_excused is not None:
        assert bnt.fraction < max_excused, f"{label}: {bnt.fraction:.2f} of best labels excused"
    okb = ok & ~bnear
    assert np.array_equal(g["best"][okb], ref["best"][okb]), f"{label} best"
    bad = ref["status"] != oracle.SLOT_OK
    bad &= ref["status"] != oracle.SLOT_BAD_NOISE
    assert np.all(g["best"][bad] == -1) and np.all(g["draws_used"][bad] == 0)
    return ok.mean()


def test_slot_read_tiny_f32(torch_cuda):
    """8 slots x 4 labels, first read + 4 averaged noise draws (flat rows re-read)."""
    inp = make_inputs(config("tiny_f32"))
    g = _read(inp)
    ref = oracle.slot_read(inp)
    assert (ref["draws_used"] == 4).all()           # flat literal rows: H ~ ln 4 > 0.1
    _check_slots(g, ref, inp, "f32", "tiny_f32")


def test_slot_read_tiny_f32_companion(torch_cuda):
    """Per-slot logit multipliers: some slots are peaked (single read), some re-read."""
    inp = make_inputs(config("tiny_f32"))
    rs = companion_row_scale(inp, (1, 8), 64.0, 4096.0)
    g = _read(inp, row_scale=rs)
    ref = oracle.slot_read(inp, row_scale=rs)
    _check_slots(g, ref, inp, "f32", "tiny_f32 companion", max_excused=0.5)
    assert (ref["draws_used"] == 1).any() and (ref["draws_used"] == 4).any()


def test_slot_read_single_draw_is_first_read(torch_cuda):
    """n_draws = 1 ('samples: 1') never re-reads and equals the first read."""
    inp = make_inputs(config("tiny_f32"))
    g1 = _read(inp, n_draws=1)
    g4 = _read(inp)
    ref = oracle.slot_read(inp, n_draws=1)
    _check_slots(g1, ref, inp, "f32", "samples:1")
    assert (g1["draws_used"] == 1).all()
    assert np.array_equal(g1["first_entropy"], g4["first_entropy"])


def test_slot_read_bad_inputs_report_status(torch_cuda):
    """Out-of-range slot positions, label counts, label ids and noise ids are reported
    per slot and never read out of bounds; the other slots are unaffected."""
    inp = make_inputs(config("tiny_f32"))
    V, C = inp["dims"].vocab, inp["dims"].canvas
    inp["slot_pos"][0, 1] = C + 5
    inp["n_labels"][0, 2] = 0
    inp["n_labels"][0, 3] = 27
    inp["label_ids"][0, 4, 1] = V
    inp["noise_ids"][2, 0, 5] = -3
    g = _read(inp)
    ref = oracle.slot_read(inp)
    assert list(ref["status"][0][:6]) == [0, 1, 2, 2, 3, 4]
    _check_slots(g, ref, inp, "f32", "bad inputs")


@pytest.mark.parametrize("B,P", [(6, 64), (3, 0)])
def test_slot_read_skeleton_bf16(torch_cuda, B, P):
    """Structured-read batch in bf16: one shared skeleton, 4 slots, k ~ U{2..26}."""
    inp = make_inputs(config("reads512"), batch=B, prompt_override=("fixed", P))
    g = _read(inp)
    ref = oracle.slot_read(inp)
    _check_slots(g, ref, inp, "bf16", f"skeleton B{B} P{P}")


def test_slot_read_wide_heads_small_vocab(torch_cuda):
    """512-wide GQA heads (d 2816) with a 4096-entry vocabulary."""
    cfg = config("bf16_step", vocab=4096, mask_id=4095)
    inp = make_inputs(cfg, prompt_override=("fixed", 200))
    g = _read(inp)
    ref = oracle.slot_read(inp)
    _check_slots(g, ref, inp, "bf16", "wide heads")


def test_slot_read_deterministic(torch_cuda):
    inp = make_inputs(config("reads512"), batch=4, prompt_override=("fixed", 100))
    a = _read(inp)
    b = _read(inp)
    for k in a:
        assert np.array_equal(a[k], b[k]), k



def _one_pass_draws(dims, B, S, nd, max_prompt):
    """The library's rule for computing the draws in the first read's pass:
    the LM-head weight stream (V x d at ~5 TB/s) outweighs the draws' forward
    pass (~1 PFLOP/s bf16, ~0.1 fp32): q/k/v of every canvas row, attention of
    the slot rows (rounded up to a query tile) over prompt + canvas, and the
    output projection of the slot rows."""
    ts = 2 if dims.dtype == "bf16" else 4
    head_s = dims.vocab * dims.d_model * ts / 5e12
    hq, hkv = dims.n_q_heads * dims.head_dim, dims.n_kv_heads * dims.head_dim
    if dims.dtype == "bf16" and dims.head_dim == 64 and S <= 1024:
        # patched draws: their slot rows' projections and attention, against the
        # LM-head stream plus a second stream of the prompts' k, v
        per_draw = (2 * dims.d_model * (hq + 2 * hkv) * S + 2 * hq * dims.d_model * S
                    + 4 * hq * (max_prompt + dims.canvas) * S)
        draw_s = B * nd * per_draw / 1e15
        kv_s = B * max_prompt * 2 * hkv * ts / 5e12
        return nd > 1 and draw_s < head_s + kv_s
    qt = 64 if dims.head_dim == 512 else 128
    s_att = -(-S // qt) * qt
    per_canvas = (2 * dims.d_model * (hq + 2 * hkv) * dims.canvas + 2 * hq * dims.d_model * S
                  + 4 * hq * (max_prompt + dims.canvas) * s_att)
    draw_s = B * nd * per_canvas / (1e15 if dims.dtype == "bf16" else 1e14)
    return nd > 1 and draw_s < head_s


def test_slot_read_one_pass_draws_f32(torch_cuda):
    """A 262,144-token vocabulary makes the draws ride in the first read's pass:
    fp32, 2 canvases x 4 slots with per-slot multipliers, so some slots stop at
    the first read and some average their draws (checked at the fp32 bar)."""
    inp = make_inputs(config("reads512", dtype="f32", vocab=262144, mask_id=262143), batch=2,
                      prompt_override=("fixed", 64))
    assert _one_pass_draws(inp["dims"], 2, inp["slot_pos"].shape[1], inp["n_draws"],
                           int(inp["max_prompt"]))
    rs = companion_row_scale(inp, (2, 4), 64.0, 2048.0)
    g = _read(inp, row_scale=rs)
    ref = oracle.slot_read(inp, row_scale=rs)
    _check_slots(g, ref, inp, "f32", "one-pass draws f32", max_excused=0.5)
    du = ref["draws_used"]
    assert (du == 1).any() and (du == 4).any()


def test_slot_read_one_pass_draws_bf16(torch_cuda):
    """Read-batch shape (1024-token prompts, k ~ U{2..26}) with a 262,144-token
    vocabulary, 8 canvases: draws computed in the first read's pass, bf16."""
    inp = make_inputs(config("reads512", vocab=262144, mask_id=262143), batch=8)
    assert _one_pass_draws(inp["dims"], 8, inp["slot_pos"].shape[1], inp["n_draws"],
                           int(inp["max_prompt"]))
    g = _read(inp)
    ref = oracle.slot_read(inp)
    _check_slots(g, ref, inp, "bf16", "one-pass draws bf16")


@pytest.mark.parametrize("window,n_slots", [(0, 4), (5, 4), (255, 4), (400, 4), (5, 40), (0, 120)])
def test_slot_read_one_pass_window_rows(torch_cuda, window, n_slots):
    """One-pass patched draws project and attend only the base rows within +-W
    of one of the canvas's slots, listed per canvas on the device: W = 0 (the
    slot positions alone), a small window, W = C - 1 and W > C (every row), and
    40 or 120 slots per canvas.  Three canvases with different slot sets (a slot
    out of range, two slots at one position, slots at both canvas ends), so the
    canvases' lists differ in length, against the oracle."""
    inp = make_inputs(config("reads512", vocab=262144, mask_id=262143, window=window, n_slots=n_slots),
                      batch=3, prompt_override=("fixed", 96))
    dims = inp["dims"]
    C = dims.canvas
    sp = inp["slot_pos"]
    assert sp.shape[1] == n_slots
    if n_slots == 4:
        sp[0] = [10, 200, C + 5, 11]
        sp[1] = [50, 50, 120, 121]
        sp[2] = [0, 1, C - 2, C - 1]
    else:
        sp[0, 2] = C + 5
        sp[1, 1] = sp[1, 0]
        sp[2, 0], sp[2, -1] = 0, C - 1
    for b in range(3):
        for p in sp[b]:
            if 0 <= p < C:
                inp["canvas_ids"][b, p] = dims.mask_id
    assert _one_pass_draws(dims, 3, n_slots, inp["n_draws"], int(inp["max_prompt"]))
    ref = oracle.slot_read(inp)
    assert ref["status"][0, 2] == oracle.SLOT_BAD_POS
    g = _read(inp)
    _check_slots(g, ref, inp, "bf16", f"one-pass window rows W={window} S={n_slots}")


@pytest.mark.parametrize("name,B", [("reads512", 52), ("tiny_f32", 34)])
def test_slot_read_label_logits_of_many_rows(torch_cuda, name, B):
    """A read whose LM head has 1,024 rows or more takes its label logits from
    a dot product per (row, label) instead of the vocabulary tiles: 52
    read-batch canvases in one pass (1,040 rows, bf16 split rows, up to 26
    labels), and 34 tiny fp32 canvases whose draws all run in a second pass
    (1,088 rows), against the oracle."""
    inp = make_inputs(config(name), batch=B, prompt_override=("fixed", 64) if name == "reads512" else None)
    S = inp["slot_pos"].shape[1]
    ref = oracle.slot_read(inp)
    flagged = int((ref["draws_used"] > 1).any(axis=1).sum())
    rows = B * (1 + inp["n_draws"]) * S if name == "reads512" else flagged * inp["n_draws"] * S
    assert rows >= 1024
    g = _read(inp)
    _check_slots(g, ref, inp, inp["dims"].dtype, f"label logits of many rows {name}")


def test_slot_read_many_slots_two_pass(torch_cuda):
    """150 slots on one canvas: more slot rows than one gathered query tile holds
    (128 at head_dim 64), and the 22 slots past the 128 masked positions all sit
    at position 0 (duplicates), read by the two-pass order."""
    inp = make_inputs(config("tiny_f32", n_slots=150))
    assert (inp["slot_pos"][0] == 0).sum() > 1
    g = _read(inp)
    ref = oracle.slot_read(inp)
    _check_slots(g, ref, inp, "f32", "many slots")


def test_slot_read_many_slots_one_pass(torch_cuda):
    """130 slots of a 65,536-entry vocabulary, fp32, read in one pass with the
    draws: two gathered query tiles per head, the k/v copy into the draw
    canvases, a duplicated slot position and an out-of-range one."""
    inp = make_inputs(config("reads512", dtype="f32", vocab=65536, mask_id=65535, n_slots=130),
                      batch=1, prompt_override=("fixed", 64))
    C = inp["dims"].canvas
    inp["slot_pos"][0, 5] = inp["slot_pos"][0, 3]
    inp["slot_pos"][0, 7] = C + 3
    assert _one_pass_draws(inp["dims"], 1, inp["slot_pos"].shape[1], inp["n_draws"],
                           int(inp["max_prompt"]))
    rs = companion_row_scale(inp, (1, 130), 64.0, 2048.0)
    g = _read(inp, row_scale=rs)
    ref = oracle.slot_read(inp, row_scale=rs)
    assert ref["status"][0, 7] == oracle.SLOT_BAD_POS
    _check_slots(g, ref, inp, "f32", "many slots one pass", max_excused=0.5)


def test_slot_read_wide_heads_mixed_rereads(torch_cuda):
    """Three canvases at d 2816 with 512-wide heads, read in two passes, where
    only canvas 0 re-reads: its slots offer 26 labels (first-read entropy near
    ln 26) and the others' offer 2 (near ln 2), with the threshold between.  The
    draw pass then projects 3 x n_draws x 8 slot rows, so its q and output
    projections split K, and the per-canvas draw flags skip the rows of the
    canvases that do not re-read in both the split GEMMs and their reduces."""
    cfg = config("bf16_step", vocab=4096, mask_id=4095)
    inp = make_inputs(cfg, batch=3, prompt_override=("fixed", 200))
    S = inp["slot_pos"].shape[1]
    assert not _one_pass_draws(inp["dims"], 3, S, inp["n_draws"], int(inp["max_prompt"]))
    rng = np.random.default_rng(11)
    lab = np.full_like(inp["label_ids"], -1)
    for s in range(S):
        lab[0, s] = rng.choice(4095, size=26, replace=False)
    lab[1:, :, :2] = inp["label_ids"][1:, :, :2]
    nl = np.full_like(inp["n_labels"], 2)
    nl[0] = 26
    inp["label_ids"], inp["n_labels"] = lab, nl
    inp["entropy_threshold"] = 2.0
    ref = oracle.slot_read(inp)
    ok = ref["status"] == oracle.SLOT_OK
    assert ok.all()
    fe = ref["first_entropy"]
    assert fe[0].min() > 2.5 and fe[1:].max() < 1.0, fe
    assert (ref["draws_used"][0] == inp["n_draws"]).all() and (ref["draws_used"][1:] == 1).all()
    g = _read(inp)
    _check_slots(g, ref, inp, "bf16", "wide heads mixed re-reads")


@pytest.mark.parametrize("name,n_kv,n_slots,batch", [
    ("tiny_f32", 1, 8, 1),      # 4 q heads x 8 slot rows = 32 columns of one query tile
    ("tiny_f32", 1, 30, 1),     # 120 columns: both 16-column blocks of every wave
    ("tiny_f32", 1, 40, 1),     # 160 columns: too many to pack, one tile per q head
    ("reads512", 2, 4, 16),     # bf16, 2 q heads per kv head
])
def test_slot_read_gqa_packed_heads(torch_cuda, name, n_kv, n_slots, batch):
    """Gathered slot queries with grouped kv heads at head_dim 64: when the q heads
    of a kv head fit one query tile together, one workgroup serves them all
    (column c is head c / rows, row c % rows); otherwise each q head has its own."""
    inp = make_inputs(config(name, n_kv_heads=n_kv, n_slots=n_slots), batch=batch,
                      prompt_override=("fixed", 100))
    dt = inp["dims"].dtype
    g = _read(inp)
    ref = oracle.slot_read(inp)
    frac = _check_slots(g, ref, inp, dt, f"gqa {name} kv{n_kv} S{n_slots}")
    assert frac > 0.5


@pytest.mark.parametrize("n_q,n_slots", [(4, 4), (8, 2)])
def test_slot_read_patched_four_kv_heads(torch_cuda, n_q, n_slots):
    """One-pass patched reads with four kv heads whose queries fit a quarter of
    a tile each, which one workgroup serves together (each wave on one kv
    head's slice of the staged rows): 4 q heads x 4 slots (MHA) and 8 q heads x
    2 slots (two q heads per kv head), 16 canvases, against the oracle."""
    inp = make_inputs(config("reads512", n_q_heads=n_q, n_kv_heads=4, n_slots=n_slots), batch=16,
                      prompt_override=("fixed", 100))
    dims = inp["dims"]
    assert _one_pass_draws(dims, 16, n_slots, inp["n_draws"], int(inp["max_prompt"]))
    assert (n_q // 4) * (1 + inp["n_draws"]) * n_slots <= 32
    g = _read(inp)
    ref = oracle.slot_read(inp)
    _check_slots(g, ref, inp, "bf16", f"patched four kv heads q{n_q} S{n_slots}")


def test_slot_read_wide_heads_peaked_rereads(torch_cuda):
    """Three canvases at d 2816 with 512-wide heads, read in two passes, with
    per-canvas logit multipliers 1, 24 and 64: flat rows and sharp ones whose
    label logprobs reach about -90.  The entropy threshold sits in the widest
    gap between the canvases' largest first-read entropies, so some canvases
    re-read and some do not.  bf16 storage at the absolute 1e-2 logprob bar:
    the slot rows carry the attention probabilities, its output and the
    hidden state as bf16 hi + lo pairs, so only the rounding of the stored
    q, k, v remains."""
    cfg = config("bf16_step", vocab=4096, mask_id=4095)
    inp = make_inputs(cfg, batch=3, prompt_override=("fixed", 200))
    S = inp["slot_pos"].shape[1]
    assert not _one_pass_draws(inp["dims"], 3, S, inp["n_draws"], int(inp["max_prompt"]))
    rs = np.repeat(np.asarray([1.0, 24.0, 64.0], np.float32)[:, None], S, axis=1)
    inp["entropy_threshold"] = 1e9                # first reads only
    r0 = oracle.slot_read(inp, row_scale=rs)
    first, ok = r0["first_entropy"], r0["status"] == oracle.SLOT_OK
    top = np.sort(np.where(ok, first, -np.inf).max(axis=1))
    gaps = np.diff(top)
    i = int(np.argmax(gaps))
    assert gaps[i] > 4 * TOL["bf16"]["entropy_abs"], top
    inp["entropy_threshold"] = float((top[i] + top[i + 1]) / 2)
    ref = oracle.slot_read(inp, row_scale=rs)
    reread = (ref["draws_used"] > 1).any(axis=1)
    assert reread.any() and not reread.all(), ref["draws_used"]
    assert ref["logprobs"][2][:, :4].min() < -80          # sharp rows: large |logprob|
    g = _read(inp, row_scale=rs)
    _check_slots(g, ref, inp, "bf16", "wide heads peaked re-reads")


@pytest.mark.parametrize("lo,hi", [(16.0, 512.0), (256.0, 1024.0)])
def test_slot_read_skeleton_bf16_companion(torch_cuda, lo, hi):
    """Read-batch dims in bf16 with per-slot logit multipliers up to 1024x
    (label logprobs down to about -100): confident single reads and averaged
    re-reads, at the absolute 1e-2 logprob bar."""
    import torch
    inp = make_inputs(config("reads512"), batch=32, prompt_override=("fixed", 300))
    rs = companion_row_scale(inp, (32, 4), lo, hi)
    g = _read(inp, row_scale=rs)
    ref = oracle.slot_read(inp, row_scale=rs)
    _check_slots(g, ref, inp, "bf16", f"skeleton bf16 companion {lo}-{hi}", max_excused=0.5)
    du = ref["draws_used"]
    assert (du == 1).any() and (du == 4).any()


@pytest.mark.parametrize("name,over,B,prompt,scales", [
    ("tiny_f32", {}, 1, ("fixed", 128), (64.0, 4096.0)),                 # fp32, two passes
    ("reads512", {}, 6, ("fixed", 200), (16.0, 512.0)),                  # bf16, two passes
    ("reads512", dict(vocab=262144, mask_id=262143), 2, ("fixed", 64), (16.0, 512.0)),  # one pass
    ("bf16_step", dict(vocab=4096, mask_id=4095), 2, ("fixed", 150), (8.0, 128.0)),    # hd 512
])
def test_slot_read_full_canvas(torch_cuda, name, over, B, prompt, scales):
    """The whole-canvas order (q, attention and the output projection over every
    canvas row, LM head at the slot rows) against the oracle, and against the
    slot-row order up to summation order."""
    inp = make_inputs(config(name, **over), batch=B, prompt_override=prompt)
    dt = inp["dims"].dtype
    rs = companion_row_scale(inp, inp["slot_pos"].shape, *scales)
    g = _read(inp, row_scale=rs, full_canvas=True)
    ref = oracle.slot_read(inp, row_scale=rs)
    _check_slots(g, ref, inp, dt, f"full canvas {name}", max_excused=0.5)
    g2 = _read(inp, row_scale=rs)
    ok = (ref["status"] == oracle.SLOT_OK) & (g["draws_used"] == g2["draws_used"])
    tol = 2e-4 if dt == "f32" else 1e-2
    assert np.abs(g["logprobs"][ok] - g2["logprobs"][ok]).max() <= tol


@pytest.mark.parametrize("name", ["tiny_f32", "reads512"])
def test_slot_read_draws_share_a_tile_at_canvas_edges(torch_cuda, name):
    """The draws of a canvas read its prompt in one tile (their gathered
    queries side by side, each draw's own canvas keys behind the prompt's):
    slots at positions 0, 1, C-2 and C-1, where a window that crossed into the
    neighbouring draw's keys would show, against the oracle."""
    inp = make_inputs(config(name, n_slots=4), batch=3, prompt_override=("fixed", 90))
    C = inp["dims"].canvas
    for b in range(3):
        inp["slot_pos"][b] = [0, 1, C - 2, C - 1]
        inp["canvas_ids"][b, [0, 1, C - 2, C - 1]] = inp["dims"].mask_id
    ref = oracle.slot_read(inp)
    assert (ref["draws_used"] == inp["n_draws"]).any()
    g = _read(inp)
    _check_slots(g, ref, inp, inp["dims"].dtype, f"draw tile edges {name}")


def test_slot_read_patched_draws_two_pass(torch_cuda):
    """Read-batch dims in bf16 with 150 slots per canvas and a 64-token prompt:
    the draws' slot rows outweigh a second pass, so the two-pass order runs with
    patched draws (the draws read their base canvas's k, v with their own slot
    rows in place), two gathered query tiles per canvas, against the oracle."""
    inp = make_inputs(config("reads512", n_slots=150), batch=2, prompt_override=("fixed", 64))
    S = inp["slot_pos"].shape[1]
    assert not _one_pass_draws(inp["dims"], 2, S, inp["n_draws"], int(inp["max_prompt"]))
    rs = companion_row_scale(inp, (2, S), 4.0, 256.0)
    g = _read(inp, row_scale=rs)
    ref = oracle.slot_read(inp, row_scale=rs)
    _check_slots(g, ref, inp, "bf16", "patched draws two-pass", max_excused=0.5)
    du = ref["draws_used"]
    assert (du == 1).any() and (du == inp["n_draws"]).any()
