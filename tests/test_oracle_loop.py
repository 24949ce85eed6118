"""Pins of the multi-step loop oracle (denoise step + commit + self-conditioning
feedback until no mask id remains), CPU only.

The loop composes the pinned single-step functions; these tests pin what the
loop adds: step order, the removal of the mask id from the softmax, the
feedback of p.E, progress and termination.  Closed forms use a zero logit
scale, where every row is exactly uniform over the V - 1 remaining ids."""
import math

import numpy as np
import pytest
from scipy.special import softmax
from scipy.stats import entropy as sp_entropy

import oracle
from synth import config, make_inputs, companion_row_scale


def _inp(canvas, **kw):
    return make_inputs(config("tiny_f32", canvas=canvas, **kw))


def _ranks(ids, mask_id):
    """rank of each masked position in position order, -1 elsewhere"""
    r = np.full(len(ids), -1)
    pos = np.nonzero(ids == mask_id)[0]
    r[pos] = np.arange(len(pos))
    return r


def test_uniform_rows_commit_one_position_per_step():
    """logit scale 0: every row is uniform over V - 1 ids (H = ln(V-1) > tau),
    confidences tie, so each step commits the lowest masked position, with
    id 0 (the lowest id among the tied maxima)."""
    inp = _inp(20)
    inp["logit_scale"] = 0.0
    V, mask_id = inp["dims"].vocab, inp["dims"].mask_id
    ids0 = inp["canvas_ids"][0].copy()
    r = oracle.denoise_loop(inp, tau=1.0)
    n = int((ids0 == mask_id).sum())
    assert n >= 3 and 1.0 < math.log(V - 1)
    assert r["steps"][0] == n
    np.testing.assert_array_equal(r["commit_step"][0], _ranks(ids0, mask_id))
    want = ids0.copy()
    want[ids0 == mask_id] = 0
    np.testing.assert_array_equal(r["ids"][0], want)


def test_uniform_rows_commit_three_positions_per_step():
    """tau = 2.5 ln(V-1): exclusive prefixes 0, H, 2H are <= tau and 3H is not,
    so each step commits the three lowest masked positions."""
    inp = _inp(22)
    inp["logit_scale"] = 0.0
    V, mask_id = inp["dims"].vocab, inp["dims"].mask_id
    ids0 = inp["canvas_ids"][0].copy()
    r = oracle.denoise_loop(inp, tau=2.5 * math.log(V - 1))
    n = int((ids0 == mask_id).sum())
    assert r["steps"][0] == math.ceil(n / 3)
    rk = _ranks(ids0, mask_id)
    np.testing.assert_array_equal(r["commit_step"][0], np.where(rk >= 0, rk // 3, -1))


def test_mask_id_is_removed_from_the_softmax():
    """A loop step's distribution is the softmax of the logits with the mask
    column deleted (scipy), with p = 0 at the mask id; its entropy is scipy's."""
    inp = _inp(32)
    d, mask_id = inp["dims"], inp["dims"].mask_id
    rs = companion_row_scale(inp, (1, 32))[0]
    kw = dict(logit_scale=inp["logit_scale"], row_scale=rs, need_logits=True)
    args = (inp["embed"], inp["wq"], inp["wk"], inp["wv"], inp["wo"], inp["prompt_k"],
            inp["prompt_v"], inp["canvas_ids"][0], d)
    full = oracle.denoise_canvas(*args, **kw)
    ex = oracle.denoise_canvas(*args, exclude_id=mask_id, **kw)
    keep = np.arange(d.vocab) != mask_id
    p_ref = softmax(full["logits"][:, keep], axis=1)
    np.testing.assert_allclose(ex["entropy"], sp_entropy(p_ref, axis=1), rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(ex["conf"], p_ref.max(axis=1), rtol=1e-10)
    l = full["logits"].copy()
    l[:, mask_id] = -np.inf
    np.testing.assert_array_equal(ex["argmax"], np.argmax(l, axis=1))
    assert (ex["argmax"] != mask_id).all()
    # p.E without the mask row
    np.testing.assert_allclose(ex["sc_out"], p_ref @ inp["embed"][keep].astype(np.float64),
                               rtol=1e-9, atol=1e-12)


@pytest.mark.parametrize("tau", [0.0, 1.0, 6.0])
def test_loop_invariants_on_peaked_rows(tau):
    """Every masked position is committed exactly once, to a real token; each
    step commits at least one; unmasked positions never change; the loop ends
    within as many steps as there were masks."""
    inp = _inp(64)
    mask_id = inp["dims"].mask_id
    rs = companion_row_scale(inp, (1, 64))
    ids0 = inp["canvas_ids"][0].copy()
    r = oracle.denoise_loop(inp, tau=tau, row_scale=rs)
    masked = ids0 == mask_id
    steps = int(r["steps"][0])
    cs = r["commit_step"][0]
    assert 1 <= steps <= masked.sum()
    assert (cs[masked] >= 0).all() and (cs[masked] < steps).all() and (cs[~masked] == -1).all()
    assert (np.bincount(cs[masked], minlength=steps) >= 1).all()
    assert not (r["ids"][0] == mask_id).any()
    np.testing.assert_array_equal(r["ids"][0][~masked], ids0[~masked])


def test_second_step_reads_the_first_steps_self_conditioning():
    """Step 1 of the loop is the step on the committed canvas with sc_in = the
    first step's p.E: a manual two-step run gives the same commits, and the
    same run without the feedback does not."""
    inp = _inp(48)
    d, mask_id, tau = inp["dims"], inp["dims"].mask_id, 1.0
    rs = companion_row_scale(inp, (1, 48))[0]
    args = (inp["embed"], inp["wq"], inp["wk"], inp["wv"], inp["wo"], inp["prompt_k"],
            inp["prompt_v"])
    kw = dict(logit_scale=inp["logit_scale"], row_scale=rs, exclude_id=mask_id)
    ids = inp["canvas_ids"][0].copy()
    s0 = oracle.denoise_canvas(*args, ids, d, **kw)
    m0, ids1, _ = oracle.commit_canvas(ids, s0["conf"], s0["entropy"], s0["argmax"], mask_id, tau)
    s1 = oracle.denoise_canvas(*args, ids1, d, sc_in=s0["sc_out"], **kw)
    m1, ids2, _ = oracle.commit_canvas(ids1, s1["conf"], s1["entropy"], s1["argmax"], mask_id, tau)
    r = oracle.denoise_loop(inp, tau=tau, row_scale=rs[None], max_steps=2)
    np.testing.assert_array_equal(r["commit_step"][0] == 0, m0 == 1)
    np.testing.assert_array_equal(r["commit_step"][0] == 1, m1 == 1)
    np.testing.assert_array_equal(r["ids"][0], ids2)
    s1n = oracle.denoise_canvas(*args, ids1, d, **kw)   # no feedback
    assert np.abs(s1n["conf"] - s1["conf"]).max() > 1e-6


def test_infinite_threshold_commits_everything_in_one_step():
    inp = _inp(40)
    d, mask_id = inp["dims"], inp["dims"].mask_id
    r = oracle.denoise_loop(inp, tau=math.inf)
    ids0 = inp["canvas_ids"][0]
    st = oracle.denoise_canvas(inp["embed"], inp["wq"], inp["wk"], inp["wv"], inp["wo"],
                               inp["prompt_k"], inp["prompt_v"], ids0, d,
                               logit_scale=inp["logit_scale"], exclude_id=mask_id)
    assert r["steps"][0] == 1
    masked = ids0 == mask_id
    np.testing.assert_array_equal(r["ids"][0][masked], st["argmax"][masked])
