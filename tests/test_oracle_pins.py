"""Pins of the CPU oracle against facts that do not come from the oracle itself:
closed forms, library routines on special cases, invariants, brute force on
tiny inputs and hand-worked fixtures.  Each test is chosen so that a plausible
slip (a dropped term, a wrong sign or index, a transposed operand) fails it.
"""
import itertools
import json
import math
import os

import numpy as np
import pytest
import scipy.special
import scipy.stats
import torch

import oracle
from oracle import dg_oracle as O
from synth import Dims

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
rng = np.random.default_rng(1234)


# ---------------------------------------------------------------- S0 ------
def test_embed_gather_is_row_lookup():
    V, d = 7, 5
    # E[v, j] = 100 v + j: every entry names its own row and column
    E = 100.0 * np.arange(V)[:, None] + np.arange(d)[None, :]
    ids = np.array([3, 0, 6, 3])
    x = O.embed_input(E, ids)
    for i, v in enumerate(ids):
        assert list(x[i]) == [100.0 * v + j for j in range(d)]
    sc = np.full((4, d), 0.5)
    x2 = O.embed_input(E, ids, sc)
    assert np.all(x2 - x == 0.5)


def test_embed_out_of_range_ids_are_zero_rows():
    # ids outside [0, V) (a negative id would otherwise wrap to a real row)
    V, d = 7, 5
    E = 100.0 * np.arange(V)[:, None] + np.arange(d)[None, :] + 1.0
    x = O.embed_input(E, np.array([2, -1, 7, 6]))
    assert np.array_equal(x[0], E[2]) and np.array_equal(x[3], E[6])
    assert not x[1].any() and not x[2].any()


# ---------------------------------------------------------------- S1/S3 ---
def test_qkv_projection_selection_matrices():
    # W is [out, in]; a rectangular selection matrix picks input coordinates,
    # so using W instead of W^T cannot even produce the right shape.
    n, d, H, hd = 3, 6, 2, 2
    x = rng.standard_normal((n, d))
    sel = [5, 0, 3, 1]
    W = np.zeros((H * hd, d))
    for o, i in enumerate(sel):
        W[o, i] = 1.0
    q, k, v = O.qkv_project(x, W, 2 * W, -W, H, H, hd)
    assert q.shape == (n, H, hd)
    assert np.array_equal(q.reshape(n, -1), x[:, sel])
    assert np.array_equal(k.reshape(n, -1), 2 * x[:, sel])
    assert np.array_equal(v.reshape(n, -1), -x[:, sel])
    # head h holds output columns h*hd .. h*hd+hd-1
    assert np.array_equal(q[:, 1, :], x[:, sel[2:4]])


def test_block_output_residual():
    n, d, hq = 4, 3, 6
    x = rng.standard_normal((n, d))
    o = rng.standard_normal((n, 2, 3))
    assert np.array_equal(O.block_output(x, o, np.zeros((d, hq))), x)
    Wo = np.zeros((d, hq))
    Wo[0, 4] = 1.0   # h[:,0] += o_flat[:,4]
    Wo[2, 1] = -2.0  # h[:,2] -= 2 o_flat[:,1]
    h = O.block_output(x, o, Wo)
    of = o.reshape(n, -1)
    assert np.allclose(h[:, 0], x[:, 0] + of[:, 4])
    assert np.allclose(h[:, 1], x[:, 1])
    assert np.allclose(h[:, 2], x[:, 2] - 2 * of[:, 1])


# ---------------------------------------------------------------- S2 ------
def _sdpa(q, K, V, mask=None):
    """torch CPU float64 scaled_dot_product_attention for one head."""
    qt = torch.from_numpy(q)[None, None]
    kt = torch.from_numpy(K)[None, None]
    vt = torch.from_numpy(V)[None, None]
    m = None if mask is None else torch.from_numpy(mask)[None, None]
    return torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, attn_mask=m)[0, 0].numpy()


@pytest.mark.parametrize("P,C,Hq,Hkv,hd,W", [(5, 9, 2, 2, 8, 8), (0, 7, 4, 2, 4, 6),
                                            (11, 12, 4, 1, 8, 40)])
def test_attention_full_window_equals_sdpa(P, C, Hq, Hkv, hd, W):
    """W >= C-1: every canvas key is visible, so the step is plain SDPA over
    [prompt; canvas] keys (agentlenshq: every token of the block sees every other)."""
    q = rng.standard_normal((C, Hq, hd))
    k = rng.standard_normal((C, Hkv, hd))
    v = rng.standard_normal((C, Hkv, hd))
    Kp = rng.standard_normal((P, Hkv, hd))
    Vp = rng.standard_normal((P, Hkv, hd))
    o = O.window_attention(q, k, v, Kp, Vp, W)
    G = Hq // Hkv
    for h in range(Hq):
        g = h // G
        ref = _sdpa(q[:, h], np.concatenate([Kp[:, g], k[:, g]]), np.concatenate([Vp[:, g], v[:, g]]))
        assert np.allclose(o[:, h], ref, rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("W", [0, 1, 3, 5])
def test_attention_window_equals_masked_sdpa(W):
    P, C, H, hd = 6, 13, 2, 8
    q = rng.standard_normal((C, H, hd))
    k = rng.standard_normal((C, H, hd))
    v = rng.standard_normal((C, H, hd))
    Kp = rng.standard_normal((P, H, hd))
    Vp = rng.standard_normal((P, H, hd))
    o = O.window_attention(q, k, v, Kp, Vp, W)
    i = np.arange(C)[:, None]
    j = np.arange(C)[None, :]
    mask = np.concatenate([np.ones((C, P), bool), np.abs(i - j) <= W], axis=1)
    for h in range(H):
        ref = _sdpa(q[:, h], np.concatenate([Kp[:, h], k[:, h]]),
                    np.concatenate([Vp[:, h], v[:, h]]), mask)
        assert np.allclose(o[:, h], ref, rtol=1e-12, atol=1e-12)


def test_attention_gqa_equals_repeated_mha():
    P, C, Hq, Hkv, hd, W = 4, 10, 6, 2, 4, 2
    q = rng.standard_normal((C, Hq, hd))
    k = rng.standard_normal((C, Hkv, hd))
    v = rng.standard_normal((C, Hkv, hd))
    Kp = rng.standard_normal((P, Hkv, hd))
    Vp = rng.standard_normal((P, Hkv, hd))
    G = Hq // Hkv
    o = O.window_attention(q, k, v, Kp, Vp, W)
    o2 = O.window_attention(q, np.repeat(k, G, axis=1), np.repeat(v, G, axis=1),
                            np.repeat(Kp, G, axis=1), np.repeat(Vp, G, axis=1), W)
    assert np.allclose(o, o2, rtol=1e-13, atol=1e-13)


def test_attention_closed_forms():
    C, H, hd = 9, 2, 4
    q = rng.standard_normal((C, H, hd))
    k = rng.standard_normal((C, H, hd))
    v = rng.standard_normal((C, H, hd))
    empty = np.zeros((0, H, hd))
    # no prompt and W = 0: each query sees only itself
    assert np.allclose(O.window_attention(q, k, v, empty, empty, 0), v)
    # all keys equal: uniform weights, output = mean of the visible values
    kc = np.ones((C, H, hd))
    Kp = np.ones((3, H, hd))
    Vp = rng.standard_normal((3, H, hd))
    o = O.window_attention(q, kc, v, Kp, Vp, 1)
    for i in range(C):
        vis = [Vp[t] for t in range(3)] + [v[j] for j in range(C) if abs(i - j) <= 1]
        assert np.allclose(o[i], np.mean(vis, axis=0))


def test_attention_row_subset_matches_full():
    C, H, hd = 12, 2, 4
    q, k, v = (rng.standard_normal((C, H, hd)) for _ in range(3))
    Kp, Vp = (rng.standard_normal((5, H, hd)) for _ in range(2))
    full = O.window_attention(q, k, v, Kp, Vp, 3)
    rows = [0, 7, 11]
    assert np.allclose(O.window_attention(q, k, v, Kp, Vp, 3, rows), full[rows])


# ---------------------------------------------------------------- S4 ------
def test_lm_logits_identity_head_and_row_scale():
    n, d, V = 3, 4, 6
    h = rng.standard_normal((n, d))
    head = np.zeros((V, d))
    head[:d] = np.eye(d)[::-1]           # row v picks coordinate d-1-v
    s = np.array([1.0, 2.0, -0.5])
    l = O.lm_logits(h, head, s, chunk=4)  # chunking crosses a boundary
    for i in range(n):
        assert np.allclose(l[i, :d], s[i] * h[i, ::-1])
        assert np.all(l[i, d:] == 0)
    assert np.allclose(O.lm_logits(h, head, 3.0)[:, :d], 3.0 * h[:, ::-1])


# ---------------------------------------------------------------- S5 ------
@pytest.mark.parametrize("V", [2048, 262144])
def test_vocab_softmax_uniform_closed_form(V):
    st = O.vocab_softmax(np.zeros((2, V)))
    assert np.allclose(st.entropy, math.log(V), rtol=0, atol=1e-12)
    assert np.allclose(st.conf, 1.0 / V)
    assert np.all(st.argmax == 0)
    # published values used in the design notes
    assert abs(math.log(2048) - 7.6246) < 1e-4
    assert abs(math.log(262144) - 12.4766) < 1e-4


def test_vocab_softmax_matches_library_routines():
    l = rng.standard_normal((5, 300)) * np.array([0.1, 1, 5, 30, 200])[:, None]
    st = O.vocab_softmax(l)
    assert np.allclose(st.p.sum(axis=1), 1.0, atol=1e-12)
    assert np.allclose(st.p, scipy.special.softmax(l, axis=1), rtol=1e-12, atol=1e-300)
    assert np.allclose(st.lse, scipy.special.logsumexp(l, axis=1), rtol=1e-13)
    assert np.allclose(st.entropy, scipy.stats.entropy(st.p, axis=1), rtol=1e-9, atol=1e-12)
    assert np.allclose(st.conf, st.p.max(axis=1), rtol=1e-13)
    assert np.all(st.entropy >= -1e-12) and np.all(st.entropy <= math.log(300) + 1e-12)


def test_vocab_softmax_ties_and_peaked_limit():
    l = np.array([[0.0, 3.0, 1.0, 3.0, 3.0]])
    assert O.vocab_softmax(l).argmax[0] == 1
    # planting h = c E_t with growing c drives H -> 0, conf -> 1, argmax -> t
    V, d, t = 50, 16, 17
    E = rng.standard_normal((V, d))
    prev = None
    for c in [1.0, 10.0, 100.0]:
        st = O.vocab_softmax(O.lm_logits(c * E[t][None], E, 1.0))
        assert st.argmax[0] == t
        if prev is not None:
            assert st.entropy[0] < prev
        prev = st.entropy[0]
    assert prev < 1e-6 and abs(st.conf[0] - 1) < 1e-6


# ---------------------------------------------------------------- S6 ------
def test_self_condition_closed_forms_and_linearity():
    V, d = 40, 7
    E = rng.standard_normal((V, d))
    uni = np.full((1, V), 1.0 / V)
    assert np.allclose(O.self_condition(uni, E)[0], E.mean(axis=0))
    onehot = np.zeros((1, V))
    onehot[0, 13] = 1.0
    assert np.array_equal(O.self_condition(onehot, E)[0], E[13])
    p = scipy.special.softmax(rng.standard_normal((3, V)), axis=1)
    E2 = rng.standard_normal((V, d))
    assert np.allclose(O.self_condition(p, 2 * E - 3 * E2),
                       2 * O.self_condition(p, E) - 3 * O.self_condition(p, E2))


# ---------------------------------------------------------------- S7 ------
def _brute_commit(ids, conf, ent, mask_id, tau):
    """Set-based restatement: the accepted set is the smallest confidence
    prefix (upward-closed under (conf desc, position asc)) whose entropy sum
    exceeds tau, or every candidate if no prefix does."""
    cand = [i for i in range(len(ids)) if ids[i] == mask_id]
    key = {i: (conf[i], -i) for i in cand}
    best = None
    for r in range(len(cand) + 1):
        for S in itertools.combinations(cand, r):
            Sset = set(S)
            closed = all(key[a] > key[b] for a in Sset for b in cand if b not in Sset)
            if not closed:
                continue
            if sum(ent[i] for i in S) > tau:
                if best is None or len(S) < len(best):
                    best = Sset
    if best is None:
        best = set(cand)
    m = np.zeros(len(ids), dtype=np.uint8)
    for i in best:
        m[i] = 1
    return m


@pytest.mark.parametrize("trial", range(40))
def test_commit_equals_brute_force(trial):
    r = np.random.default_rng(trial)
    C = int(r.integers(1, 11))
    ids = r.integers(0, 3, size=C)           # mask id 0 ~ a third of positions
    conf = np.round(r.uniform(0, 1, size=C), 1)  # coarse values -> real ties
    ent = r.choice([0.0, 0.3, 0.7, 1.5], size=C)
    tau = float(r.choice([0.0, 0.5, 1.0, 2.0]))
    am = r.integers(100, 200, size=C)
    m, out, n = O.commit_canvas(ids, conf, ent, am, 0, tau)
    bm = _brute_commit(ids, conf, ent, 0, tau)
    assert np.array_equal(m, bm)
    assert n == int(bm.sum())
    assert np.array_equal(out, np.where(m == 1, am, ids))


def test_commit_hand_cases():
    with open(os.path.join(GOLDEN, "commit_hand_cases.json")) as f:
        cases = json.load(f)["cases"]
    for c in cases:
        m, out, n = O.commit_canvas(np.array(c["ids"]), np.array(c["conf"]),
                                    np.array(c["entropy"]), np.array(c["argmax"]),
                                    c["mask_id"], c["tau"])
        assert list(m) == c["mask"], c["name"]
        assert list(out) == c["out_ids"], c["name"]
        assert n == c["n"], c["name"]


def test_commit_permutation_equivariance():
    r = np.random.default_rng(7)
    C = 30
    ids = np.where(r.uniform(size=C) < 0.6, 5, 1)
    conf = r.uniform(size=C)                 # distinct with probability 1
    ent = r.uniform(0, 0.5, size=C)
    am = r.integers(0, 9, size=C)
    m, _, _ = O.commit_canvas(ids, conf, ent, am, 5, 1.3)
    perm = r.permutation(C)
    m2, _, _ = O.commit_canvas(ids[perm], conf[perm], ent[perm], am[perm], 5, 1.3)
    assert np.array_equal(m[perm], m2)


# ---------------------------------------------------------------- S8 ------
def test_label_read_two_routes_and_invariants():
    V = 500
    l = rng.standard_normal(V) * 4
    lse = scipy.special.logsumexp(l)
    labels = np.array([3, 77, 120, 499, 0])
    lp, r = O.label_read(l, lse, labels)
    assert np.all(lp <= 0)
    assert abs(r.sum() - 1) < 1e-14
    # the full-vocabulary normaliser cancels: r is the softmax of the raw label logits
    assert np.allclose(r, scipy.special.softmax(l[labels]), rtol=1e-13)
    assert np.allclose(lp, np.log(scipy.special.softmax(l))[labels], rtol=1e-12)


def test_label_read_closed_forms():
    lp, r = O.label_read(np.array([math.log(3.0), 0.0]), 5.0, np.array([0, 1]))
    assert np.allclose(r, [0.75, 0.25])
    assert abs(O._entropy(r) - 0.5623351446188083) < 1e-15
    lp, r = O.label_read(np.full(10, 2.0), 4.0, np.arange(7))
    assert abs(O._entropy(r) - math.log(7)) < 1e-14
    lp, r = O.label_read(np.array([1.0, 2.0]), 3.0, np.array([1]))
    assert r[0] == 1.0 and O._entropy(r) == 0.0


def _tiny_problem(seed=0, C=12, P=5, V=40, d=8, Hq=2, Hkv=1, hd=4, W=3):
    r = np.random.default_rng(seed)
    dims = Dims(d_model=d, n_q_heads=Hq, n_kv_heads=Hkv, head_dim=hd, vocab=V,
                canvas=C, window=W, mask_id=V - 1, dtype="f32")
    E = r.standard_normal((V, d)) * 0.5
    Wq, Wk, Wv = (r.standard_normal((n * hd, d)) * 0.5 for n in (Hq, Hkv, Hkv))
    Wo = r.standard_normal((d, Hq * hd)) * 0.5
    Kp = r.standard_normal((P, Hkv, hd))
    Vp = r.standard_normal((P, Hkv, hd))
    ids = r.integers(0, V - 1, size=C)
    return dims, E, Wq, Wk, Wv, Wo, Kp, Vp, ids


def test_slot_read_first_read_matches_step_rows():
    dims, E, Wq, Wk, Wv, Wo, Kp, Vp, ids = _tiny_problem()
    slots = np.array([2, 9])
    ids[slots] = dims.mask_id
    labels = np.full((2, 26), -1)
    labels[0, :3] = [4, 5, 6]
    labels[1, :2] = [10, 30]
    nl = np.array([3, 2])
    noise = np.zeros((1, 2), dtype=np.int64)
    res = O.slot_read_canvas(E, Wq, Wk, Wv, Wo, Kp, Vp, ids, dims, slots, labels, nl, noise,
                             logit_scale=2.0, n_draws=1)
    step = O.denoise_canvas(E, Wq, Wk, Wv, Wo, Kp, Vp, ids, dims, logit_scale=2.0,
                            need_sc=False, need_logits=True)
    for s, pos in enumerate(slots):
        k = nl[s]
        lp = step["logits"][pos, labels[s, :k]] - step["lse"][pos]
        assert np.allclose(res["logprobs"][s, :k], lp, rtol=1e-12, atol=1e-12)
        assert abs(res["probs"][s, :k].sum() - 1) < 1e-13
        assert res["draws_used"][s] == 1
        assert np.all(res["probs"][s, k:] == 0)


def test_slot_read_reread_rules():
    dims, E, Wq, Wk, Wv, Wo, Kp, Vp, ids = _tiny_problem(seed=3)
    slots = np.array([1, 6])
    ids[slots] = dims.mask_id
    labels = np.full((2, 26), -1)
    labels[0, :4] = [4, 5, 6, 7]
    labels[1, :1] = [12]                      # k = 1: r = 1, H = 0, never re-read
    nl = np.array([4, 1])
    # draws that write the mask id back reproduce the first read exactly
    same = np.full((4, 2), dims.mask_id)
    res = O.slot_read_canvas(E, Wq, Wk, Wv, Wo, Kp, Vp, ids, dims, slots, labels, nl, same,
                             logit_scale=0.01, n_draws=4)
    assert res["first_entropy"][0] > 0.1      # near-flat over 4 labels: re-read
    assert res["draws_used"][0] == 4 and res["draws_used"][1] == 1
    assert np.allclose(res["entropy"][0], res["first_entropy"][0], rtol=1e-12)
    one = O.slot_read_canvas(E, Wq, Wk, Wv, Wo, Kp, Vp, ids, dims, slots, labels, nl, same,
                             logit_scale=0.01, n_draws=1)
    assert np.allclose(res["probs"], one["probs"], rtol=1e-12)
    assert res["probs"][1, 0] == 1.0 and res["entropy"][1] == 0.0
    # real noise draws: the average of 4 distributions, each summing to 1
    noise = np.random.default_rng(5).integers(0, dims.vocab - 1, size=(4, 2))
    res2 = O.slot_read_canvas(E, Wq, Wk, Wv, Wo, Kp, Vp, ids, dims, slots, labels, nl, noise,
                              logit_scale=0.01, n_draws=4)
    assert abs(res2["probs"][0, :4].sum() - 1) < 1e-13
    assert res2["first_entropy"][0] == res["first_entropy"][0]
    manual = []
    for d in range(4):
        cid = ids.copy()
        cid[slots] = noise[d]
        st = O.denoise_canvas(E, Wq, Wk, Wv, Wo, Kp, Vp, cid, dims, logit_scale=0.01,
                              need_sc=False, need_logits=True)
        manual.append(scipy.special.softmax(st["logits"][slots[0], labels[0, :4]]))
    assert np.allclose(res2["probs"][0, :4], np.mean(manual, axis=0), rtol=1e-12)
    # a peaked slot stays a single read: H <= 0.1
    res3 = O.slot_read_canvas(E, Wq, Wk, Wv, Wo, Kp, Vp, ids, dims, slots, labels, nl, noise,
                              logit_scale=1e4, n_draws=4)
    assert res3["first_entropy"][0] <= 0.1 and res3["draws_used"][0] == 1


def test_slot_read_status_codes():
    dims, E, Wq, Wk, Wv, Wo, Kp, Vp, ids = _tiny_problem(seed=4)
    slots = np.array([1, 50, 3, 4])
    labels = np.full((4, 26), -1)
    labels[:, :2] = [[2, 3], [2, 3], [2, 3], [2, dims.vocab]]
    nl = np.array([0, 2, 2, 2])
    res = O.slot_read_canvas(E, Wq, Wk, Wv, Wo, Kp, Vp, ids, dims, slots, labels, nl,
                             np.zeros((1, 4), dtype=np.int64), n_draws=1)
    assert list(res["status"]) == [O.SLOT_BAD_COUNT, O.SLOT_BAD_POS, O.SLOT_OK, O.SLOT_BAD_LABEL]
    assert list(res["best"][[0, 1, 3]]) == [-1, -1, -1]


def test_page_constants():
    with open(os.path.join(GOLDEN, "page_facts.json")) as f:
        facts = json.load(f)
    assert oracle.MAX_LABELS == facts["max_labels"]["value"]
    from synth import CONFIGS
    for c in CONFIGS.values():
        assert c.dims.canvas == facts["canvas_tokens"]["value"]
    assert CONFIGS["long_read"].prompt[1] == facts["long_context_tokens"]["value"]
    assert CONFIGS["bf16_step"].dims.head_dim == facts["attention_head_width"]["value"]
    assert CONFIGS["reads512"].entropy_threshold == facts["reread_entropy_threshold"]["value"]
    assert CONFIGS["reads512"].n_draws == facts["draws_per_stage"]["value"]


# -------------------------------------------------- near-tie declarations --
def test_commit_near_ties_rule():
    # distinct, well separated confidences and entropies far from tau: nothing excused
    ids = np.zeros(6, dtype=int)
    conf = np.array([0.9, 0.7, 0.5, 0.3, 0.2, 0.1])
    ent = np.array([0.2, 0.2, 0.2, 0.2, 0.2, 0.2])
    near = O.commit_near_ties(ids, conf, ent, 0, 0.5, conf_eps=1e-3)
    assert not near.any()
    # a threshold landing within 1e-3 of a prefix excuses that rank
    near = O.commit_near_ties(ids, conf, ent, 0, 0.4 + 5e-4, conf_eps=1e-3)
    assert near[2] and near.sum() == 1
    # a confidence cluster straddling the boundary is excused as a whole
    conf2 = np.array([0.9, 0.7, 0.50001, 0.5, 0.49999, 0.1])
    near = O.commit_near_ties(ids, conf2, ent, 0, 0.5, conf_eps=1e-3)
    assert list(np.nonzero(near)[0]) == [2, 3, 4]
