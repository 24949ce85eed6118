"""Pins of the prefill oracle (prompt KV cache of the one-block surrogate), CPU only."""
import numpy as np

import oracle


def test_prefill_with_selection_matrices_reads_embedding_columns():
    """Wk, Wv that select columns of the embedding make the cache entries those
    columns of E[id]; ids outside [0, V) give zero rows."""
    rng = np.random.default_rng(5)
    V, d, Hkv, hd = 40, 24, 2, 4
    E = rng.normal(size=(V, d))
    ck = rng.choice(d, size=Hkv * hd, replace=False)
    cv = rng.choice(d, size=Hkv * hd, replace=False)
    Wk = np.eye(d)[ck]          # [Hkv*hd, d]: row j picks column ck[j]
    Wv = np.eye(d)[cv]
    ids = np.array([3, 0, 39, 17, -1, 40, 3])
    k, v = oracle.prefill_kv(E, Wk, Wv, ids, Hkv, hd)
    assert k.shape == (len(ids), Hkv, hd) and v.shape == (len(ids), Hkv, hd)
    for t, i in enumerate(ids):
        if 0 <= i < V:
            np.testing.assert_array_equal(k[t].reshape(-1), E[i, ck])
            np.testing.assert_array_equal(v[t].reshape(-1), E[i, cv])
        else:
            assert not k[t].any() and not v[t].any()


def test_prefill_is_linear_in_the_weights():
    rng = np.random.default_rng(6)
    V, d, Hkv, hd = 30, 16, 1, 8
    E = rng.normal(size=(V, d))
    A, B = rng.normal(size=(hd, d)), rng.normal(size=(hd, d))
    ids = rng.integers(0, V, size=11)
    ka, _ = oracle.prefill_kv(E, A, A, ids, Hkv, hd)
    kb, _ = oracle.prefill_kv(E, B, B, ids, Hkv, hd)
    kab, _ = oracle.prefill_kv(E, 2 * A - B, A, ids, Hkv, hd)
    np.testing.assert_allclose(kab, 2 * ka - kb, rtol=1e-12, atol=1e-12)


# ------------------------------------------------ encoder-mode attention ---
def _qkv(rng, P, Hq, Hkv, hd):
    return (rng.normal(size=(P, Hq, hd)), rng.normal(size=(P, Hkv, hd)),
            rng.normal(size=(P, Hkv, hd)))


def test_causal_first_row_is_its_own_value():
    """Query 0 sees key 0 only: its output is v_0 of its kv head (GQA)."""
    rng = np.random.default_rng(21)
    q, k, v = _qkv(rng, 9, 4, 2, 8)
    o = oracle.causal_attention(q, k, v)
    for h in range(4):
        np.testing.assert_array_equal(o[0, h], v[0, h // 2])


def test_causal_rows_do_not_see_later_tokens():
    """Changing tokens after t leaves rows <= t bit for bit unchanged, and rows
    after t change."""
    rng = np.random.default_rng(22)
    q, k, v = _qkv(rng, 40, 2, 1, 16)
    o = oracle.causal_attention(q, k, v)
    k2, v2, q2 = k.copy(), v.copy(), q.copy()
    k2[25:] = rng.normal(size=k2[25:].shape)
    v2[25:] = rng.normal(size=v2[25:].shape)
    q2[25:] = rng.normal(size=q2[25:].shape)
    o2 = oracle.causal_attention(q2, k2, v2)
    np.testing.assert_array_equal(o2[:25], o[:25])
    assert np.abs(o2[25:] - o[25:]).min(axis=(1, 2)).max() > 0


def test_causal_row_equals_decoder_attention_over_a_prefix():
    """Row t equals the decoder-mode attention of query t whose prompt is
    tokens 0..t-1 and whose canvas is token t alone (window 0): the same key
    set, through the independently pinned window_attention."""
    rng = np.random.default_rng(23)
    q, k, v = _qkv(rng, 30, 4, 2, 8)
    o = oracle.causal_attention(q, k, v)
    for t in (1, 7, 29):
        ref = oracle.window_attention(q[t:t + 1], k[t:t + 1], v[t:t + 1], k[:t], v[:t], 0)
        np.testing.assert_allclose(o[t], ref[0], rtol=1e-12, atol=1e-12)


def test_causal_equal_scores_average_the_values():
    """With every key equal, all visible scores tie: row t is the mean of v_0..v_t."""
    rng = np.random.default_rng(24)
    P, hd = 17, 8
    q = rng.normal(size=(P, 2, hd))
    k = np.repeat(rng.normal(size=(1, 1, hd)), P, axis=0)
    v = rng.normal(size=(P, 1, hd))
    o = oracle.causal_attention(q, k, v)
    for t in range(P):
        for h in range(2):
            np.testing.assert_allclose(o[t, h], v[:t + 1, 0].mean(axis=0), rtol=1e-12, atol=1e-12)


def test_causal_rows_subset_matches_all_rows():
    rng = np.random.default_rng(25)
    q, k, v = _qkv(rng, 33, 2, 2, 4)
    rows = np.array([0, 5, 32, 17])
    np.testing.assert_allclose(oracle.causal_attention(q, k, v, rows),
                               oracle.causal_attention(q, k, v)[rows], rtol=1e-13, atol=1e-13)


def test_encode_prompt_assembles_the_block():
    """k, v equal the prefill cache entries; hidden_out = x + o Wo^T with x =
    E[id] (zero rows for ids outside [0, V)); Wo = 0 leaves h = x."""
    from synth import config, make_inputs
    inp = make_inputs(config("tiny_f32"), prompt_override=("fixed", 16))
    dims = inp["dims"]
    rng = np.random.default_rng(26)
    ids = rng.integers(0, dims.vocab, size=50)
    ids[3], ids[4] = -1, dims.vocab
    enc = oracle.encode_prompt(inp["embed"], inp["wq"], inp["wk"], inp["wv"], inp["wo"], ids, dims)
    k, v = oracle.prefill_kv(inp["embed"], inp["wk"], inp["wv"], ids, dims.n_kv_heads, dims.head_dim)
    np.testing.assert_array_equal(enc["k"], k)
    np.testing.assert_array_equal(enc["v"], v)
    x = oracle.embed_input(inp["embed"], ids)
    assert not x[3].any() and not x[4].any()
    np.testing.assert_allclose(enc["hidden_out"], x + enc["attn_out"] @ np.asarray(inp["wo"], np.float64).T,
                               rtol=1e-12, atol=1e-12)
    z = oracle.encode_prompt(inp["embed"], inp["wq"], inp["wk"], inp["wv"], np.zeros_like(inp["wo"]), ids, dims)
    np.testing.assert_array_equal(z["hidden_out"], x)
