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
