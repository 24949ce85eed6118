"""GPU parity of dg_prefill_encode, the encoder-mode forward over packed
prompts (causal attention per sequence, chunks of `canvas` tokens), against
the oracle's encode_prompt: ragged sequences across chunk edges, GQA at head
width 512, a 110,707-token prompt on sampled rows, clamped offsets and the
optional outputs."""
import numpy as np
import pytest

import oracle
from synth import config, make_inputs, prompt_batch
from tests.helpers import TOL, to_np, assert_row_rel

pytestmark = pytest.mark.gpu

DG_FLAG_BAD_TOKEN = 1
DG_FLAG_BAD_SEQLENS = 2


@pytest.fixture(scope="module")
def torch_cuda():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch


def _run(inp, ids, cu, max_len, total, **kw):
    import torch
    from slot_readout_amd.runtime import DeviceProblem
    dev = DeviceProblem(inp, with_embed_t=False)
    out = dev.encode(torch.from_numpy(ids).cuda(), torch.from_numpy(cu).cuda(), max_len, total, **kw)
    torch.cuda.synchronize()
    return out


def _check_seq(inp, out, ids, p0, p1, dtype, tag, rows=None):
    """Rows [p0, p1) of the outputs against the oracle's encoder over ids[p0:p1]
    (rows: positions within the sequence, default all)."""
    dm = inp["dims"]
    ref = oracle.encode_prompt(inp["embed"], inp["wq"], inp["wk"], inp["wv"], inp["wo"], ids[p0:p1],
                               dm, rows=rows)
    r = ref["rows"] + p0
    tol = TOL[dtype]
    if out["attn"] is not None:
        assert_row_rel(to_np(out["attn"])[r], ref["attn_out"], tol["attn_out"], f"{tag} attn_out")
    if out["hidden"] is not None:
        assert_row_rel(to_np(out["hidden"])[r], ref["hidden_out"], tol["hidden_out"], f"{tag} hidden_out")
    n = p1 - p0
    assert_row_rel(to_np(out["k"])[p0:p1].reshape(n, -1), ref["k"].reshape(n, -1), tol["attn_out"], f"{tag} k")
    assert_row_rel(to_np(out["v"])[p0:p1].reshape(n, -1), ref["v"].reshape(n, -1), tol["attn_out"], f"{tag} v")


@pytest.mark.parametrize("name,over,lengths", [
    # fp32, 4 heads x 64: empty, 1 token, and lengths around the 256-token chunk
    ("tiny_f32", {}, [0, 1, 255, 256, 257, 700]),
    # bf16, 4 heads x 64 (the read workloads' dims)
    ("ragged32", {}, [300, 1030, 5, 512]),
    # bf16, 8 query heads / 2 kv heads x 512 (the headline dims), V 4096
    ("bf16_step", dict(vocab=4096, mask_id=4095), [600, 130]),
])
def test_encode_matches_oracle(torch_cuda, name, over, lengths):
    inp = make_inputs(config(name, **over), prompt_override=("fixed", 16))
    dtype = inp["dims"].dtype
    ids, cu = prompt_batch(inp["dims"].vocab, lengths, seed=31)
    out = _run(inp, ids, cu, max(lengths), int(cu[-1]))
    assert int(out["flags"].item()) == 0
    for b in range(len(lengths)):
        if lengths[b]:
            _check_seq(inp, out, ids, int(cu[b]), int(cu[b + 1]), dtype, f"{name} seq {b}")


def test_encode_long_prompt_sampled_rows(torch_cuda):
    """One 110,707-token prompt at the read workloads' dims (bf16, 4 x 64):
    rows at the start, around chunk edges, spread through, and at the end."""
    inp = make_inputs(config("long_read"), prompt_override=("fixed", 16))
    P = 110_707
    ids, cu = prompt_batch(inp["dims"].vocab, [P], seed=32)
    out = _run(inp, ids, cu, P, P)
    assert int(out["flags"].item()) == 0
    rng = np.random.default_rng(33)
    rows = np.unique(np.concatenate([[0, 1, 2, 255, 256, 257, 511, 512, 65535, 65536],
                                     rng.integers(0, P, size=16), [P - 3, P - 2, P - 1]]))
    _check_seq(inp, out, ids, 0, P, "bf16", "long prompt", rows=rows)


def test_encode_bad_ids_and_clamped_offsets(torch_cuda):
    """An id out of range embeds as a zero row (DG_FLAG_BAD_TOKEN); offsets that
    decrease or run past the rows are clamped (DG_FLAG_BAD_SEQLENS): sequence b
    covers [max(cu[b], 0), min(cu[b+1], total)), empty when that end is below
    the start, cut to max_len tokens."""
    inp = make_inputs(config("ragged32"), prompt_override=("fixed", 16))
    V = inp["dims"].vocab
    ids, _ = prompt_batch(V, [900], seed=34)
    ids[40] = V + 2
    total = 900
    cu = np.array([0, 300, 200, 700, total + 50], dtype=np.int32)
    max_len = 350
    out = _run(inp, ids, cu, max_len, total)
    flags = int(out["flags"].item())
    assert flags & DG_FLAG_BAD_SEQLENS and flags & DG_FLAG_BAD_TOKEN
    ranges = []
    for b in range(4):
        p0 = max(int(cu[b]), 0)
        p1 = max(min(int(cu[b + 1]), total), p0)
        ranges.append((p0, min(p1, p0 + max_len)))
    assert ranges == [(0, 300), (300, 300), (200, 550), (700, 900)]
    # rows that two clamped sequences share (200..299 here) hold one of the two
    # results; every other row of each sequence is checked
    owners = np.zeros(total, dtype=np.int64)
    for p0, p1 in ranges:
        owners[p0:p1] += 1
    for b, (p0, p1) in enumerate(ranges):
        if p1 > p0:
            rows = np.nonzero(owners[p0:p1] == 1)[0]
            _check_seq(inp, out, ids, p0, p1, "bf16", f"clamped seq {b}", rows=rows)


def test_encode_optional_outputs(torch_cuda):
    """hidden_out alone and attn_out alone give the same rows as both together;
    with neither, the call writes the cache as dg_prefill_kv does."""
    import torch
    from slot_readout_amd import dg
    from slot_readout_amd.runtime import DeviceProblem
    inp = make_inputs(config("ragged32"), prompt_override=("fixed", 16))
    ids, cu = prompt_batch(inp["dims"].vocab, [270, 40], seed=35)
    total = int(cu[-1])
    both = _run(inp, ids, cu, 270, total)
    h_only = _run(inp, ids, cu, 270, total, want_attn=False)
    a_only = _run(inp, ids, cu, 270, total, want_hidden=False)
    assert np.array_equal(to_np(h_only["hidden"]), to_np(both["hidden"]))
    assert np.array_equal(to_np(a_only["attn"]), to_np(both["attn"]))
    none = _run(inp, ids, cu, 270, total, want_hidden=False, want_attn=False)
    dev = DeviceProblem(inp, with_embed_t=False)
    dm = inp["dims"]
    k = torch.empty((total, dm.n_kv_heads, dm.head_dim), dtype=dev.tdt, device="cuda")
    v = torch.empty_like(k)
    dg.dg_prefill_kv(dev.dims, dev.weights, total, torch.from_numpy(ids).cuda(), k, v)
    torch.cuda.synchronize()
    assert np.array_equal(to_np(none["k"]), to_np(k)) and np.array_equal(to_np(none["v"]), to_np(v))
    assert np.array_equal(to_np(both["k"]), to_np(k))


def test_encode_twice_is_deterministic(torch_cuda):
    inp = make_inputs(config("bf16_step", vocab=4096, mask_id=4095), prompt_override=("fixed", 16))
    ids, cu = prompt_batch(4096, [700], seed=36)
    a = _run(inp, ids, cu, 700, 700)
    b = _run(inp, ids, cu, 700, 700)
    for key in ("hidden", "attn", "k", "v"):
        assert np.array_equal(to_np(a[key]), to_np(b[key])), key
