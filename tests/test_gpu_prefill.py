"""GPU parity of dg_prefill_kv (prompt KV cache from prompt token ids) against
the oracle, and a denoise step that reads the cache it wrote."""
import numpy as np
import pytest

import oracle
from synth import config, make_inputs
from tests.helpers import TOL, to_np, assert_row_rel

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def torch_cuda():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch


def _prompt_ids(inp, n, seed):
    rng = np.random.default_rng(seed)
    return rng.integers(0, inp["dims"].vocab - 1, size=n).astype(np.int32)


@pytest.mark.parametrize("name,over,dtype", [
    ("tiny_f32", {}, "f32"),
    ("bf16_step", dict(vocab=4096, mask_id=4095), "bf16"),
])
def test_prefill_matches_oracle(torch_cuda, name, over, dtype):
    """Ragged token count (a partial row tile) with one id out of range: its cache
    rows are zero and the device flag reports it."""
    import torch
    from slot_readout_amd import dg
    from slot_readout_amd.runtime import DeviceProblem
    inp = make_inputs(config(name, **over), prompt_override=("fixed", 64))
    dm = inp["dims"]
    dev = DeviceProblem(inp)
    ids = _prompt_ids(inp, 333, 3)
    ids[100] = dm.vocab + 5
    n = len(ids)
    k = torch.empty((n, dm.n_kv_heads, dm.head_dim), dtype=dev.tdt, device="cuda")
    v = torch.empty_like(k)
    flags = torch.zeros(1, dtype=torch.int32, device="cuda")
    dg.dg_prefill_kv(dev.dims, dev.weights, n, torch.from_numpy(ids).cuda(), k, v, flags)
    torch.cuda.synchronize()
    rk, rv = oracle.prefill_kv(inp["embed"], inp["wk"], inp["wv"], ids, dm.n_kv_heads, dm.head_dim)
    tol = TOL[dtype]["attn_out"]
    gk, gv = to_np(k).reshape(n, -1), to_np(v).reshape(n, -1)
    ok = np.arange(n) != 100
    assert_row_rel(gk[ok], rk.reshape(n, -1)[ok], tol, f"{name} prefill k")
    assert_row_rel(gv[ok], rv.reshape(n, -1)[ok], tol, f"{name} prefill v")
    assert not gk[100].any() and not gv[100].any()
    assert int(flags.item()) & dg.DG_FLAG_BAD_TOKEN


def test_step_reads_the_prefilled_cache(torch_cuda):
    """Prompt ids -> dg_prefill_kv into the packed cache -> dg_denoise_step, against
    the oracle step over the oracle's own prefilled cache (two prompts of
    different lengths)."""
    import torch
    from slot_readout_amd import dg
    from slot_readout_amd.runtime import DeviceProblem
    from tests.test_gpu_step import _check_step
    inp = make_inputs(config("ragged32", batch=2), prompt_override=("uniform", 150, 400))
    dm = inp["dims"]
    dev = DeviceProblem(inp)
    total = int(inp["cu_seqlens"][-1])
    ids = _prompt_ids(inp, total, 4)
    dg.dg_prefill_kv(dev.dims, dev.weights, total, torch.from_numpy(ids).cuda(),
                     dev.prompt_k, dev.prompt_v)
    out = dev.step(debug=True)
    torch.cuda.synchronize()
    rk, rv = oracle.prefill_kv(inp["embed"], inp["wk"], inp["wv"], ids, dm.n_kv_heads, dm.head_dim)
    ref_inp = dict(inp, prompt_k=rk, prompt_v=rv)
    refs = oracle.denoise_step(ref_inp, need_logits=True)
    _check_step(ref_inp, out, refs, "bf16", label="prefilled cache")
