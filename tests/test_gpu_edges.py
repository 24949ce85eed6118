"""GPU parity at the edges of the method and of the input checks, through the
C-ABI: windows of 0 and >= C-1 (the full-block case), a window near INT_MAX,
non-monotone prompt offsets and out-of-range canvas ids."""
import numpy as np
import pytest

import oracle
from synth import config, make_inputs
from tests.helpers import TOL, TIE_EPS, to_np, assert_row_rel, assert_float

pytestmark = pytest.mark.gpu

DG_FLAG_BAD_TOKEN = 1
DG_FLAG_BAD_SEQLENS = 2


@pytest.fixture(scope="module")
def torch_cuda():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch


def _compare(out, refs, dtype, label):
    tol = TOL[dtype]
    for b, ref in enumerate(refs):
        tag = f"{label} canvas {b}"
        assert_row_rel(to_np(out["attn_out"][b]), ref["attn_out"], tol["attn_out"], f"{tag} attn_out")
        assert_row_rel(to_np(out["hidden_out"][b]), ref["hidden_out"], tol["hidden_out"], f"{tag} hidden_out")
        assert_row_rel(to_np(out["logits"][b]), ref["logits"], tol["logits"], f"{tag} logits")
        assert_row_rel(to_np(out["conf"][b])[None], ref["conf"][None], tol["conf"], f"{tag} conf")
        assert_float(to_np(out["entropy"][b]), ref["entropy"], dtype, "entropy", f"{tag} entropy")
        if out.get("sc_out") is not None and "sc_out" in ref:
            assert_row_rel(to_np(out["sc_out"][b]), ref["sc_out"], tol["sc_out"], f"{tag} sc_out")
        near = oracle.argmax_near_ties(ref["logits"], TIE_EPS[dtype]).mask
        bad = (to_np(out["argmax"][b]) != ref["argmax"]) & ~near
        assert not bad.any(), f"{tag} argmax at {np.nonzero(bad)[0][:8]}"


# agentlenshq, "DiffusionGemma: 4x faster text generation", section "Technical
# architecture and features": every token of the 256-block sees every other
# (W >= C-1); 24-ai.news, "How is diffusion text generation different?": the
# +-W window, inclusive.  W = 0 leaves each canvas query its own key only.
@pytest.mark.parametrize("name,over,prompt", [
    ("tiny_f32", {}, ("fixed", 128)),
    ("ragged32", {}, ("uniform", 0, 300)),
    ("bf16_step", dict(vocab=4096, mask_id=4095), ("fixed", 100)),
])
@pytest.mark.parametrize("W", [0, 255, 1000, 2 ** 31 - 1])
def test_step_window_edges(torch_cuda, name, over, prompt, W):
    import torch
    from slot_readout_amd.runtime import DeviceProblem
    B = 2 if name == "ragged32" else 1
    inp = make_inputs(config(name, window=W, **over), batch=B, prompt_override=prompt)
    dev = DeviceProblem(inp)
    out = dev.step(debug=True)
    torch.cuda.synchronize()
    assert int(out["flags"].item()) == 0
    refs = oracle.denoise_step(inp, need_logits=True)
    _compare(out, refs, inp["dims"].dtype, f"{name} W={W}")


def test_window_full_block_equals_every_key(torch_cuda):
    """W = C-1 and W = 2^31-1 give bitwise the same outputs (the same key set)."""
    import torch
    from slot_readout_amd.runtime import DeviceProblem
    outs = []
    for W in (255, 2 ** 31 - 1):
        inp = make_inputs(config("ragged32", window=W), batch=2, prompt_override=("fixed", 200))
        dev = DeviceProblem(inp)
        o = dev.step(debug=True)
        torch.cuda.synchronize()
        outs.append({k: to_np(v) for k, v in o.items() if v is not None})
    for k in outs[0]:
        assert np.array_equal(outs[0][k], outs[1][k]), k


def test_step_clamps_bad_prompt_offsets(torch_cuda):
    """cu_seqlens that decrease, or run past the cache, are clamped and flagged
    (DG_FLAG_BAD_SEQLENS): sequence b reads rows [max(cu[b], 0),
    min(cu[b+1], total)) of the cache, an empty range when that end is below
    the start, at most max_len rows.  The outputs equal the oracle's on those
    ranges."""
    import torch
    from slot_readout_amd.runtime import DeviceProblem
    from slot_readout_amd import dg
    from slot_readout_amd.runtime import to_device
    inp = make_inputs(config("ragged32"), batch=4, prompt_override=("fixed", 150))
    total = int(inp["cu_seqlens"][-1])      # 600 cache rows
    dev = DeviceProblem(inp)
    cu = np.array([0, 200, 120, 450, total + 77], dtype=np.int32)
    max_len = 400
    dev.cu = to_device(cu)
    dev.max_prompt = max_len
    dev.kv = dg.make_prompt_kv(dev.prompt_k, dev.prompt_v, dev.cu, max_len, total)
    out = dev.step(debug=True)
    torch.cuda.synchronize()
    assert int(out["flags"].item()) & DG_FLAG_BAD_SEQLENS
    ranges = []
    for b in range(4):
        p0 = max(int(cu[b]), 0)
        p1 = min(int(cu[b + 1]), total)
        p1 = max(p1, p0)
        p1 = min(p1, p0 + max_len)
        ranges.append((p0, p1))
    assert ranges == [(0, 200), (200, 200), (120, 450), (450, 600)]
    refs = []
    for b, (p0, p1) in enumerate(ranges):
        refs.append(oracle.denoise_canvas(
            inp["embed"], inp["wq"], inp["wk"], inp["wv"], inp["wo"], inp["prompt_k"][p0:p1],
            inp["prompt_v"][p0:p1], inp["canvas_ids"][b], inp["dims"],
            logit_scale=inp["logit_scale"], need_logits=True))
    _compare(out, refs, "bf16", "clamped offsets")


@pytest.mark.parametrize("name", ["tiny_f32", "ragged32"])
def test_step_out_of_range_canvas_ids(torch_cuda, name):
    """Canvas ids outside [0, V) embed as zero rows and set DG_FLAG_BAD_TOKEN; the
    rest of the step is unaffected (oracle with the same reading)."""
    import torch
    from slot_readout_amd.runtime import DeviceProblem
    inp = make_inputs(config(name), batch=1, prompt_override=("fixed", 64))
    V = inp["dims"].vocab
    ids = inp["canvas_ids"]
    ids[0, 3] = V
    ids[0, 77] = -5
    ids[0, 200] = 2 ** 30
    dev = DeviceProblem(inp)
    out = dev.step(debug=True)
    torch.cuda.synchronize()
    assert int(out["flags"].item()) == DG_FLAG_BAD_TOKEN
    refs = oracle.denoise_step(inp, need_logits=True)
    _compare(out, refs, inp["dims"].dtype, f"{name} bad ids")
    # a clean canvas leaves the flag clear
    inp2 = make_inputs(config(name), batch=1, prompt_override=("fixed", 64))
    out2 = DeviceProblem(inp2).step(debug=False)
    torch.cuda.synchronize()
    assert int(out2["flags"].item()) == 0
