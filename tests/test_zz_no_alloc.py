"""dg_slot_read_noalloc (the read with its workspace in the library's static
device array, for callers that cannot allocate) against dg_slot_read with a
caller workspace, through the C-ABI: two calls in a row, the second with a
smaller input, each bitwise equal to the workspace call on the same input
(the same kernels over the same plan), plus the size limit."""
import numpy as np
import pytest

import oracle
from synth import config, make_inputs, companion_row_scale
from tests.helpers import to_np

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def torch_cuda():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch


def _read_noalloc(dev, row_scale=None):
    from slot_readout_amd import dg
    out = dev.slot_outputs()
    dg.dg_slot_read_noalloc(dev.dims, dev.weights, dev.kv, dev.B, dev.canvas_ids, dev.S,
                            dev.slot_pos, dev.label_ids, dev.n_labels, dev.noise_ids,
                            dev.inp["logit_scale"], row_scale, dev.inp["entropy_threshold"],
                            dev.inp["n_draws"], out["logprobs"], out["probs"], out["entropy"],
                            out["first_entropy"], out["best"], out["draws_used"], out["status"])
    return out


def _same(a, b, label):
    for k in a:
        assert np.array_equal(to_np(a[k]), to_np(b[k])), f"{label}: {k}"


def test_noalloc_read_matches_workspace_read(torch_cuda):
    import torch
    from slot_readout_amd.runtime import DeviceProblem
    # first call: 12 canvases of the read batch with per-slot multipliers
    # (confident single reads and averaged re-reads)
    big = make_inputs(config("reads512"), batch=12, prompt_override=("fixed", 300))
    rs = torch.from_numpy(companion_row_scale(big, (12, 4), 256.0, 1024.0)).cuda()
    dev = DeviceProblem(big, with_embed_t=False)
    a = _read_noalloc(dev, rs)
    b = dev.slot_read(row_scale=rs)
    torch.cuda.synchronize()
    _same(a, b, "first call")
    du = to_np(a["draws_used"])
    assert (du == 1).any() and (du == 4).any()
    # the re-read decisions are the oracle's
    ref = oracle.slot_read(big, row_scale=to_np(rs))
    assert np.array_equal(du, ref["draws_used"])
    # second call, smaller: 3 canvases with shorter prompts and no multipliers;
    # the scratch still holds the first call's data
    small = make_inputs(config("reads512"), batch=3, prompt_override=("fixed", 64))
    dev2 = DeviceProblem(small, with_embed_t=False)
    c = _read_noalloc(dev2)
    d = dev2.slot_read()
    torch.cuda.synchronize()
    _same(c, d, "second call")
    # and the first input again after the smaller one
    e = _read_noalloc(dev, rs)
    torch.cuda.synchronize()
    _same(e, b, "third call")


def test_noalloc_read_headline_dims(torch_cuda):
    """The headline read (d 2816, V 262,144, 8 slots, 4 draws in one pass) fits
    the 64 MiB scratch: bitwise the workspace call."""
    import torch
    from slot_readout_amd.runtime import DeviceProblem
    inp = make_inputs(config("bf16_step"))
    dev = DeviceProblem(inp, with_embed_t=False)
    a = _read_noalloc(dev)
    b = dev.slot_read()
    torch.cuda.synchronize()
    _same(a, b, "headline")


def test_noalloc_read_rejects_reads_beyond_the_scratch(torch_cuda):
    """A read whose workspace exceeds the scratch is refused before any launch
    with DG_ERR_WORKSPACE; the outputs are left untouched."""
    import torch
    from slot_readout_amd import dg
    from slot_readout_amd.runtime import DeviceProblem
    inp = make_inputs(config("reads512"), batch=256, prompt_override=("fixed", 16))
    dev = DeviceProblem(inp, with_embed_t=False)
    need = dg.dg_slot_read_workspace(dev.dims, dev.B, dev.S, dev.max_prompt, inp["n_draws"])
    assert need > dg.DG_NOALLOC_SCRATCH_BYTES
    with pytest.raises(dg.DGError) as ei:
        _read_noalloc(dev)
    assert ei.value.status == dg.DG_ERR_WORKSPACE
    assert "static scratch" in str(ei.value)
