"""GPU parity of dg_slot_read_staged (two stages, ask_if conditions, stage-0
answers pinned into the canvas) against the oracle's staged read.

A stage-1 result depends on the stage-0 answers through the pinned tokens and
the ask_if conditions, so canvases where the oracle declares a stage-0 best
label or re-read decision a near-tie are left out of the comparison."""
import numpy as np
import pytest

import oracle
from synth import config, make_inputs, companion_row_scale
from tests.helpers import TOL, TIE_EPS, to_np

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def torch_cuda():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch


def _decisive(ref, inp, stage0, dtype):
    th = inp["entropy_threshold"]
    near_th = np.abs(ref["first_entropy"] - th) < TOL[dtype]["entropy_abs"]
    near_best = oracle.best_near_ties(ref["probs"], inp["n_labels"], TIE_EPS[dtype]).mask
    return ~(near_th[:, stage0] | near_best[:, stage0]).any(axis=1)


# Companion row scales (16-512 x) give decisive stage-0 answers, with label
# logprobs down to about -55, checked at the absolute 1e-2 bar in bf16.
@pytest.mark.parametrize("name,dtype,over,hi", [
    ("tiny_f32", "f32", dict(batch=4), 512.0),
    ("reads512", "bf16", dict(batch=16), 512.0),
])
def test_staged_read_matches_oracle(torch_cuda, name, dtype, over, hi):
    import torch
    from slot_readout_amd.runtime import DeviceProblem
    from tests.test_gpu_slot import _check_slots
    inp = make_inputs(config(name), prompt_override=("fixed", 96), **over)
    B, S = inp["slot_pos"].shape
    rs = companion_row_scale(inp, (B, S), 16.0, hi)
    stage = np.array([0] * (S // 2) + [1] * (S - S // 2))
    S0 = np.nonzero(stage == 0)[0]
    # conditions chosen from the oracle's stage-0 answers of canvas 0, so that
    # they hold on some canvases and fail on others
    plain = oracle.slot_read_staged(inp, stage, np.full(S, -1), np.zeros(S, int), row_scale=rs)
    ask = np.full(S, -1)
    lab = np.zeros(S, int)
    s1 = np.nonzero(stage == 1)[0]
    ask[s1[0]], lab[s1[0]] = S0[0], plain["best"][0, S0[0]]
    if len(s1) > 1 and len(S0) > 1:
        ask[s1[1]], lab[s1[1]] = S0[1], (plain["best"][0, S0[1]] + 1) % int(inp["n_labels"][0, S0[1]])
    ref = oracle.slot_read_staged(inp, stage, ask, lab, row_scale=rs)
    assert (ref["status"] == oracle.SLOT_NOT_ASKED).any() and (ref["status"][:, s1] == oracle.SLOT_OK).any()
    dev = DeviceProblem(inp, with_embed_t=False)
    out = dev.slot_read_staged(stage, ask, lab, row_scale=torch.from_numpy(rs).cuda())
    torch.cuda.synchronize()
    g = {k: to_np(v) for k, v in out.items()}
    keep = _decisive(ref, inp, S0, dtype)
    assert keep.sum() >= 2, f"only {keep.sum()} canvases without stage-0 near-ties"
    sub = lambda d: {k: v[keep] for k, v in d.items()}       # noqa: E731
    _check_slots(sub(g), sub(ref), dict(inp, n_labels=inp["n_labels"][keep]), dtype, f"staged {name}")
    # slots not asked report exactly the skipped-slot outputs
    na = ref["status"] == oracle.SLOT_NOT_ASKED
    assert (g["status"][na & keep[:, None]] == oracle.SLOT_NOT_ASKED).all()
    assert not g["probs"][na & keep[:, None]].any()


def test_staged_read_without_second_stage_is_the_plain_read(torch_cuda):
    """All slots in stage 0: bitwise the outputs of dg_slot_read."""
    import torch
    from slot_readout_amd.runtime import DeviceProblem
    inp = make_inputs(config("reads512"), batch=4, prompt_override=("fixed", 64))
    S = inp["slot_pos"].shape[1]
    dev = DeviceProblem(inp, with_embed_t=False)
    a = dev.slot_read_staged([0] * S, [-1] * S, [0] * S)
    b = dev.slot_read()
    torch.cuda.synchronize()
    for k in a:
        assert torch.equal(a[k], b[k]), k


def test_staged_read_deterministic(torch_cuda):
    import torch
    from slot_readout_amd.runtime import DeviceProblem
    inp = make_inputs(config("reads512"), batch=6, prompt_override=("fixed", 80))
    S = inp["slot_pos"].shape[1]
    stage, ask, lab = [0, 0, 1, 1][:S], [-1, -1, 0, -1][:S], [0, 0, 1, 0][:S]
    dev = DeviceProblem(inp, with_embed_t=False)
    a = {k: v.clone() for k, v in dev.slot_read_staged(stage, ask, lab).items()}
    b = dev.slot_read_staged(stage, ask, lab)
    torch.cuda.synchronize()
    for k in a:
        assert torch.equal(a[k], b[k]), k
