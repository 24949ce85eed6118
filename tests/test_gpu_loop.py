"""GPU parity of dg_denoise_loop (denoise step + commit + self-conditioning
feedback until no mask id remains) against the CPU oracle's loop, through the
C-ABI.

The oracle declares, from its own values, the first step of each canvas at
which a commit or argmax decision is a near-tie; up to that step the two
trajectories must agree exactly (commit step and committed id of every
position).  Invariants are checked over the whole run."""
import numpy as np
import pytest

import oracle
from synth import config, make_inputs, companion_row_scale
from tests.helpers import TIE_EPS, to_np

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def torch_cuda():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch


def _check_invariants(ids0, mask_id, g):
    B = ids0.shape[0]
    for b in range(B):
        masked = ids0[b] == mask_id
        steps = int(g["steps"][b])
        cs = g["commit_step"][b]
        assert steps <= max(int(masked.sum()), 0)
        assert (cs[~masked] == -1).all(), f"canvas {b}: unmasked position committed"
        np.testing.assert_array_equal(g["ids"][b][~masked], ids0[b][~masked])
        assert (cs[masked] >= 0).all() and (cs[masked] < steps).all(), f"canvas {b}: commit steps"
        if masked.any():
            assert (np.bincount(cs[masked], minlength=steps) >= 1).all(), f"canvas {b}: a step without progress"
        assert not (g["ids"][b] == mask_id).any(), f"canvas {b}: a mask id remains"


def _compare(inp, ref, g, label):
    compared = 0
    for b in range(inp["batch"]):
        tie = int(ref["first_tie"][b])
        upto = int(ref["steps"][b]) if tie < 0 else tie
        early = (ref["commit_step"][b] >= 0) & (ref["commit_step"][b] < upto)
        np.testing.assert_array_equal(g["commit_step"][b][early], ref["commit_step"][b][early],
                                      err_msg=f"{label} canvas {b}: commit steps before step {upto}")
        np.testing.assert_array_equal(g["ids"][b][early], ref["ids"][b][early],
                                      err_msg=f"{label} canvas {b}: committed ids before step {upto}")
        # positions the GPU committed before that step were committed by the oracle too
        g_early = (g["commit_step"][b] >= 0) & (g["commit_step"][b] < upto)
        np.testing.assert_array_equal(g_early, early, err_msg=f"{label} canvas {b}: committed sets")
        if tie < 0:
            assert int(g["steps"][b]) == int(ref["steps"][b]), f"{label} canvas {b}: step count"
        compared += upto
    return compared


def _run(dev, **kw):
    out = dev.loop(**kw)
    return {k: to_np(v) if hasattr(v, "cpu") else v for k, v in out.items()}


def test_loop_uniform_rows_closed_form(torch_cuda):
    """Logit scale 0: rows are exactly uniform over V - 1 ids on the GPU too, so
    each step commits the lowest masked position with id 0."""
    from slot_readout_amd.runtime import DeviceProblem
    inp = make_inputs(config("tiny_f32", canvas=40))
    inp["logit_scale"] = 0.0
    dev = DeviceProblem(inp)
    g = _run(dev, tau=1.0, check_every=4)
    ids0 = inp["canvas_ids"]
    mask_id = inp["dims"].mask_id
    masked = ids0[0] == mask_id
    rank = np.cumsum(masked) - 1
    np.testing.assert_array_equal(g["commit_step"][0], np.where(masked, rank, -1))
    np.testing.assert_array_equal(g["ids"][0], np.where(masked, 0, ids0[0]))
    assert int(g["steps"][0]) == int(masked.sum())
    assert int(g["flags"][0]) == 0


def test_loop_tiny_f32_companion(torch_cuda):
    """Full 256-position canvas, fp32, peaked and flat rows (companion row
    scales), tau 1.0: trajectory equal to the oracle's up to its first near-tie."""
    from slot_readout_amd.runtime import DeviceProblem
    inp = make_inputs(config("tiny_f32"))
    rs = companion_row_scale(inp, (1, 256))
    dev = DeviceProblem(inp)
    import torch
    g = _run(dev, tau=1.0, row_scale=torch.from_numpy(rs).cuda(), check_every=8)
    ref = oracle.denoise_loop(inp, 1.0, row_scale=rs, tie_eps=TIE_EPS["f32"])
    _check_invariants(inp["canvas_ids"], inp["dims"].mask_id, g)
    n = _compare(inp, ref, g, "tiny_f32")
    assert n >= 10, f"only {n} steps before a declared near-tie"


def test_loop_ragged_bf16_batch(torch_cuda):
    """Three bf16 canvases with different prompts and mask fractions finish at
    different steps (finished canvases are skipped on the device)."""
    from slot_readout_amd.runtime import DeviceProblem
    import torch
    inp = make_inputs(config("ragged32", batch=3, canvas=96), prompt_override=("uniform", 50, 300))
    rs = companion_row_scale(inp, (3, 96))
    dev = DeviceProblem(inp)
    g = _run(dev, tau=2.0, row_scale=torch.from_numpy(rs).cuda(), check_every=3)
    ref = oracle.denoise_loop(inp, 2.0, row_scale=rs, tie_eps=TIE_EPS["bf16"])
    _check_invariants(inp["canvas_ids"], inp["dims"].mask_id, g)
    _compare(inp, ref, g, "ragged bf16")
    assert len(set(int(s) for s in g["steps"])) > 1, "canvases should finish at different steps"


def test_loop_check_interval_changes_nothing(torch_cuda):
    """check_every only decides when the host looks: the outputs are the same;
    with an interval past the end every step up to max_steps is launched."""
    from slot_readout_amd.runtime import DeviceProblem
    inp = make_inputs(config("tiny_f32", canvas=64))
    dev = DeviceProblem(inp)
    a = _run(dev, tau=1.0, check_every=1, max_steps=64)
    b = _run(dev, tau=1.0, check_every=1000, max_steps=64)
    for k in ("ids", "commit_step", "steps"):
        np.testing.assert_array_equal(a[k], b[k], err_msg=k)
    assert a["launched"] == int(a["steps"].max()) and b["launched"] == 64


def test_loop_deterministic(torch_cuda):
    """Two runs of the loop (fixed-order reductions, no float atomics) give bitwise
    the same canvases, commit steps and step counts."""
    from slot_readout_amd.runtime import DeviceProblem
    import torch
    inp = make_inputs(config("ragged32", batch=3, canvas=96), prompt_override=("uniform", 50, 300))
    rs = torch.from_numpy(companion_row_scale(inp, (3, 96))).cuda()
    dev = DeviceProblem(inp)
    a = _run(dev, tau=2.0, row_scale=rs, check_every=2)
    b = _run(dev, tau=2.0, row_scale=rs, check_every=5)
    for k in ("ids", "commit_step", "steps"):
        np.testing.assert_array_equal(a[k], b[k], err_msg=k)
