"""GPU parity at the workloads' full sizes, through the same C-ABI calls and
launch configuration bench.py times, against the float64 oracle on every
canvas (these sizes still run in seconds on the host)."""
import numpy as np
import pytest

import oracle
from synth import config, make_inputs, companion_row_scale
from tests.helpers import TOL, TIE_EPS, to_np, assert_row_rel, assert_float

pytestmark = [pytest.mark.gpu, pytest.mark.slow]


@pytest.fixture(scope="module")
def torch_cuda():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch


def _step_compare(inp, out, refs, canvases, label, check_sc=True, max_excused=None):
    """conf, entropy, p.E and argmax of each canvas against the oracle; with
    max_excused, the fraction of argmax near-ties must stay below it."""
    for i, b in enumerate(canvases):
        ref = refs[i]
        tag = f"{label} canvas {b}"
        assert_row_rel(to_np(out["conf"][b])[None], ref["conf"][None], TOL["bf16"]["conf"], f"{tag} conf")
        assert_float(to_np(out["entropy"][b]), ref["entropy"], "bf16", "entropy", f"{tag} entropy")
        if check_sc:
            assert_row_rel(to_np(out["sc_out"][b]), ref["sc_out"], TOL["bf16"]["sc_out"], f"{tag} sc_out")
        nt = oracle.argmax_near_ties(ref["logits"], TIE_EPS["bf16"])
        if max_excused is not None:
            assert nt.fraction < max_excused, f"{tag}: {nt.fraction:.2f} of argmax excused"
        bad = (to_np(out["argmax"][b]) != ref["argmax"]) & ~nt.mask
        assert not bad.any(), f"{tag} argmax at {np.nonzero(bad)[0][:8]}"


def _commit_compare(inp, out, cm, refs, canvases, label):
    mask_id, tau = inp["dims"].mask_id, inp["tau"]
    gm_all = to_np(cm["mask"])
    go_all = to_np(cm["out_ids"])
    excused = 0.0
    for i, b in enumerate(canvases):
        ref = refs[i]
        ids = inp["canvas_ids"][b]
        m, o, n = oracle.commit_canvas(ids, ref["conf"], ref["entropy"], ref["argmax"], mask_id, tau)
        near = oracle.commit_near_ties(ids, ref["conf"], ref["entropy"], mask_id, tau,
                                       conf_eps=TIE_EPS["bf16"])
        am_near = oracle.argmax_near_ties(ref["logits"], TIE_EPS["bf16"]).mask
        assert np.array_equal(gm_all[b][~near], m[~near]), f"{label} commit mask canvas {b}"
        ok = ~near & ~(am_near & (m == 1))
        assert np.array_equal(go_all[b][ok], o[ok]), f"{label} commit ids canvas {b}"
        excused += near.mean()
        # the GPU's own decision is the rule applied to its own confidences and entropies
        gm2, _, _ = oracle.commit_canvas(ids, to_np(out["conf"][b]).astype(np.float64),
                                         to_np(out["entropy"][b]).astype(np.float64),
                                         to_np(out["argmax"][b]), mask_id, tau)
        near2 = oracle.commit_near_ties(ids, to_np(out["conf"][b]), to_np(out["entropy"][b]),
                                        mask_id, tau, conf_eps=0.0)
        assert np.array_equal(gm_all[b][~near2], gm2[~near2]), f"{label} self-consistency {b}"
    return excused / len(canvases)


def test_headline_step_commit_read_full(torch_cuda):
    """bf16 headline workload at full size: d 2816, 8/2 x 512 heads, 2048 prompt keys,
    W 128, V 262,144: step with self-conditioning, commit (tau 2.0) and the 8-slot
    read with 4 noise draws, exactly as the bench runs them."""
    import torch
    from slot_readout_amd.runtime import DeviceProblem
    inp = make_inputs(config("bf16_step"))
    dev = DeviceProblem(inp)
    out = dev.step(want_sc=True)
    cm = dev.commit(out["conf"], out["entropy"], out["argmax"])
    rd = dev.slot_read()
    torch.cuda.synchronize()
    g_read = {k: to_np(v) for k, v in rd.items()}
    refs = oracle.denoise_step(inp, need_logits=True)
    _step_compare(inp, out, refs, [0], "headline")
    _commit_compare(inp, out, cm, refs, [0], "headline")
    assert int(cm["n"][0]) >= 1
    from tests.test_gpu_slot import _check_slots
    del refs
    ref_read = oracle.slot_read(inp)
    _check_slots(g_read, ref_read, inp, "bf16", "headline read")


def test_ragged32_full(torch_cuda):
    """32 canvases, prompts U{512..8192}, mask fractions U(0.1, 0.9): step + commit."""
    import torch
    from slot_readout_amd.runtime import DeviceProblem
    inp = make_inputs(config("ragged32"))
    dev = DeviceProblem(inp)
    out = dev.step(want_sc=True, debug=False)
    cm = dev.commit(out["conf"], out["entropy"], out["argmax"])
    torch.cuda.synchronize()
    refs = oracle.denoise_step(inp, need_logits=True)
    _step_compare(inp, out, refs, range(32), "ragged32")
    _commit_compare(inp, out, cm, refs, range(32), "ragged32")


def test_ragged32_companion_commit(torch_cuda):
    """Same batch with peaked/flat companion rows so argmax and commit order are real."""
    import torch
    from slot_readout_amd.runtime import DeviceProblem
    inp = make_inputs(config("ragged32"))
    rs = companion_row_scale(inp, (32, 256))
    dev = DeviceProblem(inp, with_embed_t=False)
    out = dev.step(want_sc=False, row_scale=torch.from_numpy(rs).cuda())
    cm = dev.commit(out["conf"], out["entropy"], out["argmax"])
    torch.cuda.synchronize()
    refs = oracle.denoise_step(inp, row_scale=rs, need_sc=False, need_logits=True)
    _step_compare(inp, out, refs, range(32), "ragged32 companion", check_sc=False, max_excused=0.5)
    excused = _commit_compare(inp, out, cm, refs, range(32), "ragged32 companion")
    assert excused < 0.5


def test_long_read_full(torch_cuda):
    """One canvas over a 110,707-token cached prompt (W 128): step + commit."""
    import torch
    from slot_readout_amd.runtime import DeviceProblem
    inp = make_inputs(config("long_read"))
    dev = DeviceProblem(inp)
    out = dev.step(want_sc=True, debug=True)
    cm = dev.commit(out["conf"], out["entropy"], out["argmax"])
    torch.cuda.synchronize()
    refs = oracle.denoise_step(inp, need_logits=True)
    assert_row_rel(to_np(out["attn_out"][0]), refs[0]["attn_out"], TOL["bf16"]["attn_out"], "long attn_out")
    _step_compare(inp, out, refs, [0], "long_read")
    _commit_compare(inp, out, cm, refs, [0], "long_read")


def test_reads512_full(torch_cuda):
    """512 canvases x 4 slots, k ~ U{2..26}, 1024-token prompts, 4 noise draws."""
    import torch
    from slot_readout_amd.runtime import DeviceProblem
    inp = make_inputs(config("reads512"))
    dev = DeviceProblem(inp, with_embed_t=False)
    g = {k: to_np(v) for k, v in dev.slot_read().items()}
    torch.cuda.synchronize()
    ref = oracle.slot_read(inp)
    from tests.test_gpu_slot import _check_slots
    _check_slots(g, ref, inp, "bf16", "reads512")


def test_read_batch_f32_mixed_rereads(torch_cuda):
    """Read-batch shape (1024-token prompts, 4 slots, k ~ U{2..26}) in fp32 storage
    with per-slot logit multipliers: a real mix of confident single reads and
    averaged re-reads, checked at the fp32 bar (1e-4 relative)."""
    import torch
    from slot_readout_amd.runtime import DeviceProblem
    inp = make_inputs(config("reads512", dtype="f32"), batch=64)
    rs = companion_row_scale(inp, (64, 4), 64.0, 2048.0)
    dev = DeviceProblem(inp, with_embed_t=False)
    g = {k: to_np(v) for k, v in dev.slot_read(row_scale=torch.from_numpy(rs).cuda()).items()}
    torch.cuda.synchronize()
    ref = oracle.slot_read(inp, row_scale=rs)
    from tests.test_gpu_slot import _check_slots
    _check_slots(g, ref, inp, "f32", "read batch f32 companion")
    du = ref["draws_used"]
    assert (du == 1).mean() > 0.05 and (du == 4).mean() > 0.05


def test_headline_step_companion_full(torch_cuda):
    """The headline step at full size (d 2816, 8/2 x 512 heads, 2048 prompt keys,
    W 128, V 262,144) with per-row logit multipliers logUniform(0.5, 32): flat
    rows (H near ln V) and peaked ones, so argmax and the commit order are real
    decisions.  Compared elementwise: attention output and hidden state of
    every row, the logits of 16 rows (the 8 flattest and 8 sharpest), conf,
    entropy, argmax and p.E of every row, then the commit (tau 2.0) with the
    declared near-tie fraction below one half."""
    import torch
    from slot_readout_amd.runtime import DeviceProblem
    inp = make_inputs(config("bf16_step"))
    rs = companion_row_scale(inp, (1, 256), 0.5, 32.0)
    dev = DeviceProblem(inp)
    out = dev.step(want_sc=True, debug=True, row_scale=torch.from_numpy(rs).cuda())
    cm = dev.commit(out["conf"], out["entropy"], out["argmax"])
    torch.cuda.synchronize()
    ref = oracle.denoise_step(inp, row_scale=rs, need_logits=True)[0]
    H = ref["entropy"]
    assert (H < 1).mean() > 0.1 and (H > 6).mean() > 0.1
    assert_row_rel(to_np(out["attn_out"][0]), ref["attn_out"], TOL["bf16"]["attn_out"], "attn_out")
    assert_row_rel(to_np(out["hidden_out"][0]), ref["hidden_out"], TOL["bf16"]["hidden_out"], "hidden_out")
    order = np.argsort(H, kind="stable")
    rows = np.concatenate([order[:8], order[-8:]])
    g_l = to_np(out["logits"][0, torch.from_numpy(rows).cuda()])
    assert_row_rel(g_l, ref["logits"][rows], TOL["bf16"]["logits"], "logits (16 rows)")
    del g_l
    out["logits"] = None
    _step_compare(inp, out, [ref], [0], "headline companion", max_excused=0.5)
    excused = _commit_compare(inp, out, cm, [ref], [0], "headline companion")
    assert excused < 0.5
    assert int(cm["n"][0]) >= 2


@pytest.mark.parametrize("full_canvas", [False, True])
def test_headline_read_peaked_full(torch_cuda, full_canvas):
    """The headline read at full size (V 262,144; the draws ride in the first
    read's pass) with per-slot logit multipliers logUniform(8, 128): label
    logprobs down to about -110, some slots confident enough to stop at the
    first read and others re-read with 4 draws (the threshold sits in the
    widest gap of the first-read entropies).  bf16 at the absolute 1e-2
    logprob bar."""
    import torch
    from slot_readout_amd.runtime import DeviceProblem
    from tests.test_gpu_slot import _check_slots, _one_pass_draws
    inp = make_inputs(config("bf16_step"))
    S = inp["slot_pos"].shape[1]
    assert _one_pass_draws(inp["dims"], 1, S, inp["n_draws"], int(inp["max_prompt"]))
    rs = companion_row_scale(inp, (1, S), 8.0, 128.0)
    inp["entropy_threshold"] = 1e9
    first = oracle.slot_read(inp, row_scale=rs, n_draws=1)["first_entropy"][0]
    top = np.sort(first)
    gaps = np.diff(top)
    i = int(np.argmax(gaps))
    assert gaps[i] > 4 * TOL["bf16"]["entropy_abs"], top
    inp["entropy_threshold"] = float((top[i] + top[i + 1]) / 2)
    ref = oracle.slot_read(inp, row_scale=rs)
    du = ref["draws_used"]
    assert (du == 1).any() and (du == 4).any(), du
    assert ref["logprobs"].min() < -60
    dev = DeviceProblem(inp, with_embed_t=False)
    g = {k: to_np(v) for k, v in dev.slot_read(row_scale=torch.from_numpy(rs).cuda(),
                                                full_canvas=full_canvas).items()}
    torch.cuda.synchronize()
    _check_slots(g, ref, inp, "bf16", f"headline peaked read (full canvas {full_canvas})",
                 max_excused=0.5)
