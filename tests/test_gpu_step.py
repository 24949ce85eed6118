"""GPU parity of dg_denoise_step and dg_commit against the CPU oracle, through the
C-ABI, on seeded inputs at sizes the oracle finishes in seconds."""
import numpy as np
import pytest

import oracle
from synth import config, make_inputs, companion_row_scale
from tests.helpers import TOL, TIE_EPS, to_np, assert_row_rel, assert_float

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def torch_cuda():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch


def _problem(inp):
    from slot_readout_amd.runtime import DeviceProblem
    return DeviceProblem(inp)


def _check_step(inp, out, refs, dtype, row_scale=None, label=""):
    """Compare every step output of every canvas with the oracle."""
    tol = TOL[dtype]
    for b, ref in enumerate(refs):
        tag = f"{label} canvas {b}"
        assert_row_rel(to_np(out["attn_out"][b]), ref["attn_out"], tol["attn_out"], f"{tag} attn_out")
        assert_row_rel(to_np(out["hidden_out"][b]), ref["hidden_out"], tol["hidden_out"], f"{tag} hidden_out")
        assert_row_rel(to_np(out["logits"][b]), ref["logits"], tol["logits"], f"{tag} logits")
        assert_row_rel(to_np(out["conf"][b])[None], ref["conf"][None], tol["conf"], f"{tag} conf")
        assert_float(to_np(out["entropy"][b]), ref["entropy"], dtype, "entropy", f"{tag} entropy")
        if out.get("sc_out") is not None:
            assert_row_rel(to_np(out["sc_out"][b]), ref["sc_out"], tol["sc_out"], f"{tag} sc_out")
        near = oracle.argmax_near_ties(ref["logits"], TIE_EPS[dtype]).mask
        g_am = to_np(out["argmax"][b])
        bad = (g_am != ref["argmax"]) & ~near
        assert not bad.any(), f"{tag} argmax differs at {np.nonzero(bad)[0][:8]} (near-ties {near.mean():.3f})"


def test_step_tiny_f32(torch_cuda):
    """Tiny fp32 workload: 128 prompt keys, canvas 256, d 256, 4x64 heads, W 16, V 2048."""
    inp = make_inputs(config("tiny_f32"))
    dev = _problem(inp)
    out = dev.step(debug=True)
    torch_cuda.cuda.synchronize()
    assert int(out["flags"].item()) == 0
    refs = oracle.denoise_step(inp, need_logits=True)
    _check_step(inp, out, refs, "f32", label="tiny_f32")


def test_step_tiny_f32_sc_in_row_scale(torch_cuda):
    inp = make_inputs(config("tiny_f32"), with_sc_in=True)
    rs = companion_row_scale(inp, (1, 256))
    dev = _problem(inp)
    import torch
    sc = torch.from_numpy(inp["sc_in"]).cuda()
    rst = torch.from_numpy(rs).cuda()
    out = dev.step(sc_in=sc, row_scale=rst, debug=True)
    torch.cuda.synchronize()
    refs = oracle.denoise_step(inp, sc_in=inp["sc_in"], row_scale=rs, need_logits=True)
    _check_step(inp, out, refs, "f32", label="tiny_f32+sc+rows")
    # the companion scales give a real mix of peaked and flat rows
    H = refs[0]["entropy"]
    assert (H < 1).mean() > 0.1 and (H > 6).mean() > 0.1


def test_commit_exact_on_shared_inputs(torch_cuda):
    """dg_commit vs the oracle commit on identical fp32 confidences/entropies:
    bit-exact except ranks whose entropy prefix lies within 1e-3 of tau."""
    import torch
    rng = np.random.default_rng(11)
    B, C = 6, 256
    ids = rng.integers(0, 50, size=(B, C)).astype(np.int32)
    mask_id = 7
    ids[rng.uniform(size=(B, C)) < 0.5] = mask_id
    conf = rng.uniform(size=(B, C)).astype(np.float32)
    conf[:, ::9] = conf[:, 1::9][:, :conf[:, ::9].shape[1]]  # exact ties between positions
    ent = rng.exponential(0.05, size=(B, C)).astype(np.float32)
    am = rng.integers(0, 1000, size=(B, C)).astype(np.int32)
    ids[5, :] = 3                                         # a canvas with no candidates
    for tau in (0.0, 0.3, 1.0, 2.0, 1e30):
        g_mask = torch.empty((B, C), dtype=torch.uint8, device="cuda")
        g_out = torch.from_numpy(ids.copy()).cuda()        # in-place commit (aliasing allowed)
        g_n = torch.empty(B, dtype=torch.int32, device="cuda")
        from slot_readout_amd import dg
        dg.dg_commit(B, C, mask_id, g_out, torch.from_numpy(conf).cuda(),
                     torch.from_numpy(ent).cuda(), torch.from_numpy(am).cuda(), tau, g_mask, g_out, g_n)
        torch.cuda.synchronize()
        m, o, n = oracle.commit(ids, conf.astype(np.float64), ent.astype(np.float64), am, mask_id, tau)
        for b in range(B):
            near = oracle.commit_near_ties(ids[b], conf[b], ent[b], mask_id, tau, conf_eps=0.0)
            gm = to_np(g_mask[b])
            assert np.array_equal(gm[~near], m[b][~near]), (tau, b)
            assert np.array_equal(to_np(g_out[b])[~near], o[b][~near]), (tau, b)
            if not near.any():
                assert int(g_n[b]) == n[b]
        assert int(g_n[5]) == 0


def test_step_then_commit_companion(torch_cuda):
    """End to end: GPU step + GPU commit vs oracle step + oracle commit, with the
    oracle's declared near-ties excused; the companion row scales make the
    ordering meaningful."""
    import torch
    inp = make_inputs(config("tiny_f32"))
    rs = companion_row_scale(inp, (1, 256))
    dev = _problem(inp)
    out = dev.step(row_scale=torch.from_numpy(rs).cuda(), want_sc=False)
    cm = dev.commit(out["conf"], out["entropy"], out["argmax"])
    torch.cuda.synchronize()
    ref = oracle.denoise_step(inp, row_scale=rs, need_sc=False, need_logits=True)[0]
    ids = inp["canvas_ids"][0]
    m, o, n = oracle.commit_canvas(ids, ref["conf"], ref["entropy"], ref["argmax"],
                                   inp["dims"].mask_id, inp["tau"])
    near = oracle.commit_near_ties(ids, ref["conf"], ref["entropy"], inp["dims"].mask_id,
                                   inp["tau"], conf_eps=TIE_EPS["f32"])
    am_near = oracle.argmax_near_ties(ref["logits"], TIE_EPS["f32"]).mask
    assert oracle.argmax_near_ties(ref["logits"], TIE_EPS["f32"]).fraction < 0.5
    gm = to_np(cm["mask"][0])
    assert np.array_equal(gm[~near], m[~near])
    ok_ids = ~near & ~(am_near & (m == 1))
    assert np.array_equal(to_np(cm["out_ids"][0])[ok_ids], o[ok_ids])
    assert n >= 1 and near.mean() < 0.5


@pytest.mark.parametrize("B,prompt", [(3, ("uniform", 0, 300)), (1, ("fixed", 0))])
def test_step_tiny_bf16_ragged(torch_cuda, B, prompt):
    """Tiny dims in bf16 with ragged prompt lengths (including empty prompts)."""
    import torch
    cfg = config("ragged32")
    inp = make_inputs(cfg, batch=B, prompt_override=prompt, with_sc_in=True)
    dev = _problem(inp)
    out = dev.step(sc_in=torch.from_numpy(inp["sc_in"]).to(torch.bfloat16).cuda(), debug=True)
    torch.cuda.synchronize()
    refs = oracle.denoise_step(inp, sc_in=inp["sc_in"], need_logits=True)
    _check_step(inp, out, refs, "bf16", label=f"bf16 B{B}")


def test_step_wide_heads_small_vocab(torch_cuda):
    """Headline dims (d 2816, 8 q / 2 kv heads x 512, W 128) with the vocabulary
    cut to 4096 and 300 prompt keys so the oracle runs in seconds."""
    cfg = config("bf16_step", vocab=4096, mask_id=4095)
    inp = make_inputs(cfg, prompt_override=("fixed", 300))
    dev = _problem(inp)
    out = dev.step(debug=True)
    import torch
    torch.cuda.synchronize()
    refs = oracle.denoise_step(inp, need_logits=True)
    _check_step(inp, out, refs, "bf16", label="wide-heads")


def test_step_deterministic(torch_cuda):
    """Two runs of the same step give bitwise-identical outputs."""
    import torch
    inp = make_inputs(config("ragged32"), batch=2, prompt_override=("uniform", 100, 700))
    dev = _problem(inp)
    a = dev.step(debug=True)
    b = dev.step(debug=True)
    torch.cuda.synchronize()
    for k in ("conf", "entropy", "argmax", "sc_out", "attn_out", "hidden_out", "logits"):
        assert torch.equal(a[k], b[k]), k


def test_blocked_lm_head_matches_row_major(torch_cuda):
    """The LM head read from its 256 x 32 blocked copy (dg_prepare_lm_tiled) gives
    bitwise the same step and slot-read outputs as the row-major head: the same
    MFMAs over the same K order, only the addresses differ.  Covers the 256-row
    tile (the step) and the few-row tile (the read)."""
    from slot_readout_amd.runtime import DeviceProblem
    cfg = config("bf16_step", vocab=4096, mask_id=4095)
    inp = make_inputs(cfg, prompt_override=("fixed", 200))
    outs = []
    for tiled in (True, False):
        dev = DeviceProblem(inp, with_lm_tiled=tiled)
        assert (dev.lm_tiled is not None) == tiled
        st = dev.step(want_sc=True)
        rd = dev.slot_read()
        torch_cuda.cuda.synchronize()
        outs.append({**{"step_" + k: to_np(v) for k, v in st.items()},
                     **{"read_" + k: to_np(v) for k, v in rd.items()}})
    for k in outs[0]:
        assert np.array_equal(outs[0][k], outs[1][k]), k


def test_blocked_self_conditioning_matches_row_major(torch_cuda):
    """p.E read from the 256 x 32 blocked embed^T (dg_prepare_embed_t_tiled) gives
    bitwise the same sc_out as the row-major embed^T: the same MFMAs in the same
    K order, only the addresses differ."""
    from slot_readout_amd.runtime import DeviceProblem
    cfg = config("bf16_step", vocab=4096, mask_id=4095)
    inp = make_inputs(cfg, prompt_override=("fixed", 200))
    outs = []
    for tiled in (True, False):
        dev = DeviceProblem(inp, with_embed_t_tiled=tiled)
        assert (dev.embed_t_tiled is not None) == tiled
        st = dev.step(want_sc=True)
        torch_cuda.cuda.synchronize()
        outs.append({k: to_np(v) for k, v in st.items()})
    for k in outs[0]:
        assert np.array_equal(outs[0][k], outs[1][k]), k


def test_step_bf16_partial_row_block(torch_cuda):
    """bf16 canvases whose rows do not fill the last 256-row block of p~
    (2 x 200 rows): every output, sc_out included, against the oracle."""
    inp = make_inputs(config("ragged32", batch=2, canvas=200),
                      prompt_override=("uniform", 100, 300))
    dev = _problem(inp)
    assert dev.embed_t_tiled is not None
    out = dev.step(debug=True)
    torch_cuda.cuda.synchronize()
    refs = oracle.denoise_step(inp, need_logits=True)
    _check_step(inp, out, refs, "bf16", label="ragged 2x200")


@pytest.mark.parametrize("name,n_kv,B", [("tiny_f32", 1, 1), ("tiny_f32", 2, 2), ("ragged32", 2, 3)])
def test_step_gqa_head_dim_64(torch_cuda, name, n_kv, B):
    """Grouped kv heads at head_dim 64 (4 q heads over 1 or 2 kv heads), every
    canvas position queried, in fp32 and bf16 (ragged prompts for bf16)."""
    import torch
    prompt = ("uniform", 0, 300) if name == "ragged32" else ("fixed", 128)
    inp = make_inputs(config(name, n_kv_heads=n_kv), batch=B, prompt_override=prompt)
    dev = _problem(inp)
    out = dev.step(debug=True)
    torch.cuda.synchronize()
    assert int(out["flags"].item()) == 0
    refs = oracle.denoise_step(inp, need_logits=True)
    _check_step(inp, out, refs, inp["dims"].dtype, label=f"gqa {name} kv{n_kv} B{B}")
