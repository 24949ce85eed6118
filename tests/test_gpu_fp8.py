"""GPU parity of the e4m3 (FP8) LM head: dg_prepare_lm_fp8's codes and
exponents bit-exact against the oracle's own quantisation, then the denoise
step and the slot read with the FP8 head against the oracle run with the
decoded head (weight-only FP8: bf16 activations, fp32 accumulation)."""
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


def _bf16_exact(x):
    """float32 values that are exactly representable in bf16"""
    u = np.asarray(x, np.float32).view(np.uint32) & np.uint32(0xFFFF0000)
    return u.view(np.float32)


def _inputs_with_edge_rows(name, **over):
    """The workload's inputs with a zero row, a row of exact rounding ties and a
    row spanning subnormal codes placed in the embedding (the tied head)."""
    inp = make_inputs(config(name, **over), prompt_override=("fixed", 128))
    E = inp["embed"].copy()
    d = E.shape[1]
    E[5] = 0.0
    # row 6: amax 448 (exponent 0); values halfway between neighbouring codes
    ties = np.array([1.0625, 1.1875, 3 * 2.0 ** -10, 2.0 ** -10, 448.0, -2.125], np.float32)
    E[6] = np.resize(ties, d)
    # row 7: a wide dynamic range, so small entries land on subnormal codes
    E[7] = _bf16_exact(np.geomspace(1e-6, 1.0, d) * np.where(np.arange(d) % 2, -1, 1))
    inp["embed"] = E.astype(E.dtype)
    return inp


@pytest.mark.parametrize("name,over", [("bf16_step", dict(vocab=4096, mask_id=4095)), ("ragged32", {})])
def test_prepare_codes_match_the_oracle(torch_cuda, name, over):
    from slot_readout_amd.runtime import DeviceProblem
    inp = _inputs_with_edge_rows(name, **over)
    dev = DeviceProblem(inp, with_lm_fp8=True)
    torch_cuda.cuda.synchronize()
    codes, exps = oracle.quantize_head_e4m3(inp["embed"])
    g_codes, g_exps = to_np(dev.lm_fp8), to_np(dev.lm_fp8_exp)
    np.testing.assert_array_equal(g_exps, exps)
    bad = np.nonzero(g_codes != codes)
    assert bad[0].size == 0, f"codes differ at {list(zip(bad[0][:5], bad[1][:5]))}"
    assert exps[5] == 0 and not g_codes[5].any()


def test_step_with_fp8_head(torch_cuda):
    """Headline dims with a 4096 vocabulary, peaked and flat rows (companion
    scales): every step output against the oracle step with the decoded head."""
    import torch
    from slot_readout_amd.runtime import DeviceProblem
    from tests.test_gpu_step import _check_step
    inp = make_inputs(config("bf16_step", vocab=4096, mask_id=4095), prompt_override=("fixed", 200))
    rs = companion_row_scale(inp, (1, 256))
    dev = DeviceProblem(inp, with_lm_fp8=True)
    out = dev.step(row_scale=torch.from_numpy(rs).cuda(), debug=True)
    torch.cuda.synchronize()
    codes, exps = oracle.quantize_head_e4m3(inp["embed"])
    ref_inp = dict(inp, lm_head=oracle.dequantize_head_e4m3(codes, exps))
    refs = oracle.denoise_step(ref_inp, row_scale=rs, need_logits=True)
    _check_step(ref_inp, out, refs, "bf16", label="fp8 head")


def test_slot_read_with_fp8_head(torch_cuda):
    """Few-row LM head of the read (first read + 4 draws) with the FP8 head."""
    import torch
    from slot_readout_amd.runtime import DeviceProblem
    from tests.test_gpu_slot import _check_slots
    inp = make_inputs(config("reads512"), batch=6, prompt_override=("fixed", 120))
    dev = DeviceProblem(inp, with_embed_t=False, with_lm_fp8=True)
    out = dev.slot_read()
    torch.cuda.synchronize()
    g = {k: to_np(v) for k, v in out.items()}
    codes, exps = oracle.quantize_head_e4m3(inp["embed"])
    ref_inp = dict(inp, lm_head=oracle.dequantize_head_e4m3(codes, exps))
    ref = oracle.slot_read(ref_inp)
    _check_slots(g, ref, ref_inp, "bf16", "fp8 head")


# --------------------------------------------------- FP8 activations ------
def _fp8_act_inputs(vocab):
    """Headline dims with the given vocabulary and an output projection of zeros,
    so that h = x = E[id] exactly (bf16 values) on both sides: the GPU and the
    oracle then quantise the same h, and the FP8 LM head is compared alone.
    Canvas rows at ids 5, 6, 7 and an out-of-range id give h rows of zeros, of
    exact rounding ties and of subnormal codes."""
    inp = _inputs_with_edge_rows("bf16_step", vocab=vocab, mask_id=vocab - 1)
    E = inp["embed"]
    E[6] = E[6] * np.float32(2.0 ** -14)      # ties kept: the row exponent moves by -14
    inp["embed"] = E
    inp["wo"] = np.zeros_like(inp["wo"])
    ids = inp["canvas_ids"]
    ids[0, 10], ids[0, 11], ids[0, 12], ids[0, 13] = 5, 6, 7, vocab + 3
    return inp


def test_step_fp8_activations_exact_hidden_rows(torch_cuda):
    """FP8 activations with h known exactly on both sides: the GPU's codes equal
    the oracle's, the products are exact in fp32, so the logits and the
    softmax statistics meet the fp32 bars; p.E (bf16 probabilities) the bf16 bar."""
    import torch
    from slot_readout_amd.runtime import DeviceProblem
    from tests.helpers import TOL, TIE_EPS, assert_row_rel, assert_float, row_rel_fail
    inp = _fp8_act_inputs(32768)
    # h = E[id] makes each row's own id stand out by |E[id]|^2 ~ 1.1: total
    # logit scales of 0.5 .. 32 give both flat and peaked rows
    rs = companion_row_scale(inp, (1, 256), lo=0.5, hi=32.0)
    dev = DeviceProblem(inp, with_lm_fp8=True, lm_fp8_act=True)
    out = dev.step(row_scale=torch.from_numpy(rs).cuda(), debug=True)
    torch.cuda.synchronize()
    assert int(out["flags"].item()) == 1      # the out-of-range id
    codes, exps = oracle.quantize_head_e4m3(inp["embed"])
    ref_inp = dict(inp, lm_head=oracle.dequantize_head_e4m3(codes, exps))
    ref = oracle.denoise_step(ref_inp, row_scale=rs, need_logits=True, act_fp8=True)[0]
    h = to_np(out["hidden_out"][0])
    np.testing.assert_array_equal(h, ref["hidden_out"])
    assert not h[13].any()
    f32 = TOL["f32"]
    # the fp32 bar, or the worst-case bound of a d-term fp32 sum of exact products,
    # d 2^-24 s sum_k |h_k E_vk| (the matrix cores' own order of addition)
    gl = to_np(out["logits"][0]).astype(np.float64)
    s = inp["logit_scale"] * rs[0].astype(np.float64)[:, None]
    hq = oracle.fp8_activations(ref["hidden_out"])
    absum = np.abs(hq) @ np.abs(ref_inp["lm_head"]).T * s
    d = hq.shape[1]
    fail = row_rel_fail(gl, ref["logits"], f32["logits"]) & (np.abs(gl - ref["logits"]) > d * 2.0 ** -24 * absum)
    assert not fail.any(), f"fp8 act logits at {np.argwhere(fail)[:5].tolist()}"
    assert row_rel_fail(gl, ref["logits"], f32["logits"]).mean() < 1e-4
    assert_row_rel(to_np(out["conf"][0])[None], ref["conf"][None], f32["conf"], "fp8 act conf")
    assert_float(to_np(out["entropy"][0]), ref["entropy"], "f32", "entropy", "fp8 act entropy")
    assert_row_rel(to_np(out["sc_out"][0]), ref["sc_out"], TOL["bf16"]["sc_out"], "fp8 act sc_out")
    near = oracle.argmax_near_ties(ref["logits"], TIE_EPS["f32"]).mask
    bad = (to_np(out["argmax"][0]) != ref["argmax"]) & ~near
    assert not bad.any(), f"argmax at {np.nonzero(bad)[0][:8]}"
    H = ref["entropy"]
    assert (H < 1).mean() > 0.05 and (H > 6).mean() > 0.05
    # the zero row: every logit 0, a uniform distribution
    assert np.all(to_np(out["logits"][0][13]) == 0)


# One e4m3 step of a normal value is at most 2^-3 of it.  The GPU's h differs
# from the oracle's by bf16 rounding (far below a step), so each of the GPU's
# codes lies within one step of the oracle's; a logit moved by one step in every
# element of h is at most 2^-3 of |h| . |E| row-wise, which bounds the bar
# below (row-relative, as the other logit bars).
FP8_ACT_LOGIT_RTOL = 2.0 ** -3


def test_step_fp8_activations_full_block(torch_cuda):
    """The whole step with FP8 activations (real output projection): logits
    within one e4m3 step of the oracle's FP8-activation logits, the softmax
    statistics and p.E consistent with the GPU's own logits (properties at
    any size), attention and hidden state at the bf16 bars."""
    import torch
    from slot_readout_amd.runtime import DeviceProblem
    from tests.helpers import TOL, assert_row_rel
    inp = make_inputs(config("bf16_step", vocab=4096, mask_id=4095), prompt_override=("fixed", 200))
    rs = companion_row_scale(inp, (1, 256))
    dev = DeviceProblem(inp, with_lm_fp8=True, lm_fp8_act=True)
    out = dev.step(row_scale=torch.from_numpy(rs).cuda(), debug=True)
    torch.cuda.synchronize()
    assert int(out["flags"].item()) == 0
    codes, exps = oracle.quantize_head_e4m3(inp["embed"])
    ref_inp = dict(inp, lm_head=oracle.dequantize_head_e4m3(codes, exps))
    ref = oracle.denoise_step(ref_inp, row_scale=rs, need_logits=True, act_fp8=True)[0]
    bf = TOL["bf16"]
    assert_row_rel(to_np(out["attn_out"][0]), ref["attn_out"], bf["attn_out"], "attn_out")
    assert_row_rel(to_np(out["hidden_out"][0]), ref["hidden_out"], bf["hidden_out"], "hidden_out")
    gl = to_np(out["logits"][0]).astype(np.float64)
    assert_row_rel(gl, ref["logits"], FP8_ACT_LOGIT_RTOL, "fp8 act logits")
    # the bar is far from the typical error: most logits agree to a few percent of it
    err = np.abs(gl - ref["logits"]) / np.sqrt(np.mean(ref["logits"] ** 2, axis=1, keepdims=True))
    assert np.median(err) < FP8_ACT_LOGIT_RTOL / 8
    # conf, entropy, argmax and p.E as functions of the GPU's logits
    st = oracle.vocab_softmax(gl)
    f32 = TOL["f32"]
    assert_row_rel(to_np(out["conf"][0])[None], st.conf[None], f32["conf"], "conf vs own logits")
    # fp32 statistics of fp32 logits: the fp32 bar, plus 2^-20 absolute for the
    # cancellation of lse - sum p l at near-zero entropy
    gH = to_np(out["entropy"][0]).astype(np.float64)
    bad = np.abs(gH - st.entropy) > f32["entropy_abs"] * st.entropy + 2.0 ** -20
    assert not bad.any(), f"entropy vs own logits at {np.nonzero(bad)[0][:8]}: {gH[bad][:4]} vs {st.entropy[bad][:4]}"
    near = oracle.argmax_near_ties(gl, 1e-5).mask
    bad = (to_np(out["argmax"][0]) != st.argmax) & ~near
    assert not bad.any(), f"argmax vs own logits at {np.nonzero(bad)[0][:8]}"
    sc = oracle.self_condition(st.p, inp["embed"])
    assert_row_rel(to_np(out["sc_out"][0]), sc, bf["sc_out"], "sc_out vs own logits")
