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
