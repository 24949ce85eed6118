"""Pins of the e4m3 (FP8) head quantisation used by the FP8 LM head, CPU only.

The e4m3 format (OCP 8-bit float: sign, 4 exponent bits with bias 7, 3 mantissa
bits, subnormals, largest finite value 448, no infinities) fixes every decoded
value; the encoder rounds to nearest, ties to even."""
import numpy as np
import pytest

import oracle


@pytest.mark.parametrize("code,value", [
    (0x00, 0.0), (0x01, 2.0 ** -9), (0x07, 7 * 2.0 ** -9), (0x08, 2.0 ** -6),
    (0x38, 1.0), (0x39, 1.125), (0x3F, 1.875), (0x40, 2.0), (0x7E, 448.0),
    (0xB8, -1.0), (0xFE, -448.0), (0x80, -0.0),
])
def test_decode_values_fixed_by_the_format(code, value):
    assert oracle.e4m3_decode([code])[0] == value


def test_every_code_round_trips():
    codes = np.array([c for c in range(256) if (c & 0x7F) != 0x7F])
    back = oracle.e4m3_encode(oracle.e4m3_decode(codes)).astype(np.int64)
    np.testing.assert_array_equal(back, codes)


def test_round_to_nearest_even_and_error_bound():
    # ties between neighbouring codes go to the even mantissa
    assert oracle.e4m3_encode([1.0625])[0] == 0x38        # 1.0 vs 1.125 -> 1.0
    assert oracle.e4m3_encode([1.1875])[0] == 0x3A        # 1.125 vs 1.25 -> 1.25
    assert oracle.e4m3_encode([2.0 ** -10])[0] == 0x00    # 0 vs 2^-9 -> 0
    assert oracle.e4m3_encode([3 * 2.0 ** -10])[0] == 0x02  # 2^-9 vs 2^-8 -> 2^-8
    # brute force: the nearest code, within half a step of the value
    rng = np.random.default_rng(8)
    x = np.concatenate([rng.uniform(-448, 448, 4000), rng.uniform(-0.05, 0.05, 4000)]).astype(np.float32)
    got = oracle.e4m3_decode(oracle.e4m3_encode(x))
    grid = np.unique(oracle.e4m3_decode([c for c in range(256) if (c & 0x7F) != 0x7F]))
    best = grid[np.abs(grid[None, :] - x[:, None].astype(np.float64)).argmin(axis=1)]
    np.testing.assert_array_equal(np.abs(got - x), np.abs(best - x))
    normal = np.abs(x) >= 2.0 ** -6
    assert (np.abs(got - x)[normal] <= 2.0 ** -4 * np.abs(x[normal])).all()
    assert (np.abs(got - x)[~normal] <= 2.0 ** -10).all()


def test_row_exponent_is_the_smallest_that_fits():
    amax = np.array([448.0, 449.0, 1.0, 1.75, 1.76, 3.5e-3, 0.0], dtype=np.float32)
    e = oracle.e4m3_row_exponent(amax)
    np.testing.assert_array_equal(e, [0, 1, -8, -8, -7, -16, 0])
    pos = amax > 0
    assert (amax[pos] <= 448.0 * np.exp2(e[pos])).all()
    assert (amax[pos] > 448.0 * np.exp2(e[pos] - 1.0)).all()


def test_quantized_head_is_within_half_a_step_of_the_head():
    rng = np.random.default_rng(9)
    head = (rng.normal(size=(64, 96)) * 0.02).astype(np.float32)
    head[3] = 0.0
    codes, exps = oracle.quantize_head_e4m3(head)
    deq = oracle.dequantize_head_e4m3(codes, exps)
    assert codes.dtype == np.uint8 and exps[3] == 0 and not deq[3].any()
    scale = np.exp2(exps.astype(np.float64))[:, None]
    q = head / scale
    err = np.abs(deq / scale - q)
    normal = np.abs(q) >= 2.0 ** -6
    assert (err[normal] <= 2.0 ** -4 * np.abs(q[normal])).all()
    assert (err[~normal] <= 2.0 ** -10).all()
    # each row's largest magnitude lands in the top binade: 256 <= |q| <= 448
    qmax = np.abs(q).max(axis=1)[np.arange(64) != 3]
    assert ((qmax > 224) & (qmax <= 448)).all()


# ------------------------------------------------- FP8 activations --------
def test_rows_are_quantised_in_float64_not_float32():
    # 1.0625 + 2^-40 lies just above the tie between 1.0 and 1.125: the nearest
    # code is 1.125.  Through float32 the value would become the tie itself and
    # round to the even code 1.0.
    x = np.array([[1.0625 + 2.0 ** -40, 448.0]])
    codes, e = oracle.quantize_rows_e4m3(x)
    assert e[0] == 0 and codes[0, 0] == 0x39 and codes[0, 1] == 0x7E
    # an amax a hair above 448 needs the next exponent (float32 would round it to 448)
    codes, e = oracle.quantize_rows_e4m3(np.array([[448.0 * (1 + 2.0 ** -40), 1.0]]))
    assert e[0] == 1 and codes[0, 0] == 0x76   # 224 * (1 + tiny) -> 224 = 1.75 * 2^7


def test_fp8_activations_on_the_grid_are_unchanged():
    # rows whose entries are e4m3 values times the row's power of two come back
    # exactly, so the FP8-activation logits equal the plain ones
    rng = np.random.default_rng(12)
    grid = oracle.e4m3_decode(np.arange(0x40, 0x7F))          # 2 .. 448, normal codes
    h = rng.choice(grid, size=(6, 40)) * rng.choice([-1.0, 1.0], size=(6, 40))
    h[:, 0] = 448.0                                            # fixes each row's exponent at 0
    h *= np.exp2(np.arange(-3, 3))[:, None]                    # then 2^-3 .. 2^2
    np.testing.assert_array_equal(oracle.fp8_activations(h), h)
    head = rng.normal(size=(30, 40))
    np.testing.assert_array_equal(oracle.lm_logits(oracle.fp8_activations(h), head, 2.0),
                                  oracle.lm_logits(h, head, 2.0))


def test_fp8_activations_scale_with_powers_of_two_and_stay_within_half_a_step():
    rng = np.random.default_rng(13)
    h = rng.normal(size=(8, 64)) * np.exp2(rng.integers(-12, 6, size=(8, 1)))
    h[2] = 0.0
    q = oracle.fp8_activations(h)
    # a power-of-two scale of a row moves its exponent only: the same codes
    np.testing.assert_array_equal(oracle.fp8_activations(h * 2.0 ** 7), q * 2.0 ** 7)
    np.testing.assert_array_equal(oracle.fp8_activations(-h), -q)
    assert not q[2].any()
    # within half a step: 2^-4 relative for normals of the scaled row, 2^-10 * 2^e below
    codes, e = oracle.quantize_rows_e4m3(h)
    s = np.exp2(e.astype(np.float64))[:, None]
    err = np.abs(q - h) / s
    normal = np.abs(h / s) >= 2.0 ** -6
    assert (err[normal] <= 2.0 ** -4 * np.abs(h / s)[normal]).all()
    assert (err[~normal] <= 2.0 ** -10).all()
    # and the nearest grid point (brute force over every code, per row)
    grid = oracle.e4m3_decode(np.array([c for c in range(256) if (c & 0x7F) != 0x7F]))
    for r in range(8):
        best = grid[np.abs(grid[None, :] - (h[r] / s[r])[:, None]).argmin(axis=1)] * s[r]
        np.testing.assert_array_equal(np.abs(q[r] - h[r]), np.abs(best - h[r]))


def test_denoise_canvas_act_fp8_reads_quantised_rows():
    # the FP8-activation step differs from the plain one only in the LM head input
    from synth import config, make_inputs
    inp = make_inputs(config("tiny_f32"), prompt_override=("fixed", 16))
    plain = oracle.denoise_step(inp, need_logits=True)[0]
    act = oracle.denoise_step(inp, need_logits=True, act_fp8=True)[0]
    np.testing.assert_array_equal(act["hidden_out"], plain["hidden_out"])
    want = oracle.lm_logits(oracle.fp8_activations(plain["hidden_out"]), inp["embed"], inp["logit_scale"])
    np.testing.assert_allclose(act["logits"], want, rtol=0, atol=0)
    assert np.abs(act["logits"] - plain["logits"]).max() > 0
