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
