"""Pins of the oracle's near-tie declarations for argmax and slot-best labels.

The declarations excuse GPU/oracle mismatches of integer decisions that
floating-point rounding can flip (24-ai.news, "vLLM integrates DiffusionGemma",
section "Mechanism for deciding completed tokens": the committed token is the
most confident one).  Each case below sits on one side of the rule's boundary,
so a plausible slip fails at least one of them:
  * |top1| in place of max(1, |top1|) (the floor below magnitude 1);
  * <= in place of < (gaps exactly at the width, all exactly representable);
  * the wrong axis or the first two entries instead of the top two;
  * slot labels past n_labels, k = 1 slots, 3-D probability arrays.
"""
import numpy as np

from oracle import dg_oracle as O


# ------------------------------------------------------------ argmax -------
def test_argmax_gap_just_under_and_over_width():
    eps = 1e-2
    # |top1| = 10 > 1: width 0.1
    rows = np.array([[0.0, 10.0, 10.0 - 0.099, -3.0],
                     [0.0, 10.0, 10.0 - 0.101, -3.0]])
    nt = O.argmax_near_ties(rows, eps)
    assert list(nt.mask) == [True, False]
    assert nt.fraction == 0.5


def test_argmax_width_floor_below_magnitude_one():
    eps = 1e-2
    # |top1| = 0.5 < 1: the width is eps * 1 = 0.01, not eps * 0.5 = 0.005
    rows = np.array([[0.5, 0.5 - 0.008, 0.1],
                     [0.5, 0.5 - 0.012, 0.1]])
    assert list(O.argmax_near_ties(rows, eps).mask) == [True, False]


def test_argmax_width_uses_magnitude_of_negative_top1():
    eps = 1e-2
    # top1 = -10: width eps * |top1| = 0.1 (a signed width would be negative)
    rows = np.array([[-10.0, -10.09, -30.0],
                     [-10.0, -10.11, -30.0]])
    assert list(O.argmax_near_ties(rows, eps).mask) == [True, False]


def test_argmax_gap_equal_to_width_is_not_excused():
    # every value exactly representable: width 4 * 2^-6 = 2^-4, gap 2^-4
    eps = 2.0 ** -6
    rows = np.array([[4.0, 4.0 - 2.0 ** -4, 0.0],
                     [4.0, 4.0 - 2.0 ** -5, 0.0]])
    assert list(O.argmax_near_ties(rows, eps).mask) == [False, True]


def test_argmax_exact_tie_excused_and_top_two_found_anywhere():
    eps = 1e-4
    # equal maxima (the lowest id wins on the GPU and in the oracle): excused.
    # second row: the runner-up is the last entry, far from the first two
    rows = np.array([[1.0, 3.0, 3.0, 2.0],
                     [1.0, 5.0, 3.0, 5.0 - 1e-5]])
    assert list(O.argmax_near_ties(rows, eps).mask) == [True, True]
    # a gap between the first two entries does not matter, only the top two do
    rows2 = np.array([[7.0, 7.0 - 1e-6, 9.0, 1.0]])
    assert list(O.argmax_near_ties(rows2, eps).mask) == [False]


def test_argmax_rows_not_columns():
    eps = 1e-2
    # row-wise: row 0 tied (gap 0.001 < 0.03), row 1 clear (gap 2), row 2 clear
    # (gap 1). Column-wise the answer would have three entries of another pattern.
    rows = np.array([[3.0, 2.999, 0.0],
                     [0.0, 1.0, 3.0],
                     [2.0, 1.0, 0.0]])
    nt = O.argmax_near_ties(rows, eps)
    assert nt.mask.shape == (3,)
    assert list(nt.mask) == [True, False, False]
    # transposed input: columns become rows, so the declaration changes
    assert list(O.argmax_near_ties(rows.T, eps).mask) == [False, False, False]


# ------------------------------------------------------------ slot best ----
def _probs(rows):
    out = np.zeros((len(rows), O.MAX_LABELS))
    for i, r in enumerate(rows):
        out[i, :len(r)] = r
    return out


def test_best_gap_just_under_and_over_eps():
    eps = 1e-2
    pr = _probs([[0.504, 0.496], [0.506, 0.494]])
    nt = O.best_near_ties(pr, np.array([2, 2]), eps)
    assert list(nt.mask) == [True, False]
    assert nt.fraction == 0.5


def test_best_gap_equal_to_eps_is_not_excused():
    # exactly representable: 0.625 - 0.375 = 0.25 = eps
    pr = _probs([[0.625, 0.375], [0.5625, 0.4375]])
    assert list(O.best_near_ties(pr, np.array([2, 2]), 0.25).mask) == [False, True]


def test_best_single_label_never_excused():
    pr = _probs([[1.0], [1.0]])
    nt = O.best_near_ties(pr, np.array([1, 1]), 0.5)
    assert not nt.mask.any()


def test_best_ignores_entries_past_n_labels_and_sorts():
    eps = 1e-2
    # k = 2: the third entry (0.6, a stale value past the label count) is not a label
    pr = _probs([[0.6, 0.4, 0.6]])
    assert list(O.best_near_ties(pr, np.array([2]), eps).mask) == [False]
    assert list(O.best_near_ties(pr, np.array([3]), eps).mask) == [True]
    # the top two are found in any position
    pr2 = _probs([[0.1, 0.45, 0.01, 0.44]])
    assert list(O.best_near_ties(pr2, np.array([4]), 0.02).mask) == [True]
    assert list(O.best_near_ties(pr2, np.array([4]), 0.005).mask) == [False]


def test_best_three_dimensional_probs():
    eps = 1e-2
    pr = np.zeros((2, 3, O.MAX_LABELS))
    pr[0, 0, :2] = [0.5, 0.5]            # tie
    pr[0, 1, :3] = [0.2, 0.7, 0.1]       # clear
    pr[0, 2, :1] = [1.0]                 # k = 1
    pr[1, 0, :4] = [0.3, 0.3, 0.2, 0.2]  # tie among the top two
    pr[1, 1, :2] = [0.9, 0.1]            # clear
    pr[1, 2, :3] = [0.333, 0.334, 0.333]  # tie
    nl = np.array([[2, 3, 1], [4, 2, 3]])
    nt = O.best_near_ties(pr, nl, eps)
    assert nt.mask.shape == (2, 3)
    assert nt.mask.tolist() == [[True, False, False], [True, False, True]]
    assert nt.fraction == 0.5
