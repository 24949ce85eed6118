"""Pins of the two-stage structured read oracle (ask_if and answer pinning), CPU only."""
import numpy as np

import oracle
from synth import config, make_inputs, companion_row_scale


def _inp():
    inp = make_inputs(config("tiny_f32", canvas=48), batch=2)
    return inp, companion_row_scale(inp, (2, inp["slot_pos"].shape[1]))


def test_single_stage_is_the_plain_read():
    inp, rs = _inp()
    S = inp["slot_pos"].shape[1]
    a = oracle.slot_read_staged(inp, np.zeros(S, int), np.full(S, -1), np.zeros(S, int), row_scale=rs)
    b = oracle.slot_read(inp, row_scale=rs)
    for k in a:
        np.testing.assert_array_equal(a[k], b[k], err_msg=k)


def test_second_stage_reads_the_pinned_canvas():
    """Stage-1 results equal a plain read of only the stage-1 slots on the canvas
    with the stage-0 best labels written at their positions (and differ from a
    read on the unpinned canvas)."""
    inp, rs = _inp()
    S = inp["slot_pos"].shape[1]
    stage = np.array([0] * (S // 2) + [1] * (S - S // 2))
    st = oracle.slot_read_staged(inp, stage, np.full(S, -1), np.zeros(S, int), row_scale=rs)
    S0, S1 = np.nonzero(stage == 0)[0], np.nonzero(stage == 1)[0]
    first = dict(inp, slot_pos=inp["slot_pos"][:, S0], label_ids=inp["label_ids"][:, S0],
                 n_labels=inp["n_labels"][:, S0], noise_ids=inp["noise_ids"][:, :, S0])
    r0 = oracle.slot_read(first, row_scale=rs[:, S0])
    pinned = inp["canvas_ids"].copy()
    for b in range(inp["batch"]):
        for j, s in enumerate(S0):
            pinned[b, inp["slot_pos"][b, s]] = inp["label_ids"][b, s, r0["best"][b, j]]
    second = dict(inp, canvas_ids=pinned, slot_pos=inp["slot_pos"][:, S1],
                  label_ids=inp["label_ids"][:, S1], n_labels=inp["n_labels"][:, S1],
                  noise_ids=inp["noise_ids"][:, :, S1])
    r1 = oracle.slot_read(second, row_scale=rs[:, S1])
    for k in st:
        np.testing.assert_array_equal(st[k][:, S0], r0[k], err_msg=k)
        np.testing.assert_array_equal(st[k][:, S1], r1[k], err_msg=k)
    unpinned = dict(second, canvas_ids=inp["canvas_ids"])
    r1u = oracle.slot_read(unpinned, row_scale=rs[:, S1])
    assert np.abs(r1u["logprobs"] - r1["logprobs"]).max() > 1e-6


def test_ask_if_skips_slots_whose_condition_fails():
    """A stage-1 slot conditioned on the answer of slot 0 is read exactly when
    slot 0's best label matches, and otherwise reports SLOT_NOT_ASKED with zeros."""
    inp, rs = _inp()
    S = inp["slot_pos"].shape[1]
    stage = np.array([0, 0] + [1] * (S - 2))
    base = oracle.slot_read_staged(inp, stage, np.full(S, -1), np.zeros(S, int), row_scale=rs)
    best0 = base["best"][:, 0]
    ask = np.full(S, -1)
    lab = np.zeros(S, int)
    ask[2], lab[2] = 0, best0[0]          # holds on canvas 0
    ask[3], lab[3] = 0, (best0[1] + 1) % int(inp["n_labels"][1, 0])   # fails on canvas 1
    st = oracle.slot_read_staged(inp, stage, ask, lab, row_scale=rs)
    for b in range(inp["batch"]):
        for s in (2, 3):
            held = best0[b] == lab[s]
            if held:
                assert st["status"][b, s] == oracle.SLOT_OK
                np.testing.assert_array_equal(st["probs"][b, s], base["probs"][b, s])
            else:
                assert st["status"][b, s] == oracle.SLOT_NOT_ASKED
                assert st["best"][b, s] == -1 and not st["probs"][b, s].any()
                assert st["draws_used"][b, s] == 0
    assert st["status"][0, 2] == oracle.SLOT_OK
    assert st["status"][1, 3] == oracle.SLOT_NOT_ASKED
