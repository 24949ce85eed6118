"""The seeded input generator: determinism, storage rounding and recipe facts."""
import numpy as np
import torch

from synth import config, make_inputs, round_bf16


def test_round_bf16_matches_torch():
    x = np.random.default_rng(0).standard_normal(100000).astype(np.float32) * 3
    x[:4] = [0.0, -0.0, 1e-30, 65504.0]
    ref = torch.from_numpy(x.copy()).to(torch.bfloat16).to(torch.float32).numpy()
    assert np.array_equal(round_bf16(x.copy()), ref)


def test_tiny_inputs_deterministic_and_recipe():
    a = make_inputs(config("tiny_f32"))
    b = make_inputs(config("tiny_f32"))
    for k in ("embed", "wq", "prompt_k", "canvas_ids", "slot_pos", "label_ids", "noise_ids"):
        assert np.array_equal(a[k], b[k])
    dm = a["dims"]
    ids = a["canvas_ids"]
    assert ids.shape == (1, 256)
    assert int((ids == dm.mask_id).sum()) == 128          # exact round(0.5 * 256)
    assert ids.max() <= dm.mask_id
    assert np.all(ids[ids != dm.mask_id] < dm.vocab - 1)
    assert np.all(ids[0, a["slot_pos"][0]] == dm.mask_id)  # slots are masked positions
    nl = a["n_labels"][0]
    for s in range(8):
        lab = a["label_ids"][0, s, :nl[s]]
        assert len(set(lab.tolist())) == nl[s] == 4
        assert np.all(a["label_ids"][0, s, nl[s]:] == -1)
    assert a["cu_seqlens"].tolist() == [0, 128]


def test_skeleton_and_ragged_recipes():
    r = make_inputs(config("reads512"), batch=6, prompt_override=("fixed", 16))
    ids = r["canvas_ids"]
    assert np.all(ids == ids[0])                        # one shared skeleton
    assert int((ids[0] == r["dims"].mask_id).sum()) == 4
    assert np.all(r["n_labels"] >= 2) and np.all(r["n_labels"] <= 26)
    g = make_inputs(config("ragged32"), batch=5, prompt_override=("uniform", 3, 9))
    lens = np.diff(g["cu_seqlens"])
    assert np.all((lens >= 3) & (lens <= 9))
    fr = (g["canvas_ids"] == g["dims"].mask_id).mean(axis=1)
    assert np.all((fr > 0.05) & (fr < 0.95))
    bf = g["embed"]
    assert np.array_equal(round_bf16(bf.copy()), bf)   # already bf16-representable
