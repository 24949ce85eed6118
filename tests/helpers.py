"""Comparison helpers shared by the parity tests."""
import numpy as np

# Tolerances (elementwise: |g - o| <= rtol * max(|o|, RMS of o's row)):
#   fp32 storage: 1e-4 relative on every float output (entropies and logprobs too).
#   bf16 storage: 2e-2 on attention output, hidden state and self-conditioning;
#                 1e-2 absolute on logprobs and entropies; 2e-2 relative on
#                 confidences and label probabilities.
TOL = {
    "f32": {"attn_out": 1e-4, "hidden_out": 1e-4, "logits": 1e-4, "sc_out": 1e-4,
            "conf": 1e-4, "entropy_abs": 1e-4, "probs": 1e-4, "logprob_abs": 1e-4},
    "bf16": {"attn_out": 2e-2, "hidden_out": 2e-2, "logits": 2e-2, "sc_out": 2e-2,
             "conf": 2e-2, "entropy_abs": 1e-2, "probs": 2e-2, "logprob_abs": 1e-2},
}
# near-tie widths for integer decisions taken from floating point (argmax, commit order)
TIE_EPS = {"f32": 1e-4, "bf16": 1e-2}


def to_np(t):
    import torch
    if isinstance(t, torch.Tensor):
        if t.dtype == torch.bfloat16:
            t = t.float()
        return t.detach().cpu().numpy()
    return np.asarray(t)


def row_rel_fail(g, o, rtol):
    """Boolean mask of elements failing |g-o| <= rtol*max(|o|, RMS_row(o))."""
    g = np.asarray(g, np.float64)
    o = np.asarray(o, np.float64)
    assert g.shape == o.shape, (g.shape, o.shape)
    if o.ndim == 0:
        o = o.reshape(1)
        g = g.reshape(1)
    rms = np.sqrt(np.mean(o * o, axis=-1, keepdims=True))
    bound = rtol * np.maximum(np.abs(o), rms)
    return ~(np.abs(g - o) <= bound)


def assert_row_rel(g, o, rtol, name):
    bad = row_rel_fail(g, o, rtol)
    if bad.any():
        g = np.asarray(g, np.float64)
        o = np.asarray(o, np.float64)
        idx = np.argwhere(bad)[:5]
        rel = np.abs(g - o) / np.maximum(np.abs(o), 1e-30)
        raise AssertionError(
            f"{name}: {int(bad.sum())}/{bad.size} elements outside rtol {rtol}; "
            f"first {idx.tolist()} got {[float(g[tuple(i)]) for i in idx]} "
            f"want {[float(o[tuple(i)]) for i in idx]}; max rel {float(rel.max()):.3g}")


def assert_abs(g, o, atol, name):
    g = np.asarray(g, np.float64)
    o = np.asarray(o, np.float64)
    err = np.abs(g - o)
    if not np.all(err <= atol):
        i = np.unravel_index(np.argmax(err), err.shape)
        raise AssertionError(f"{name}: max abs err {float(err.max()):.3g} at {i} "
                             f"(got {float(g[i])}, want {float(o[i])}), atol {atol}")


def assert_float(g, o, dtype, kind, name):
    """Apply the bar for `kind` at `dtype`: bf16 entropies/logprobs are absolute,
    everything else (and everything in fp32) is row-relative."""
    t = TOL[dtype]
    if kind in ("entropy", "logprob"):
        key = "entropy_abs" if kind == "entropy" else "logprob_abs"
        if dtype == "bf16":
            assert_abs(g, o, t[key], name)
        else:
            assert_row_rel(np.atleast_2d(g), np.atleast_2d(o), t[key], name)
    else:
        assert_row_rel(g, o, t[kind], name)

