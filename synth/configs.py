"""The five workloads of the denoise step and slot read, as plain data.

Sizes follow the pages' workload descriptions: a 256-token canvas (24-ai.news,
"how is diffusion text generation different"), bidirectional attention with a
+-W window over the canvas plus the cached prompt KV (same section; thakicloud,
"DiffusionGemma"), 512-wide attention heads (sotaaz, "running it on the A100"),
at most 26 single-token labels per slot and a re-read above entropy 0.1 with 4
draws (sotaaz, "the server only takes 26 alternatives per question"), and a
110,707-token context (tau-home, "cache reuse").  Dimensions the pages leave
open (d_model, head counts, vocab, W, thresholds, weight scales, batch shapes)
are those of the workload list this project was specified against.
"""
from dataclasses import dataclass, field, replace
from typing import Optional, Tuple


@dataclass(frozen=True)
class Dims:
    d_model: int
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    vocab: int
    canvas: int
    window: int
    mask_id: int
    dtype: str  # "f32" or "bf16": the storage type of weights and activations


@dataclass(frozen=True)
class Config:
    name: str
    seed: int
    dims: Dims
    batch: int
    # prompt length recipe: ("fixed", P) or ("uniform", lo, hi) inclusive
    prompt: Tuple
    # mask recipe: ("frac", f) exact count round(f*C); ("uniform_frac", lo, hi)
    # per canvas; ("skeleton",) = only slot positions masked, one shared skeleton
    mask: Tuple
    logit_scale: float
    tau: float
    # slots: (n_slots, "masked" | "skeleton"); labels: ("fixed", k) | ("uniform", lo, hi)
    n_slots: int = 0
    slot_from: str = "masked"
    labels: Tuple = ("fixed", 4)
    entropy_threshold: float = 0.1
    n_draws: int = 4
    note: str = ""


def _tiny(dtype="f32", window=16):
    return Dims(d_model=256, n_q_heads=4, n_kv_heads=4, head_dim=64, vocab=2048,
                canvas=256, window=window, mask_id=2047, dtype=dtype)


_BIG = Dims(d_model=2816, n_q_heads=8, n_kv_heads=2, head_dim=512, vocab=262144,
            canvas=256, window=128, mask_id=262143, dtype="bf16")

CONFIGS = {
    # small fp32 case: the oracle finishes in seconds
    "tiny_f32": Config("tiny_f32", 1, _tiny("f32", 16), batch=1, prompt=("fixed", 128),
                       mask=("frac", 0.5), logit_scale=8.0, tau=1.0, n_slots=8,
                       slot_from="masked", labels=("fixed", 4)),
    # the headline single-canvas bf16 step (LM head + fused softmax + p.E + commit);
    # the read leg of a full pass uses 8 slots among the masked positions, 4 labels
    "bf16_step": Config("bf16_step", 2, _BIG, batch=1, prompt=("fixed", 2048),
                        mask=("frac", 0.5), logit_scale=1.0, tau=2.0, n_slots=8,
                        slot_from="masked", labels=("fixed", 4)),
    # ragged throughput batch, tiny dims in bf16
    "ragged32": Config("ragged32", 3, _tiny("bf16", 16), batch=32,
                       prompt=("uniform", 512, 8192), mask=("uniform_frac", 0.1, 0.9),
                       logit_scale=8.0, tau=2.0, n_slots=4, slot_from="masked",
                       labels=("fixed", 4)),
    # long cached prompt, read cold from HBM
    "long_read": Config("long_read", 4, _tiny("bf16", 128), batch=1,
                        prompt=("fixed", 110707), mask=("frac", 0.5), logit_scale=8.0,
                        tau=2.0, n_slots=8, slot_from="masked", labels=("fixed", 4)),
    # structured-read batch: one shared skeleton, 4 slots, k ~ U{2..26}
    "reads512": Config("reads512", 5, _tiny("bf16", 16), batch=512,
                       prompt=("fixed", 1024), mask=("skeleton",), logit_scale=8.0,
                       tau=2.0, n_slots=4, slot_from="skeleton",
                       labels=("uniform", 2, 26), entropy_threshold=0.1, n_draws=4),
}


def config(name: str, **overrides) -> Config:
    """Return a named config, optionally with fields replaced (e.g. batch=2)."""
    cfg = CONFIGS[name]
    dims_over = {k: overrides.pop(k) for k in list(overrides) if hasattr(cfg.dims, k)}
    if dims_over:
        cfg = replace(cfg, dims=replace(cfg.dims, **dims_over))
    if overrides:
        cfg = replace(cfg, **overrides)
    return cfg
