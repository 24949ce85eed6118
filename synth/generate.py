"""Seeded input generation.

Recipe (the same for every workload):

* one ``numpy.random.Generator(PCG64(SeedSequence(seed)))`` per workload; child
  streams are spawned in a fixed order: embed, wq, wk, wv, wo, prompt K, prompt V,
  prompt lengths, canvas ids, mask positions, slots, labels, noise ids,
  companion row scales, sc_in;
* embedding and projection weights ~ N(0, 0.02); prompt K and V ~ N(0, 1);
  values are drawn in float32 and, for bf16 storage, rounded to the nearest
  bf16 (ties to even) so every returned float is exactly representable in the
  storage type;
* canvas ids are uniform over [0, V-2] so the mask id V-1 appears only where it
  is placed; masked positions are an exact count round(f*C) taken from a seeded
  permutation;
* slot positions are a seeded choice among the masked positions (or, for a
  shared skeleton, a seeded choice of positions that are then masked in every
  canvas); labels are distinct ids drawn without replacement from [0, V-2];
* noise-draw token ids (the placeholder tokens a re-read writes at the slots)
  are uniform over [0, V-2] and are passed to both sides as an input.
"""
import numpy as np

from .configs import Config

_STREAMS = ("embed", "wq", "wk", "wv", "wo", "prompt_k", "prompt_v", "prompt_len",
            "canvas_ids", "mask_pos", "slots", "labels", "noise", "row_scale", "sc_in")

MAX_LABELS = 26


def round_bf16(a: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bfloat16 (ties to even), in place.

    Returns the same float32 array whose values are now bf16-representable.
    """
    assert a.dtype == np.float32
    u = a.view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    u += np.uint32(0x7FFF) + lsb
    u &= np.uint32(0xFFFF0000)
    return a


def _streams(seed: int):
    ss = np.random.SeedSequence(seed)
    children = ss.spawn(len(_STREAMS))
    return {name: np.random.Generator(np.random.PCG64(c)) for name, c in zip(_STREAMS, children)}


def _normal(rng, shape, std, dtype_name):
    a = rng.standard_normal(size=shape, dtype=np.float32)
    if std != 1.0:
        a *= np.float32(std)
    if dtype_name == "bf16":
        round_bf16(a)
    return a


def make_inputs(cfg: Config, with_sc_in: bool = False, batch: int = None,
                prompt_override=None) -> dict:
    """Draw every input of a workload.

    ``batch`` (if given) overrides cfg.batch; ``prompt_override`` replaces the
    prompt-length recipe (used by tests to shrink a workload).
    """
    dm = cfg.dims
    B = cfg.batch if batch is None else batch
    C, d, V = dm.canvas, dm.d_model, dm.vocab
    hd, Hq, Hkv = dm.head_dim, dm.n_q_heads, dm.n_kv_heads
    r = _streams(cfg.seed)
    out = {"cfg": cfg, "dims": dm, "batch": B}

    out["embed"] = _normal(r["embed"], (V, d), 0.02, dm.dtype)
    out["wq"] = _normal(r["wq"], (Hq * hd, d), 0.02, dm.dtype)
    out["wk"] = _normal(r["wk"], (Hkv * hd, d), 0.02, dm.dtype)
    out["wv"] = _normal(r["wv"], (Hkv * hd, d), 0.02, dm.dtype)
    out["wo"] = _normal(r["wo"], (d, Hq * hd), 0.02, dm.dtype)

    prompt = cfg.prompt if prompt_override is None else prompt_override
    if prompt[0] == "fixed":
        lens = np.full(B, prompt[1], dtype=np.int64)
    elif prompt[0] == "uniform":
        lens = r["prompt_len"].integers(prompt[1], prompt[2] + 1, size=B)
    else:
        raise ValueError(prompt)
    cu = np.zeros(B + 1, dtype=np.int64)
    cu[1:] = np.cumsum(lens)
    total = int(cu[-1])
    out["cu_seqlens"] = cu.astype(np.int32)
    out["prompt_lens"] = lens.astype(np.int32)
    out["max_prompt"] = int(lens.max()) if B > 0 else 0
    out["prompt_k"] = _normal(r["prompt_k"], (total, Hkv, hd), 1.0, dm.dtype)
    out["prompt_v"] = _normal(r["prompt_v"], (total, Hkv, hd), 1.0, dm.dtype)

    S = cfg.n_slots
    ids = r["canvas_ids"].integers(0, V - 1, size=(B, C)).astype(np.int32)
    slot_pos = np.zeros((B, S), dtype=np.int32)
    rm, rs = r["mask_pos"], r["slots"]
    if cfg.mask[0] == "skeleton":
        skel = ids[0].copy()
        pos = np.sort(rs.choice(C, size=S, replace=False)).astype(np.int32)
        skel[pos] = dm.mask_id
        ids[:] = skel[None, :]
        slot_pos[:] = pos[None, :]
        out["mask_frac"] = np.full(B, S / C)
    else:
        if cfg.mask[0] == "frac":
            fr = np.full(B, cfg.mask[1])
        elif cfg.mask[0] == "uniform_frac":
            fr = rm.uniform(cfg.mask[1], cfg.mask[2], size=B)
        else:
            raise ValueError(cfg.mask)
        for b in range(B):
            n = int(round(fr[b] * C))
            perm = rm.permutation(C)
            masked = np.sort(perm[:n])
            ids[b, masked] = dm.mask_id
            if S:
                pick = rs.choice(masked, size=min(S, n), replace=False)
                slot_pos[b, :len(pick)] = np.sort(pick)
        out["mask_frac"] = fr
    out["canvas_ids"] = ids
    out["slot_pos"] = slot_pos

    lab = np.full((B, S, MAX_LABELS), -1, dtype=np.int32)
    nl = np.zeros((B, S), dtype=np.int32)
    rl = r["labels"]
    for b in range(B):
        for s in range(S):
            if cfg.labels[0] == "fixed":
                k = cfg.labels[1]
            else:
                k = int(rl.integers(cfg.labels[1], cfg.labels[2] + 1))
            lab[b, s, :k] = rl.choice(V - 1, size=k, replace=False)
            nl[b, s] = k
    out["label_ids"] = lab
    out["n_labels"] = nl
    out["noise_ids"] = r["noise"].integers(0, V - 1, size=(max(cfg.n_draws, 1), B, S)).astype(np.int32)
    out["logit_scale"] = float(cfg.logit_scale)
    out["tau"] = float(cfg.tau)
    out["entropy_threshold"] = float(cfg.entropy_threshold)
    out["n_draws"] = int(cfg.n_draws)
    out["_row_scale_rng"] = r["row_scale"]
    if with_sc_in:
        out["sc_in"] = _normal(r["sc_in"], (B, C, d), 0.02, dm.dtype)
    return out


def companion_row_scale(inp: dict, shape, lo: float = 16.0, hi: float = 512.0) -> np.ndarray:
    """Per-row logit multipliers such that logit_scale * multiplier ~ logUniform(lo, hi).

    With the literal weight scales nearly every vocabulary row is flat, so
    argmax and commit order would be decided by rounding noise; these
    multipliers give a mix of peaked and flat rows so those checks have teeth.
    """
    rng = inp["_row_scale_rng"]
    total = np.exp(rng.uniform(np.log(lo), np.log(hi), size=shape))
    # the multipliers scale on top of the workload's own logit scale
    return (total / inp["logit_scale"]).astype(np.float32)


def prompt_batch(vocab: int, lengths, seed: int):
    """Packed prompt token ids for the encoder-mode forward: sequence b holds
    lengths[b] ids uniform over [0, V-2] (the mask id V-1 never appears), the
    sequences back to back.  Returns (ids int32 [sum lengths], cu int32 [B+1])."""
    rng = np.random.default_rng(np.random.SeedSequence(seed))
    lengths = np.asarray(lengths, dtype=np.int64)
    cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)
    ids = rng.integers(0, vocab - 1, size=int(cu[-1])).astype(np.int32)
    return ids, cu
