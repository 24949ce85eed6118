"""Device-side plumbing around the C-ABI: move host arrays into HBM as torch
tensors, allocate outputs and workspaces, and call the library.  No step of
the computation happens here.
"""
import numpy as np
import torch

from . import dg


def _dtype(name):
    return torch.bfloat16 if name == "bf16" else torch.float32


def to_device(a, dtype=None, device="cuda"):
    """numpy -> torch device tensor (float arrays converted to `dtype`)."""
    t = torch.from_numpy(np.ascontiguousarray(a))
    if dtype is not None:
        t = t.to(dtype)
    return t.to(device)


class DeviceProblem:
    """A workload's weights, prompt KV and canvases resident in device memory."""

    def __init__(self, inp, device="cuda", with_embed_t=True, with_lm_tiled=True,
                 with_embed_t_tiled=True, with_lm_fp8=False, lm_fp8_act=False):
        dm = inp["dims"]
        self.inp = inp
        self.device = device
        self.dims = dg.make_dims(dm.d_model, dm.n_q_heads, dm.n_kv_heads, dm.head_dim, dm.vocab,
                                 dm.canvas, dm.window, dm.mask_id, dm.dtype)
        self.tdt = _dtype(dm.dtype)
        self.B = inp["batch"]
        self.C = dm.canvas
        self.d = dm.d_model
        self.V = dm.vocab
        T = self.tdt
        self.embed = to_device(inp["embed"], T, device)
        self.wq = to_device(inp["wq"], T, device)
        self.wk = to_device(inp["wk"], T, device)
        self.wv = to_device(inp["wv"], T, device)
        self.wo = to_device(inp["wo"], T, device)
        self.lm_head = to_device(inp["lm_head"], T, device) if inp.get("lm_head") is not None else None
        self.embed_t = None
        if with_embed_t:
            self.embed_t = torch.empty((self.d, self.V), dtype=T, device=device)
            dg.dg_prepare_embed_t(self.dims, self.embed, self.embed_t)
        # the LM head in 256 x 32 blocks (bf16 only): same results, faster reads
        self.lm_tiled = None
        if with_lm_tiled and dm.dtype == "bf16" and self.d % 32 == 0:
            head = self.lm_head if self.lm_head is not None else self.embed
            self.lm_tiled = torch.empty((self.V * self.d,), dtype=T, device=device)
            dg.dg_prepare_lm_tiled(self.dims, head, self.lm_tiled)
        # embed^T in 256 x 32 blocks (bf16, d % 256 == 0) for the p.E contraction
        self.embed_t_tiled = None
        if (with_embed_t_tiled and self.embed_t is not None and dm.dtype == "bf16"
                and self.d % 256 == 0):
            self.embed_t_tiled = torch.empty((self.V * self.d,), dtype=T, device=device)
            dg.dg_prepare_embed_t_tiled(self.dims, self.embed_t, self.embed_t_tiled)
        # opt-in e4m3 copy of the LM head (bf16 only): every LM-head pass uses it;
        # lm_fp8_act: the step also quantises h per row and runs the FP8 MFMA
        self.lm_fp8 = self.lm_fp8_exp = None
        if with_lm_fp8:
            head = self.lm_head if self.lm_head is not None else self.embed
            self.lm_fp8 = torch.empty((self.V, self.d), dtype=torch.uint8, device=device)
            self.lm_fp8_exp = torch.empty((self.V,), dtype=torch.int32, device=device)
            dg.dg_prepare_lm_fp8(self.dims, head, self.lm_fp8, self.lm_fp8_exp)
        total = int(inp["cu_seqlens"][-1])
        kshape = (max(total, 1),) + inp["prompt_k"].shape[1:]
        self.prompt_k = torch.zeros(kshape, dtype=T, device=device)
        self.prompt_v = torch.zeros(kshape, dtype=T, device=device)
        if total:
            self.prompt_k[:total] = to_device(inp["prompt_k"], T, device)
            self.prompt_v[:total] = to_device(inp["prompt_v"], T, device)
        self.cu = to_device(inp["cu_seqlens"].astype(np.int32), None, device)
        self.max_prompt = int(inp["max_prompt"])
        self.total_len = total
        self.canvas_ids = to_device(inp["canvas_ids"].astype(np.int32), None, device)
        self.slot_pos = to_device(inp["slot_pos"].astype(np.int32), None, device)
        self.label_ids = to_device(inp["label_ids"].astype(np.int32), None, device)
        self.n_labels = to_device(inp["n_labels"].astype(np.int32), None, device)
        self.noise_ids = to_device(inp["noise_ids"].astype(np.int32), None, device)
        self.S = int(inp["slot_pos"].shape[1])
        self.weights = dg.make_weights(self.embed, self.wq, self.wk, self.wv, self.wo,
                                       embed_t=self.embed_t, lm_head=self.lm_head,
                                       lm_tiled=self.lm_tiled,
                                       embed_t_tiled=self.embed_t_tiled,
                                       lm_fp8=self.lm_fp8, lm_fp8_exp=self.lm_fp8_exp,
                                       lm_fp8_act=lm_fp8_act and with_lm_fp8)
        self.kv = dg.make_prompt_kv(self.prompt_k, self.prompt_v, self.cu, self.max_prompt,
                                    total)
        self._ws = {}

    # ---------------------------------------------------------------- step --
    def workspace(self, key, nbytes):
        ws = self._ws.get(key)
        if ws is None or ws.numel() < nbytes:
            ws = torch.empty(max(int(nbytes), 256), dtype=torch.uint8, device=self.device)
            self._ws[key] = ws
        return ws

    def step_outputs(self, want_sc=True, debug=False):
        B, C, d, V = self.B, self.C, self.d, self.V
        dm = self.inp["dims"]
        out = {
            "conf": torch.empty((B, C), dtype=torch.float32, device=self.device),
            "entropy": torch.empty((B, C), dtype=torch.float32, device=self.device),
            "argmax": torch.empty((B, C), dtype=torch.int32, device=self.device),
            "sc_out": torch.empty((B, C, d), dtype=self.tdt, device=self.device) if want_sc else None,
            "flags": torch.zeros(1, dtype=torch.int32, device=self.device),
        }
        if debug:
            out["attn_out"] = torch.empty((B, C, dm.n_q_heads * dm.head_dim), dtype=self.tdt,
                                          device=self.device)
            out["hidden_out"] = torch.empty((B, C, d), dtype=self.tdt, device=self.device)
            out["logits"] = torch.empty((B, C, V), dtype=torch.float32, device=self.device)
        return out

    def step(self, sc_in=None, row_scale=None, want_sc=True, debug=False, out=None,
             canvas_ids=None, stream=None):
        """One dg_denoise_step over every canvas; returns the output tensors."""
        if out is None:
            out = self.step_outputs(want_sc, debug)
        ws = self.workspace("step", dg.dg_denoise_step_workspace(self.dims, self.B, self.max_prompt))
        dbg = None
        if debug:
            dbg = dg.make_debug(out["attn_out"], out["hidden_out"], out["logits"])
        dg.dg_denoise_step(self.dims, self.weights, self.kv, self.B,
                           self.canvas_ids if canvas_ids is None else canvas_ids, sc_in,
                           self.inp["logit_scale"], row_scale, out["conf"], out["entropy"],
                           out["argmax"], out["sc_out"], dbg, out["flags"], ws, stream)
        return out

    # ------------------------------------------------------------- encoder --
    def encode(self, prompt_ids, cu, max_len, total_len, want_hidden=True, want_attn=True,
               stream=None):
        """dg_prefill_encode of packed prompts (device int32 ids and offsets):
        returns k, v (cache rows), hidden, attn (or None) and the flag word."""
        dm = self.inp["dims"]
        n = max(int(total_len), 1)
        out = {"k": torch.empty((n, dm.n_kv_heads, dm.head_dim), dtype=self.tdt, device=self.device),
               "flags": torch.zeros(1, dtype=torch.int32, device=self.device)}
        out["v"] = torch.empty_like(out["k"])
        out["hidden"] = (torch.empty((n, self.d), dtype=self.tdt, device=self.device)
                         if want_hidden else None)
        out["attn"] = (torch.empty((n, dm.n_q_heads * dm.head_dim), dtype=self.tdt, device=self.device)
                       if want_attn else None)
        B = int(cu.numel()) - 1
        ws = self.workspace("encode", dg.dg_prefill_encode_workspace(self.dims, B, int(max_len)))
        dg.dg_prefill_encode(self.dims, self.weights, B, cu, int(max_len), int(total_len), prompt_ids,
                             out["k"], out["v"], out["hidden"], out["attn"], out["flags"], ws, stream)
        return out

    # -------------------------------------------------------------- commit --
    def commit_outputs(self):
        B, C = self.B, self.C
        return {"mask": torch.empty((B, C), dtype=torch.uint8, device=self.device),
                "out_ids": torch.empty((B, C), dtype=torch.int32, device=self.device),
                "n": torch.empty((B,), dtype=torch.int32, device=self.device)}

    def commit(self, conf, entropy, argmax, tau=None, canvas_ids=None, out=None, stream=None):
        if out is None:
            out = self.commit_outputs()
        ids = self.canvas_ids if canvas_ids is None else canvas_ids
        dg.dg_commit(self.B, self.C, self.inp["dims"].mask_id, ids, conf, entropy, argmax,
                     self.inp["tau"] if tau is None else tau, out["mask"], out["out_ids"], out["n"],
                     stream)
        return out

    def slot_read_staged(self, stage, ask_if_slot, ask_if_label, row_scale=None, n_draws=None,
                         threshold=None, out=None, stream=None):
        """dg_slot_read_staged over the problem's slots (stage arrays are host lists)."""
        nd = self.inp["n_draws"] if n_draws is None else n_draws
        th = self.inp["entropy_threshold"] if threshold is None else threshold
        if out is None:
            out = self.slot_outputs()
        ws = self.workspace("staged", dg.dg_slot_read_staged_workspace(self.dims, self.B, self.S,
                                                                       self.max_prompt, nd))
        dg.dg_slot_read_staged(self.dims, self.weights, self.kv, self.B, self.canvas_ids, self.S,
                               self.slot_pos, self.label_ids, self.n_labels, self.noise_ids,
                               [int(x) for x in stage], [int(x) for x in ask_if_slot],
                               [int(x) for x in ask_if_label], self.inp["logit_scale"], row_scale,
                               th, nd, out["logprobs"], out["probs"], out["entropy"],
                               out["first_entropy"], out["best"], out["draws_used"], out["status"],
                               ws, stream)
        return out

    # ---------------------------------------------------------------- loop --
    def loop(self, tau=None, max_steps=None, check_every=8, sc_in=None, row_scale=None,
             canvas_ids=None, stream=None):
        """dg_denoise_loop from the problem's canvas (or canvas_ids, which is left
        untouched): returns the final canvas, commit steps, steps per canvas, the
        steps launched and the device flag word."""
        ids = (self.canvas_ids if canvas_ids is None else canvas_ids).clone()
        cs = torch.empty((self.B, self.C), dtype=torch.int32, device=self.device)
        steps = torch.empty((self.B,), dtype=torch.int32, device=self.device)
        flags = torch.zeros(1, dtype=torch.int32, device=self.device)
        ws = self.workspace("loop", dg.dg_denoise_loop_workspace(self.dims, self.B, self.max_prompt))
        n = dg.dg_denoise_loop(self.dims, self.weights, self.kv, self.B, ids, sc_in,
                               self.inp["logit_scale"], row_scale,
                               self.inp["tau"] if tau is None else tau,
                               self.C if max_steps is None else max_steps, check_every, cs, steps,
                               flags, ws, stream)
        return {"ids": ids, "commit_step": cs, "steps": steps, "launched": n, "flags": flags}

    # ----------------------------------------------------------- slot read --
    def slot_outputs(self):
        B, S = self.B, self.S
        f = lambda *s: torch.empty(s, dtype=torch.float32, device=self.device)  # noqa: E731
        i = lambda *s: torch.empty(s, dtype=torch.int32, device=self.device)    # noqa: E731
        return {"logprobs": f(B, S, dg.DG_MAX_LABELS), "probs": f(B, S, dg.DG_MAX_LABELS),
                "entropy": f(B, S), "first_entropy": f(B, S), "best": i(B, S),
                "draws_used": i(B, S), "status": i(B, S)}

    def slot_read(self, row_scale=None, n_draws=None, threshold=None, out=None, stream=None,
                  label_ids=None, n_labels=None, slot_pos=None, noise_ids=None,
                  full_canvas=False):
        """dg_slot_read (slot-row order), or dg_slot_read_full_canvas."""
        nd = self.inp["n_draws"] if n_draws is None else n_draws
        th = self.inp["entropy_threshold"] if threshold is None else threshold
        if out is None:
            out = self.slot_outputs()
        wsf = dg.dg_slot_read_full_canvas_workspace if full_canvas else dg.dg_slot_read_workspace
        call = dg.dg_slot_read_full_canvas if full_canvas else dg.dg_slot_read
        ws = self.workspace("slot_full" if full_canvas else "slot",
                            wsf(self.dims, self.B, self.S, self.max_prompt, nd))
        call(self.dims, self.weights, self.kv, self.B, self.canvas_ids, self.S,
                        self.slot_pos if slot_pos is None else slot_pos,
                        self.label_ids if label_ids is None else label_ids,
                        self.n_labels if n_labels is None else n_labels,
                        self.noise_ids if noise_ids is None else noise_ids,
                        self.inp["logit_scale"], row_scale, th, nd, out["logprobs"], out["probs"],
                        out["entropy"], out["first_entropy"], out["best"], out["draws_used"],
                        out["status"], ws, stream)
        return out
