"""ctypes binding of libdg.so: the same calls as include/dg.h, argument
marshalling only.  Arrays are torch tensors on the GPU (or None); every step of
the computation runs in the HIP library.  Loading fails loudly if the library
has not been built.
"""
import ctypes
import os

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libdg.so")

DG_OK, DG_ERR_INVALID_ARG, DG_ERR_TOO_MANY_LABELS, DG_ERR_UNSUPPORTED, DG_ERR_WORKSPACE, DG_ERR_HIP = range(6)
DG_F32, DG_BF16 = 0, 1
DG_MAX_LABELS = 26
DG_MAX_CANVAS = 1024
DG_FLAG_BAD_TOKEN = 1
DG_FLAG_BAD_SEQLENS = 2
DG_SLOT_OK, DG_SLOT_BAD_POS, DG_SLOT_BAD_COUNT, DG_SLOT_BAD_LABEL, DG_SLOT_BAD_NOISE = range(5)
DG_SLOT_NOT_ASKED = 5
DG_NOALLOC_SCRATCH_BYTES = 64 << 20


class DGError(RuntimeError):
    def __init__(self, status, message):
        super().__init__(f"{message} (status {status})")
        self.status = status


class Dims(ctypes.Structure):
    _fields_ = [("d_model", ctypes.c_int32), ("n_q_heads", ctypes.c_int32),
                ("n_kv_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("vocab", ctypes.c_int32), ("canvas", ctypes.c_int32),
                ("window", ctypes.c_int32), ("mask_id", ctypes.c_int32),
                ("dtype", ctypes.c_int32)]


class Weights(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in
                ("embed", "embed_t", "lm_head", "wq", "wk", "wv", "wo", "lm_tiled",
                 "embed_t_tiled", "lm_fp8", "lm_fp8_exp")] + [("lm_fp8_act", ctypes.c_int32)]


class PromptKV(ctypes.Structure):
    _fields_ = [("k", ctypes.c_void_p), ("v", ctypes.c_void_p),
                ("cu_seqlens", ctypes.c_void_p), ("max_len", ctypes.c_int32),
                ("total_len", ctypes.c_int64)]


class Debug(ctypes.Structure):
    _fields_ = [("attn_out", ctypes.c_void_p), ("hidden_out", ctypes.c_void_p),
                ("logits_out", ctypes.c_void_p), ("stage_events", ctypes.c_void_p)]


DG_STAGES = ("qkv", "attention", "oproj", "lmhead", "vocab_merge", "selfcond")
DG_N_STAGES = len(DG_STAGES)


_P = ctypes.c_void_p
_I32 = ctypes.c_int32
_F = ctypes.c_float
_SZ = ctypes.c_size_t

# name -> (restype, argtypes), mirroring include/dg.h
_SIGS = {
    "dg_denoise_step_workspace": (_SZ, [ctypes.POINTER(Dims), _I32, _I32]),
    "dg_denoise_step": (_I32, [ctypes.POINTER(Dims), ctypes.POINTER(Weights), ctypes.POINTER(PromptKV),
                               _I32, _P, _P, _F, _P, _P, _P, _P, _P, ctypes.POINTER(Debug), _P,
                               _P, _SZ, _P]),
    "dg_commit": (_I32, [_I32, _I32, _I32, _P, _P, _P, _P, _F, _P, _P, _P, _P]),
    "dg_prefill_kv": (_I32, [ctypes.POINTER(Dims), ctypes.POINTER(Weights), ctypes.c_int64, _P, _P,
                             _P, _P, _P]),
    "dg_prefill_encode_workspace": (_SZ, [ctypes.POINTER(Dims), _I32, _I32]),
    "dg_prefill_encode": (_I32, [ctypes.POINTER(Dims), ctypes.POINTER(Weights), _I32, _P, _I32,
                                 ctypes.c_int64, _P, _P, _P, _P, _P, _P, _P, _SZ, _P]),
    "dg_denoise_loop_workspace": (_SZ, [ctypes.POINTER(Dims), _I32, _I32]),
    "dg_denoise_loop": (_I32, [ctypes.POINTER(Dims), ctypes.POINTER(Weights), ctypes.POINTER(PromptKV),
                               _I32, _P, _P, _F, _P, _F, _I32, _I32, _P, _P,
                               ctypes.POINTER(_I32), _P, _P, _SZ, _P]),
    "dg_slot_read_workspace": (_SZ, [ctypes.POINTER(Dims), _I32, _I32, _I32, _I32]),
    "dg_slot_read": (_I32, [ctypes.POINTER(Dims), ctypes.POINTER(Weights), ctypes.POINTER(PromptKV),
                            _I32, _P, _I32, _P, _P, _P, _P, _F, _P, _F, _I32,
                            _P, _P, _P, _P, _P, _P, _P, _P, _SZ, _P]),
    "dg_slot_read_full_canvas_workspace": (_SZ, [ctypes.POINTER(Dims), _I32, _I32, _I32, _I32]),
    "dg_slot_read_full_canvas": (_I32, [ctypes.POINTER(Dims), ctypes.POINTER(Weights),
                                        ctypes.POINTER(PromptKV), _I32, _P, _I32, _P, _P, _P, _P,
                                        _F, _P, _F, _I32, _P, _P, _P, _P, _P, _P, _P, _P, _SZ, _P]),
    "dg_slot_read_noalloc": (_I32, [ctypes.POINTER(Dims), ctypes.POINTER(Weights), ctypes.POINTER(PromptKV),
                                    _I32, _P, _I32, _P, _P, _P, _P, _F, _P, _F, _I32,
                                    _P, _P, _P, _P, _P, _P, _P, _P]),
    "dg_slot_read_staged_workspace": (_SZ, [ctypes.POINTER(Dims), _I32, _I32, _I32, _I32]),
    "dg_slot_read_staged": (_I32, [ctypes.POINTER(Dims), ctypes.POINTER(Weights), ctypes.POINTER(PromptKV),
                                   _I32, _P, _I32, _P, _P, _P, _P, _P, _P, _P, _F, _P, _F, _I32,
                                   _P, _P, _P, _P, _P, _P, _P, _P, _SZ, _P]),
    "dg_prepare_embed_t": (_I32, [ctypes.POINTER(Dims), _P, _P, _P]),
    "dg_prepare_lm_tiled": (_I32, [ctypes.POINTER(Dims), _P, _P, _P]),
    "dg_prepare_embed_t_tiled": (_I32, [ctypes.POINTER(Dims), _P, _P, _P]),
    "dg_prepare_lm_fp8": (_I32, [ctypes.POINTER(Dims), _P, _P, _P, _P]),
    "dg_denoise_step_validate": (_I32, [ctypes.POINTER(Dims), _I32, _I32, ctypes.POINTER(Weights),
                                        ctypes.POINTER(PromptKV)]),
    "dg_slot_read_validate": (_I32, [ctypes.POINTER(Dims), _I32, _I32, _I32, _F]),
    "dg_commit_validate": (_I32, [_I32, _I32]),
    "dg_check_label_count": (_I32, [_I32]),
    "dg_status_string": (ctypes.c_char_p, [_I32]),
    "dg_last_error": (ctypes.c_char_p, []),
    "dg_version": (ctypes.c_char_p, []),
}

_lib = None


def lib():
    """Load libdg.so (once).  Raises if it is missing: there is no fallback."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: build it with `python -m slot_readout_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGS.items():
            f = getattr(L, name)
            f.restype = res
            f.argtypes = args
        _lib = L
    return _lib


def exported_symbols():
    return list(_SIGS)


def _ptr(t):
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _check(status):
    if status != DG_OK:
        L = lib()
        raise DGError(status, f"{L.dg_status_string(status).decode()}: {L.dg_last_error().decode()}")


def _stream(stream):
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def make_dims(d_model, n_q_heads, n_kv_heads, head_dim, vocab, canvas, window, mask_id, dtype):
    dt = {"f32": DG_F32, "bf16": DG_BF16}.get(dtype, dtype)
    return Dims(d_model, n_q_heads, n_kv_heads, head_dim, vocab, canvas, window, mask_id, dt)


def make_weights(embed, wq, wk, wv, wo, embed_t=None, lm_head=None, lm_tiled=None,
                 embed_t_tiled=None, lm_fp8=None, lm_fp8_exp=None, lm_fp8_act=False):
    return Weights(_ptr(embed), _ptr(embed_t), _ptr(lm_head), _ptr(wq), _ptr(wk), _ptr(wv), _ptr(wo),
                   _ptr(lm_tiled), _ptr(embed_t_tiled), _ptr(lm_fp8), _ptr(lm_fp8_exp),
                   int(bool(lm_fp8_act)))


def make_prompt_kv(k, v, cu_seqlens, max_len, total_len):
    return PromptKV(_ptr(k), _ptr(v), _ptr(cu_seqlens), int(max_len), int(total_len))


def make_debug(attn_out=None, hidden_out=None, logits_out=None, stage_events=None):
    """stage_events: a ctypes array of 2*DG_N_STAGES hipEvent_t handles, or None."""
    ev = ctypes.cast(stage_events, ctypes.c_void_p) if stage_events is not None else None
    return Debug(_ptr(attn_out), _ptr(hidden_out), _ptr(logits_out), ev)


# ---------------------------------------------------------------- calls -----
def dg_denoise_step_workspace(dims, batch, max_prompt):
    return lib().dg_denoise_step_workspace(ctypes.byref(dims), batch, max_prompt)


def dg_denoise_step(dims, weights, kv, batch, canvas_ids, sc_in, logit_scale, row_scale,
                    conf, entropy, argmax, sc_out, debug, dev_flags, workspace, stream=None):
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _check(lib().dg_denoise_step(
        ctypes.byref(dims), ctypes.byref(weights), ctypes.byref(kv), batch, _ptr(canvas_ids),
        _ptr(sc_in), float(logit_scale), _ptr(row_scale), _ptr(conf), _ptr(entropy), _ptr(argmax),
        _ptr(sc_out), ctypes.byref(debug) if debug is not None else None, _ptr(dev_flags),
        _ptr(workspace), ws_bytes, _stream(stream)))


def dg_commit(batch, canvas, mask_id, canvas_ids, conf, entropy, argmax, threshold_nats,
              commit_mask, out_ids, n_committed, stream=None):
    _check(lib().dg_commit(batch, canvas, mask_id, _ptr(canvas_ids), _ptr(conf), _ptr(entropy),
                           _ptr(argmax), float(threshold_nats), _ptr(commit_mask), _ptr(out_ids),
                           _ptr(n_committed), _stream(stream)))


def dg_prefill_kv(dims, weights, n_tokens, prompt_ids, k_out, v_out, dev_flags=None, stream=None):
    _check(lib().dg_prefill_kv(ctypes.byref(dims), ctypes.byref(weights), int(n_tokens),
                               _ptr(prompt_ids), _ptr(k_out), _ptr(v_out), _ptr(dev_flags),
                               _stream(stream)))


def dg_prefill_encode_workspace(dims, batch, max_len):
    return lib().dg_prefill_encode_workspace(ctypes.byref(dims), batch, max_len)


def dg_prefill_encode(dims, weights, batch, cu_seqlens, max_len, total_len, prompt_ids, k_out, v_out,
                      hidden_out=None, attn_out=None, dev_flags=None, workspace=None, stream=None):
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _check(lib().dg_prefill_encode(ctypes.byref(dims), ctypes.byref(weights), int(batch),
                                   _ptr(cu_seqlens), int(max_len), int(total_len), _ptr(prompt_ids),
                                   _ptr(k_out), _ptr(v_out), _ptr(hidden_out), _ptr(attn_out),
                                   _ptr(dev_flags), _ptr(workspace), ws_bytes, _stream(stream)))


def dg_denoise_loop_workspace(dims, batch, max_prompt):
    return lib().dg_denoise_loop_workspace(ctypes.byref(dims), batch, max_prompt)


def dg_denoise_loop(dims, weights, kv, batch, canvas_ids, sc_in, logit_scale, row_scale,
                    threshold_nats, max_steps, check_every, commit_step, steps_taken, dev_flags,
                    workspace, stream=None):
    """Runs the loop; returns the number of steps launched."""
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    launched = _I32(0)
    _check(lib().dg_denoise_loop(
        ctypes.byref(dims), ctypes.byref(weights), ctypes.byref(kv), batch, _ptr(canvas_ids),
        _ptr(sc_in), float(logit_scale), _ptr(row_scale), float(threshold_nats), int(max_steps),
        int(check_every), _ptr(commit_step), _ptr(steps_taken), ctypes.byref(launched),
        _ptr(dev_flags), _ptr(workspace), ws_bytes, _stream(stream)))
    return int(launched.value)


def dg_slot_read_workspace(dims, batch, n_slots, max_prompt, n_draws):
    return lib().dg_slot_read_workspace(ctypes.byref(dims), batch, n_slots, max_prompt, n_draws)


def dg_slot_read(dims, weights, kv, batch, canvas_ids, n_slots, slot_pos, label_ids, n_labels,
                 noise_ids, logit_scale, row_scale, entropy_threshold, n_draws, logprobs, probs,
                 entropy, first_entropy, best, draws_used, status, workspace, stream=None):
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _check(lib().dg_slot_read(
        ctypes.byref(dims), ctypes.byref(weights), ctypes.byref(kv), batch, _ptr(canvas_ids),
        n_slots, _ptr(slot_pos), _ptr(label_ids), _ptr(n_labels), _ptr(noise_ids),
        float(logit_scale), _ptr(row_scale), float(entropy_threshold), n_draws, _ptr(logprobs),
        _ptr(probs), _ptr(entropy), _ptr(first_entropy), _ptr(best), _ptr(draws_used),
        _ptr(status), _ptr(workspace), ws_bytes, _stream(stream)))


def dg_slot_read_full_canvas_workspace(dims, batch, n_slots, max_prompt, n_draws):
    return lib().dg_slot_read_full_canvas_workspace(ctypes.byref(dims), batch, n_slots, max_prompt,
                                                    n_draws)


def dg_slot_read_full_canvas(dims, weights, kv, batch, canvas_ids, n_slots, slot_pos, label_ids,
                             n_labels, noise_ids, logit_scale, row_scale, entropy_threshold,
                             n_draws, logprobs, probs, entropy, first_entropy, best, draws_used,
                             status, workspace, stream=None):
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _check(lib().dg_slot_read_full_canvas(
        ctypes.byref(dims), ctypes.byref(weights), ctypes.byref(kv), batch, _ptr(canvas_ids),
        n_slots, _ptr(slot_pos), _ptr(label_ids), _ptr(n_labels), _ptr(noise_ids),
        float(logit_scale), _ptr(row_scale), float(entropy_threshold), n_draws, _ptr(logprobs),
        _ptr(probs), _ptr(entropy), _ptr(first_entropy), _ptr(best), _ptr(draws_used),
        _ptr(status), _ptr(workspace), ws_bytes, _stream(stream)))


def dg_slot_read_noalloc(dims, weights, kv, batch, canvas_ids, n_slots, slot_pos, label_ids,
                         n_labels, noise_ids, logit_scale, row_scale, entropy_threshold, n_draws,
                         logprobs, probs, entropy, first_entropy, best, draws_used, status,
                         stream=None):
    _check(lib().dg_slot_read_noalloc(
        ctypes.byref(dims), ctypes.byref(weights), ctypes.byref(kv), batch, _ptr(canvas_ids),
        n_slots, _ptr(slot_pos), _ptr(label_ids), _ptr(n_labels), _ptr(noise_ids),
        float(logit_scale), _ptr(row_scale), float(entropy_threshold), n_draws, _ptr(logprobs),
        _ptr(probs), _ptr(entropy), _ptr(first_entropy), _ptr(best), _ptr(draws_used),
        _ptr(status), _stream(stream)))


def dg_slot_read_staged_workspace(dims, batch, n_slots, max_prompt, n_draws):
    return lib().dg_slot_read_staged_workspace(ctypes.byref(dims), batch, n_slots, max_prompt, n_draws)


def dg_slot_read_staged(dims, weights, kv, batch, canvas_ids, n_slots, slot_pos, label_ids,
                        n_labels, noise_ids, slot_stage, ask_if_slot, ask_if_label, logit_scale,
                        row_scale, entropy_threshold, n_draws, logprobs, probs, entropy,
                        first_entropy, best, draws_used, status, workspace, stream=None):
    """slot_stage, ask_if_slot, ask_if_label: host sequences of n_slots ints."""
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    arr = ctypes.c_int32 * max(int(n_slots), 1)
    st, ak, al = arr(*slot_stage), arr(*ask_if_slot), arr(*ask_if_label)
    _check(lib().dg_slot_read_staged(
        ctypes.byref(dims), ctypes.byref(weights), ctypes.byref(kv), batch, _ptr(canvas_ids),
        n_slots, _ptr(slot_pos), _ptr(label_ids), _ptr(n_labels), _ptr(noise_ids),
        ctypes.addressof(st), ctypes.addressof(ak), ctypes.addressof(al), float(logit_scale),
        _ptr(row_scale), float(entropy_threshold), n_draws, _ptr(logprobs), _ptr(probs),
        _ptr(entropy), _ptr(first_entropy), _ptr(best), _ptr(draws_used), _ptr(status),
        _ptr(workspace), ws_bytes, _stream(stream)))


def dg_prepare_embed_t(dims, embed, embed_t, stream=None):
    _check(lib().dg_prepare_embed_t(ctypes.byref(dims), _ptr(embed), _ptr(embed_t), _stream(stream)))


def dg_prepare_lm_tiled(dims, head, lm_tiled, stream=None):
    _check(lib().dg_prepare_lm_tiled(ctypes.byref(dims), _ptr(head), _ptr(lm_tiled), _stream(stream)))


def dg_prepare_lm_fp8(dims, head, codes, exps, stream=None):
    _check(lib().dg_prepare_lm_fp8(ctypes.byref(dims), _ptr(head), _ptr(codes), _ptr(exps),
                                   _stream(stream)))


def dg_prepare_embed_t_tiled(dims, embed_t, embed_t_tiled, stream=None):
    _check(lib().dg_prepare_embed_t_tiled(ctypes.byref(dims), _ptr(embed_t), _ptr(embed_t_tiled),
                                          _stream(stream)))


def dg_denoise_step_validate(dims, batch, max_prompt, weights, kv):
    return lib().dg_denoise_step_validate(ctypes.byref(dims) if dims is not None else None, batch,
                                          max_prompt, ctypes.byref(weights) if weights is not None else None,
                                          ctypes.byref(kv) if kv is not None else None)


def dg_slot_read_validate(dims, batch, n_slots, n_draws, entropy_threshold):
    return lib().dg_slot_read_validate(ctypes.byref(dims), batch, n_slots, n_draws, float(entropy_threshold))


def dg_commit_validate(batch, canvas):
    return lib().dg_commit_validate(batch, canvas)


def dg_check_label_count(n):
    return lib().dg_check_label_count(n)


def dg_last_error():
    return lib().dg_last_error().decode()


def dg_status_string(s):
    return lib().dg_status_string(s).decode()


def dg_version():
    return lib().dg_version().decode()


def check_alternatives(question: str, alternatives) -> None:
    """Reject a question with more alternatives than single-token labels A..Z allow."""
    n = len(alternatives)
    s = dg_check_label_count(n)
    if s == DG_ERR_TOO_MANY_LABELS:
        raise ValueError(f"too many labels for '{question}': {n} > {DG_MAX_LABELS}")
    if s != DG_OK:
        raise ValueError(f"question '{question}': needs at least one alternative")
