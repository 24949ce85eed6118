"""The C-ABI library on the host: it loads without a GPU, exports every symbol
include/dg.h declares, and its host-side validation rejects bad arguments
before anything is launched (no compute calls here)."""
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "dg.h")


def _lib_or_skip():
    from slot_readout_amd import dg
    if not os.path.exists(dg.LIB_PATH):
        pytest.skip("libdg.so not built (run python -m slot_readout_amd.build)")
    return dg


def _declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(dg_[a-z0-9_]+)\s*\(", src)))


def test_header_declares_the_three_calls():
    names = _declared_functions()
    for n in ("dg_denoise_step", "dg_commit", "dg_slot_read"):
        assert n in names


def test_library_exports_every_declared_symbol():
    dg = _lib_or_skip()
    L = dg.lib()
    for name in _declared_functions():
        assert hasattr(L, name), name
    assert set(_declared_functions()) == set(dg.exported_symbols())
    assert "gfx950" in dg.dg_version()


def _dims(dg, **kw):
    base = dict(d_model=256, n_q_heads=4, n_kv_heads=4, head_dim=64, vocab=2048, canvas=256,
                window=16, mask_id=2047, dtype="bf16")
    base.update(kw)
    return dg.make_dims(**base)


def _weights(dg):
    return dg.make_weights(256, 256, 256, 256, 256)   # non-null, aligned fake addresses


def _kv(dg, max_len=128, total=128):
    return dg.make_prompt_kv(512, 512, 1024, max_len, total)


def test_validation_accepts_the_workload_dims():
    dg = _lib_or_skip()
    assert dg.dg_denoise_step_validate(_dims(dg), 1, 128, _weights(dg), _kv(dg)) == dg.DG_OK
    big = _dims(dg, d_model=2816, n_q_heads=8, n_kv_heads=2, head_dim=512, vocab=262144,
                window=128, mask_id=262143)
    assert dg.dg_denoise_step_validate(big, 1, 2048, _weights(dg), _kv(dg, 2048, 2048)) == dg.DG_OK
    assert dg.dg_denoise_step_workspace(big, 1, 2048) > 256 * 262144 * 2  # holds p~


@pytest.mark.parametrize("kw,code", [
    (dict(head_dim=128), "DG_ERR_UNSUPPORTED"),
    (dict(head_dim=512, dtype="f32"), "DG_ERR_UNSUPPORTED"),
    (dict(dtype=7), "DG_ERR_UNSUPPORTED"),
    (dict(d_model=250), "DG_ERR_INVALID_ARG"),
    (dict(d_model=96, dtype="bf16"), "DG_ERR_UNSUPPORTED"),   # bf16 steps d_model by 64
    (dict(n_q_heads=6, n_kv_heads=4), "DG_ERR_INVALID_ARG"),
    (dict(vocab=2000), "DG_ERR_INVALID_ARG"),
    (dict(canvas=0), "DG_ERR_INVALID_ARG"),
    (dict(canvas=1025), "DG_ERR_INVALID_ARG"),
    (dict(window=-1), "DG_ERR_INVALID_ARG"),
    (dict(mask_id=2048), "DG_ERR_INVALID_ARG"),
])
def test_validation_rejects_bad_dims(kw, code):
    dg = _lib_or_skip()
    s = dg.dg_denoise_step_validate(_dims(dg, **kw), 1, 128, _weights(dg), _kv(dg))
    assert s == getattr(dg, code), (kw, s, dg.dg_last_error())
    assert dg.dg_last_error()


def test_validation_rejects_bad_pointers_and_sizes():
    dg = _lib_or_skip()
    d = _dims(dg)
    assert dg.dg_denoise_step_validate(None, 1, 128, _weights(dg), _kv(dg)) == dg.DG_ERR_INVALID_ARG
    assert dg.dg_denoise_step_validate(d, -1, 128, _weights(dg), _kv(dg)) == dg.DG_ERR_INVALID_ARG
    assert dg.dg_denoise_step_validate(d, 1, 128, None, _kv(dg)) == dg.DG_ERR_INVALID_ARG
    w = dg.make_weights(256, 0, 256, 256, 256)
    assert dg.dg_denoise_step_validate(d, 1, 128, w, _kv(dg)) == dg.DG_ERR_INVALID_ARG
    w = dg.make_weights(258, 256, 256, 256, 256)        # misaligned embedding
    assert dg.dg_denoise_step_validate(d, 1, 128, w, _kv(dg)) == dg.DG_ERR_INVALID_ARG
    kv = dg.make_prompt_kv(512, 512, 0, 128, 128)         # no cu_seqlens
    assert dg.dg_denoise_step_validate(d, 1, 128, _weights(dg), kv) == dg.DG_ERR_INVALID_ARG
    kv = dg.make_prompt_kv(0, 0, 1024, 128, 128)          # KV missing with a prompt
    assert dg.dg_denoise_step_validate(d, 1, 128, _weights(dg), kv) == dg.DG_ERR_INVALID_ARG
    assert dg.dg_denoise_step_validate(d, 1, 64, _weights(dg), _kv(dg)) == dg.DG_ERR_INVALID_ARG
    kv0 = dg.make_prompt_kv(0, 0, 1024, 0, 0)             # empty prompts are fine
    assert dg.dg_denoise_step_validate(d, 1, 0, _weights(dg), kv0) == dg.DG_OK


def test_validation_of_the_fp8_head_options():
    dg = _lib_or_skip()
    d = _dims(dg)
    ok = dg.make_weights(256, 256, 256, 256, 256, lm_fp8=1024, lm_fp8_exp=2048)
    assert dg.dg_denoise_step_validate(d, 1, 128, ok, _kv(dg)) == dg.DG_OK
    act = dg.make_weights(256, 256, 256, 256, 256, lm_fp8=1024, lm_fp8_exp=2048, lm_fp8_act=True)
    assert dg.dg_denoise_step_validate(d, 1, 128, act, _kv(dg)) == dg.DG_OK
    # codes without exponents, activations without the e4m3 head
    w = dg.make_weights(256, 256, 256, 256, 256, lm_fp8=1024)
    assert dg.dg_denoise_step_validate(d, 1, 128, w, _kv(dg)) == dg.DG_ERR_INVALID_ARG
    w = dg.make_weights(256, 256, 256, 256, 256, lm_fp8_act=True)
    assert dg.dg_denoise_step_validate(d, 1, 128, w, _kv(dg)) == dg.DG_ERR_INVALID_ARG
    assert "lm_fp8_act" in dg.dg_last_error()
    # FP8 activations step K by 128; fp32 storage has no e4m3 head
    d192 = _dims(dg, d_model=192)
    assert dg.dg_denoise_step_validate(d192, 1, 128, ok, _kv(dg)) == dg.DG_OK
    assert dg.dg_denoise_step_validate(d192, 1, 128, act, _kv(dg)) == dg.DG_ERR_UNSUPPORTED
    assert dg.dg_denoise_step_validate(_dims(dg, dtype="f32"), 1, 128, ok, _kv(dg)) == dg.DG_ERR_UNSUPPORTED


def test_slot_read_and_commit_validation():
    dg = _lib_or_skip()
    d = _dims(dg)
    assert dg.dg_slot_read_validate(d, 2, 4, 4, 0.1) == dg.DG_OK
    assert dg.dg_slot_read_validate(d, 2, 4, 0, 0.1) == dg.DG_ERR_INVALID_ARG
    assert dg.dg_slot_read_validate(d, 2, 4, 17, 0.1) == dg.DG_ERR_INVALID_ARG
    assert dg.dg_slot_read_validate(d, 2, -1, 4, 0.1) == dg.DG_ERR_INVALID_ARG
    assert dg.dg_slot_read_validate(d, 2, 4, 4, -0.5) == dg.DG_ERR_INVALID_ARG
    assert dg.dg_slot_read_validate(d, 2, 4, 4, float("nan")) == dg.DG_ERR_INVALID_ARG
    assert dg.dg_commit_validate(3, 256) == dg.DG_OK
    assert dg.dg_commit_validate(3, 0) == dg.DG_ERR_INVALID_ARG
    assert dg.dg_commit_validate(3, 1025) == dg.DG_ERR_INVALID_ARG
    assert dg.dg_commit_validate(-1, 4) == dg.DG_ERR_INVALID_ARG
    assert dg.dg_slot_read_workspace(d, 512, 4, 1024, 4) > 0
    assert dg.dg_slot_read_workspace(d, 512, 4, 1024, 0) == 0


def test_label_count_rule():
    """sotaaz, 'The server takes at most 26 alternatives': 77 alternatives in one
    question are refused; up to 26 single-token labels A..Z are accepted."""
    dg = _lib_or_skip()
    assert dg.dg_check_label_count(26) == dg.DG_OK
    assert dg.dg_check_label_count(1) == dg.DG_OK
    assert dg.dg_check_label_count(27) == dg.DG_ERR_TOO_MANY_LABELS
    assert dg.dg_check_label_count(0) == dg.DG_ERR_INVALID_ARG
    with pytest.raises(ValueError, match=r"too many labels for 'intent': 77 > 26"):
        dg.check_alternatives("intent", [f"i{k}" for k in range(77)])
    dg.check_alternatives("urgent", ["yes", "no"])


def test_loop_rejects_bad_arguments_before_any_launch():
    """dg_denoise_loop checks its threshold (>= 0: the loop must progress), step
    counts, outputs, the p.E weights and the workspace size on the host; these
    calls carry fake device addresses and return before touching a device."""
    import ctypes
    dg = _lib_or_skip()
    L = dg.lib()
    d = _dims(dg)
    w_t = dg.make_weights(256, 256, 256, 256, 256, embed_t=256)
    launched = ctypes.c_int32(-1)

    def call(w=w_t, tau=1.0, max_steps=16, check_every=4, cs=2048, steps=4096, ws=8192,
             ws_bytes=1 << 40):
        return L.dg_denoise_loop(ctypes.byref(d), ctypes.byref(w), ctypes.byref(_kv(dg)), 1, 1024,
                                 None, 8.0, None, tau, max_steps, check_every, cs, steps,
                                 ctypes.byref(launched), None, ws, ws_bytes, None)

    assert call(tau=-0.5) == dg.DG_ERR_INVALID_ARG
    assert call(tau=float("nan")) == dg.DG_ERR_INVALID_ARG
    assert launched.value == 0
    assert call(max_steps=-1) == dg.DG_ERR_INVALID_ARG
    assert call(check_every=0) == dg.DG_ERR_INVALID_ARG
    assert call(cs=None) == dg.DG_ERR_INVALID_ARG
    assert call(steps=None) == dg.DG_ERR_INVALID_ARG
    assert call(w=_weights(dg)) == dg.DG_ERR_INVALID_ARG          # no embed_t for p.E
    need = dg.dg_denoise_loop_workspace(d, 1, 128)
    assert need > dg.dg_denoise_step_workspace(d, 1, 128) > 0
    assert call(ws_bytes=need - 1) == dg.DG_ERR_WORKSPACE
    assert "workspace" in dg.lib().dg_last_error().decode()


def test_staged_read_rejects_bad_stage_arrays_before_any_launch():
    """dg_slot_read_staged checks its host stage arrays first: stages 0/1 only,
    ask_if naming a stage-0 slot from a stage-1 slot, labels in [0, 26), at most
    DG_MAX_STAGED_SLOTS slots.  Fake device addresses: nothing is launched."""
    import ctypes
    dg = _lib_or_skip()
    L = dg.lib()
    d = _dims(dg)

    def call(stage, ask, lab, n=None):
        n = len(stage) if n is None else n
        arr = ctypes.c_int32 * max(len(stage), 1)
        st, ak, al = arr(*stage), arr(*ask), arr(*lab)     # alive for the whole call
        w, kv = _weights(dg), _kv(dg)
        return L.dg_slot_read_staged(ctypes.byref(d), ctypes.byref(w), ctypes.byref(kv), 1, 1024, n,
                                     2048, 4096, 6144, 8192, ctypes.addressof(st),
                                     ctypes.addressof(ak), ctypes.addressof(al), 8.0, None, 0.1, 4,
                                     *([1 << 20] * 7), 1 << 21, 16, None)

    I = dg.DG_ERR_INVALID_ARG
    assert call([0, 2], [-1, -1], [0, 0]) == I                # stage 2
    assert call([0, 1], [-1, 1], [0, 0]) == I                 # ask_if naming a stage-1 slot
    assert call([0, 1], [1, -1], [0, 0]) == I                 # ask_if on a stage-0 slot
    assert call([0, 1], [-1, 0], [0, 26]) == I                # label out of range
    assert call([0, 1], [-1, 5], [0, 0]) == I                 # slot out of range
    assert call([0] * 65, [-1] * 65, [0] * 65) == I           # too many slots
    # a valid schema gets past these checks (and fails on the tiny workspace)
    assert call([0, 1], [-1, 0], [0, 3]) == dg.DG_ERR_WORKSPACE


@pytest.mark.parametrize("dtype_name", ["DG_BF16", "DG_F32"])
def test_staged_workspace_covers_every_stage_size(dtype_name):
    """A two-stage read calls the one-pass read once per stage with that stage's
    slot count, inside its own workspace.  The one-pass read's workspace is not
    monotone in the slot count (speculated draws, split-K partials of the
    projections), so the staged workspace must hold the largest of 1..S."""
    dg = _lib_or_skip()
    dt = getattr(dg, dtype_name)
    cases = [
        dg.make_dims(2816, 8, 2, 512, 262144, 256, 128, 262143, dt),   # the headline model
        dg.make_dims(2816, 8, 2, 512, 4096, 256, 128, 4095, dt),       # wide heads, small vocabulary
        dg.make_dims(256, 4, 4, 64, 2048, 256, 16, 2047, dt),
    ]
    if dt == dg.DG_F32:
        cases = cases[2:]   # 512-wide heads are bf16 only
    for d in cases:
        for B, S, P, nd in [(1, 8, 2048, 4), (4, 12, 512, 3), (2, 26, 4096, 5)]:
            staged = dg.dg_slot_read_staged_workspace(d, B, S, P, nd)
            one = max(dg.dg_slot_read_workspace(d, B, n, P, nd) for n in range(1, S + 1))
            assert staged > one > 0, (B, S, P, nd)


def _headline(dg, **kw):
    base = dict(d_model=2816, n_q_heads=8, n_kv_heads=2, head_dim=512, vocab=262144,
                canvas=256, window=128, mask_id=262143, dtype="bf16")
    base.update(kw)
    return dg.make_dims(**base)


@pytest.mark.parametrize("which", ["step", "loop", "read", "read_full", "staged", "encode"])
@pytest.mark.parametrize("dims_kind", ["headline", "tiny"])
def test_workspace_queries_are_monotone_in_max_prompt(which, dims_kind):
    """A workspace sized for max_prompt = M must hold a call whose prompts are
    shorter (the call plans with prompt_kv.max_len <= M): every query is
    non-decreasing in max_prompt.  The split-KV plan rounds its chunk length,
    which can give more splits for a shorter prompt; the partials are sized by
    a bound that only grows, and the read also covers its one-pass order."""
    dg = _lib_or_skip()
    d = _headline(dg) if dims_kind == "headline" else _dims(dg)
    B = 1 if dims_kind == "headline" else 32
    q = {"step": lambda m: dg.dg_denoise_step_workspace(d, B, m),
         "loop": lambda m: dg.dg_denoise_loop_workspace(d, B, m),
         "read": lambda m: dg.dg_slot_read_workspace(d, B, 8, m, 4),
         "read_full": lambda m: dg.dg_slot_read_full_canvas_workspace(d, B, 8, m, 4),
         "staged": lambda m: dg.dg_slot_read_staged_workspace(d, B, 8, m, 4),
         "encode": lambda m: dg.dg_prefill_encode_workspace(d, B, m)}[which]
    lens = list(range(0, 4200, 7)) + list(range(4200, 120000, 997))
    prev = 0
    for m in lens:
        w = q(m)
        assert w > 0 or (which == "encode" and m == 0)   # no prompt: nothing to encode
        assert w >= prev, f"{which}: workspace({m}) = {w} < workspace of a shorter prompt ({prev})"
        prev = w


def test_noalloc_scratch_size_matches_the_header():
    dg = _lib_or_skip()
    src = open(HEADER).read()
    m = re.search(r"#define DG_NOALLOC_SCRATCH_BYTES \((\d+)u << (\d+)\)", src)
    assert m and int(m.group(1)) << int(m.group(2)) == dg.DG_NOALLOC_SCRATCH_BYTES


def test_encode_rejects_bad_arguments_before_any_launch():
    """dg_prefill_encode's checks run on the host before anything is launched."""
    dg = _lib_or_skip()
    d = _dims(dg)
    full = dg.make_weights(256, 256, 256, 256, 256)
    assert dg.dg_prefill_encode_workspace(d, 2, 0) == 0
    assert dg.dg_prefill_encode_workspace(d, 0, 700) == 0
    ws = dg.dg_prefill_encode_workspace(d, 2, 700)
    assert ws > dg.dg_prefill_encode_workspace(d, 2, 256) > 0
    L = dg.lib()

    def call(dims=d, w=full, batch=2, cu=1024, max_len=700, total=900, ids=2048, k=4096, v=8192,
             hidden=16384, attn=None, wsp=32768, wsb=ws):
        return L.dg_prefill_encode(dims, w, batch, cu, max_len, total, ids, k, v, hidden, attn, None,
                                   wsp, wsb, None)
    assert call(batch=-1) == dg.DG_ERR_INVALID_ARG
    assert call(max_len=-1) == dg.DG_ERR_INVALID_ARG
    assert call(total=-5) == dg.DG_ERR_INVALID_ARG
    assert call(cu=None) == dg.DG_ERR_INVALID_ARG
    assert call(ids=None) == dg.DG_ERR_INVALID_ARG
    assert call(k=None) == dg.DG_ERR_INVALID_ARG
    assert call(hidden=16388) == dg.DG_ERR_INVALID_ARG            # misaligned output
    assert call(w=dg.make_weights(256, 256, 256, 256, 0)) == dg.DG_ERR_INVALID_ARG   # no wo
    assert "wq, wo" in dg.dg_last_error()
    assert call(wsb=ws - 1) == dg.DG_ERR_WORKSPACE
    assert call(wsp=None) == dg.DG_ERR_WORKSPACE
    assert call(dims=_dims(dg, head_dim=128)) == dg.DG_ERR_UNSUPPORTED


def test_status_string_of_any_int():
    """A C caller may pass any int as a status: values outside the enumerators
    name no status."""
    dg = _lib_or_skip()
    L = dg.lib()
    f = L.dg_status_string
    f.restype = __import__("ctypes").c_char_p
    f.argtypes = [__import__("ctypes").c_int]
    assert f(0) == b"ok"
    for bad in (-2, -1, 6, 99, 2 ** 31 - 1):
        assert f(bad) == b"unknown status"
