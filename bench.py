"""Throughput of the hot path on one MI355X.

A step = dg_denoise_step (attention, LM head, fused softmax/entropy, p.E
self-conditioning) + dg_commit + dg_slot_read (8 slots x 4 labels, first read
plus averaged noise draws) over one bf16 canvas of 256 tokens with a 2048-token
cached prompt: d_model 2816, 8 query / 2 KV heads x 512, window +-128, vocab
262,144.  Inputs are seeded and synthetic and already in HBM when timing
starts.  Each of the K timed steps carries one HIP event pair and nothing
else (value = K steps / their total time; median and p95 of the per-step
times beside it); K further steps with per-stage HIP events give the stage
breakdown and the dominant kernel's launch duration for the roofline.

After the headline steps the same process measures the other workloads, each
with its own roofline: the read in the whole-canvas order, the 110,707-token
cold long read, the ragged batch of 32 canvases and the 512-canvas structured
read batch; then the generation loop, prefill, two-stage read and FP8-head
legs, the achievable copy / matmul ceilings, and the CPU oracle on a sample.
Prints one JSON line.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline]
                    [--workload NAME] [--no-legs]
"""
import argparse
import ctypes
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
BF16_PEAK_TFLOPS = 2500.0      # MI355X dense bf16 MFMA
FP8_PEAK_TFLOPS = 5000.0       # MI355X dense fp8 MFMA
FP32_PEAK_TFLOPS = 157.3       # MI355X fp32 vector
WORKLOAD = "bf16_step"
LEG_STEPS = 100                # timed steps of each secondary workload

# Kernels whose operands reach LDS through direct-to-LDS loads: their FETCH_SIZE
# readings are not scaled by the plain-copy calibration (which uses ordinary
# vector loads), so no measured traffic is reported for them.
DMA_KERNELS = ("lmhead", "selfcond")


def _hip():
    L = ctypes.CDLL("libamdhip64.so.7")
    L.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
    L.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
    L.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
    L.hipEventDestroy.argtypes = [ctypes.c_void_p]
    return L


class Events:
    """A block of raw hipEvents (timing enabled), recorded on a given stream."""

    def __init__(self, hip, n):
        self.hip = hip
        self.arr = (ctypes.c_void_p * n)()
        for i in range(n):
            e = ctypes.c_void_p()
            assert hip.hipEventCreate(ctypes.byref(e)) == 0
            self.arr[i] = e
        self.n = n

    def record(self, i, stream):
        assert self.hip.hipEventRecord(self.arr[i], stream) == 0

    def ms(self, i, j):
        out = ctypes.c_float()
        assert self.hip.hipEventElapsedTime(ctypes.byref(out), self.arr[i], self.arr[j]) == 0
        return float(out.value)

    def sub(self, offset):
        return ctypes.cast(ctypes.byref(self.arr, offset * ctypes.sizeof(ctypes.c_void_p)),
                           ctypes.POINTER(ctypes.c_void_p))

    def destroy(self):
        for i in range(self.n):
            self.hip.hipEventDestroy(self.arr[i])


def attention_work(inp, queries=None, canvases=None):
    """Algorithmic bytes and flops of one attention launch: every prompt key and
    value once, the canvas k and v, and q and o of the queries (every canvas
    position, or `queries` per canvas); flops of QK^T and PV over the visible
    keys.  canvases: canvases per prompt (a read's draws share their prompt)."""
    dm = inp["dims"]
    C, Hq, Hkv, hd, W = dm.canvas, dm.n_q_heads, dm.n_kv_heads, dm.head_dim, dm.window
    es = 2 if dm.dtype == "bf16" else 4
    lens = inp["prompt_lens"].astype("int64")
    ncv = len(lens) * (canvases or 1)
    kv_bytes = int(lens.sum()) * Hkv * hd * 2 * es
    nq = C if queries is None else queries
    canvas_bytes = ncv * (2 * nq * Hq + 2 * C * Hkv) * hd * es
    if queries is None:
        win = sum(min(C, i + W + 1) - max(0, i - W) for i in range(C))   # visible canvas keys
        flops = 4.0 * Hq * hd * (C * float(lens.sum()) * (canvases or 1) + ncv * win)
    else:
        flops = 4.0 * Hq * hd * nq * (float(lens.sum()) * (canvases or 1) + ncv * min(C, 2 * W + 1))
    return kv_bytes + canvas_bytes, flops, kv_bytes


def kernel_source_hash():
    """Hash of the kernel sources (the .hip files and their headers; the host-side
    C-ABI layer does not change what a kernel moves)."""
    h = hashlib.sha256()
    for f in sorted(os.listdir(os.path.join(ROOT, "slot_readout_amd", "csrc"))):
        if not f.endswith((".hip", ".h")):
            continue
        with open(os.path.join(ROOT, "slot_readout_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def measured_traffic(kernel, workload):
    """HBM bytes per launch from the committed rocprofv3 counter summary of the
    workload, if it was taken on the current kernel sources; else None."""
    if kernel in DMA_KERNELS:
        return None
    path = os.path.join(ROOT, "profiles", f"counters_{workload}.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        c = json.load(f)
    if c.get("source_hash") != kernel_source_hash():
        return None
    k = c.get("kernels", {}).get(kernel)
    return None if k is None else k.get("hbm_bytes_per_launch")


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def cpu_baseline(inp):
    """The CPU oracle as it stands, timed on this host on the same workload."""
    import numpy as np
    import oracle
    from threadpoolctl import threadpool_info
    threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    t0 = time.perf_counter()
    st = oracle.denoise_step(inp)[0]
    t1 = time.perf_counter()
    oracle.commit_canvas(inp["canvas_ids"][0], st["conf"], st["entropy"], st["argmax"],
                         inp["dims"].mask_id, inp["tau"])
    t2 = time.perf_counter()
    rd = oracle.slot_read(inp)
    t3 = time.perf_counter()
    B, C, S = inp["batch"], inp["dims"].canvas, inp["slot_pos"].shape[1]
    total = t3 - t0
    return {
        "value": B * C / total, "unit": "canvas tokens/s", "cores": int(threads), "kind": "oracle",
        "sample": (f"one whole step of the same workload (one canvas) in float64 numpy: denoise "
                   f"step {t1 - t0:.2f} s + commit {t2 - t1:.3f} s + slot read of {S} slots "
                   f"({int(np.max(rd['draws_used']))} draws) {t3 - t2:.2f} s"),
        "seconds": round(total, 3), "cpu_model": cpu_model(),
    }


def loop_leg(dev, inp, stream, runs=3, check_every=16):
    """The multi-step loop (dg_denoise_loop: step, commit, p.E feedback until no
    mask id remains) from the workload's canvas, timed after the step bench; it
    synchronises the host every check_every steps.  Committed canvas tokens per
    second of wall time, median of `runs` complete loops."""
    import numpy as np
    import torch
    mask_id = inp["dims"].mask_id
    n_masked = int((inp["canvas_ids"] == mask_id).sum())
    times, out = [], None
    for _ in range(runs + 1):          # the first run warms up
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        out = dev.loop(tau=inp["tau"], check_every=check_every, stream=stream)
        torch.cuda.synchronize()
        times.append(time.perf_counter() - t0)
    t = float(np.median(times[1:]))
    steps = int(out["steps"].max().item())
    left = int((out["ids"] == mask_id).sum().item())
    return {"committed_tokens": n_masked - left, "steps": steps, "steps_launched": out["launched"],
            "ms": round(t * 1e3, 3), "ms_per_step": round(t * 1e3 / max(steps, 1), 4),
            "committed_tokens_per_s": round((n_masked - left) / t, 1), "check_every": check_every,
            "tau": inp["tau"]}


def timed_median(fn, runs=5):
    """Median HIP-event time (ms) of `runs` calls of fn after one warm-up call."""
    import numpy as np
    import torch
    ts = []
    for i in range(runs + 1):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        fn()
        e1.record()
        torch.cuda.synchronize()
        if i:
            ts.append(e0.elapsed_time(e1))
    return float(np.median(ts))


def prefill_leg(dev, inp, stream):
    """dg_prefill_kv of the workload's prompt tokens (seeded ids) into a scratch
    cache of the same shape, then the encoder-mode forward over the same
    prompts (dg_prefill_encode: cache rows, causal attention, block output)."""
    import numpy as np
    import torch
    from slot_readout_amd import dg
    dm = inp["dims"]
    n = int(inp["cu_seqlens"][-1])
    if n == 0:
        return None
    ids = torch.from_numpy(np.random.default_rng(7).integers(0, dm.vocab - 1, size=n)
                           .astype(np.int32)).cuda()
    k = torch.empty((n, dm.n_kv_heads, dm.head_dim), dtype=dev.tdt, device="cuda")
    v = torch.empty_like(k)
    t = timed_median(lambda: dg.dg_prefill_kv(dev.dims, dev.weights, n, ids, k, v, None, stream))
    out = {"tokens": n, "ms": round(t, 4), "tokens_per_s": round(n / (t * 1e-3), 1)}
    # encoder-mode forward: causal attention over each prompt
    cu = torch.from_numpy(inp["cu_seqlens"].astype(np.int32)).cuda()
    B, max_len = len(inp["cu_seqlens"]) - 1, int(inp["max_prompt"])
    hid = torch.empty((n, dm.d_model), dtype=dev.tdt, device="cuda")
    ws = torch.empty(max(dg.dg_prefill_encode_workspace(dev.dims, B, max_len), 256), dtype=torch.uint8,
                     device="cuda")
    te = timed_median(lambda: dg.dg_prefill_encode(dev.dims, dev.weights, B, cu, max_len, n, ids, k, v,
                                                   hid, None, None, ws, stream))
    lens = inp["prompt_lens"].astype(np.float64)
    causal_flops = 4.0 * dm.n_q_heads * dm.head_dim * float((lens * (lens + 1) / 2).sum())
    out["encode"] = {"ms": round(te, 4), "tokens_per_s": round(n / (te * 1e-3), 1),
                     "causal_attention_TFLOPs_of_call": round(causal_flops / (te * 1e-3) / 1e12, 1),
                     "note": "whole call (projections, causal attention, output projection); "
                             "TFLOP/s counts the causal attention's flops only"}
    return out


def staged_leg(dev, inp, stream):
    """dg_slot_read_staged of the workload's slots: the first half in stage 0, the
    second half in stage 1, whose first slot is asked only if stage-0 slot 0
    answers label 0."""
    S = dev.S
    stage = [0] * (S // 2) + [1] * (S - S // 2)
    ask, lab = [-1] * S, [0] * S
    if S >= 2:
        ask[S // 2] = 0
    out = dev.slot_outputs()
    t = timed_median(lambda: dev.slot_read_staged(stage, ask, lab, out=out, stream=stream))
    return {"slots": S, "stages": 2, "ms": round(t, 4), "slot_reads_per_s": round(dev.B * S / (t * 1e-3), 1),
            "reads_per_slot": int(out["draws_used"].max().item()) + 1}


def fp8_leg(hip, stream, K, W):
    """The headline step (step + commit + read) with the e4m3 copy of the LM head,
    weight-only (bf16 activations) and with FP8 activations (both operands e4m3
    on the FP8 matrix cores): step time, and the LM head's own time and rate
    against the FP8 and bf16 peaks."""
    out = {"lm_head": "e4m3 codes, per-row power-of-two scales"}
    for key, act in (("weight_only", False), ("fp8_activations", True)):
        w = Workload(WORKLOAD, hip, stream, lm_fp8=True, lm_fp8_act=act)
        t = w.run(K, W)
        nbytes, flops = kernel_work(w, lm_fp8=True, act=act)["lmhead"]
        lm_ms = t["stages"]["lmhead"]
        tf = flops / (lm_ms * 1e-3) / 1e12
        out[key] = {"ms_per_step": round(t["ms_per_step"], 4), "ms_median": t["ms_median"],
                    "canvas_tokens_per_s": round(w.dev.B * w.dev.C / (t["ms_per_step"] * 1e-3), 1),
                    "lmhead_ms": round(lm_ms, 4), "lmhead_TFLOPs": round(tf, 1),
                    "lmhead_frac_of_fp8_peak": round(tf / FP8_PEAK_TFLOPS, 4),
                    "lmhead_frac_of_bf16_peak": round(tf / BF16_PEAK_TFLOPS, 4),
                    "lmhead_GBs": round(nbytes / (lm_ms * 1e-3) / 1e9, 1),
                    "quantise_note": "activation quantisation is inside the lmhead stage" if act else None}
        w.release()
    return out


def achievable_peaks():
    """Measured ceilings on this GPU, beside the vendor peaks: a 1 GiB device-to-device
    copy (bytes read + written per second) and a bf16 8192^3 matrix product
    (contiguous operands)."""
    import torch
    x = torch.ones(1 << 28, dtype=torch.float32, device="cuda:0")
    y = torch.empty_like(x)
    a = torch.randn((8192, 8192), dtype=torch.bfloat16, device="cuda:0")
    b = torch.randn((8192, 8192), dtype=torch.bfloat16, device="cuda:0")

    def timed(fn, n):
        for _ in range(2):
            fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(n):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / n

    t_copy = timed(lambda: y.copy_(x), 10)
    t_mm = timed(lambda: torch.matmul(a, b), 10)
    out = {"copy_GBs": round(2 * x.numel() * 4 / (t_copy * 1e-3) / 1e9, 1),
           "matmul_bf16_TFLOPs": round(2 * 8192 ** 3 / (t_mm * 1e-3) / 1e12, 1)}
    del x, y, a, b
    return out


def _pct(xs, q):
    import numpy as np
    return round(float(np.percentile(np.asarray(xs), q)), 4)


class Workload:
    """Device-resident inputs of one workload and its timed step.

    kind: "step" (dg_denoise_step + dg_commit [+ dg_slot_read]) or "read"
    (dg_slot_read only).  full_canvas selects the read's whole-canvas order."""

    DESC = {
        "bf16_step": ("one canvas of 256 tokens, 2048-token cached prompt, d_model 2816, 8q/2kv "
                      "heads x 512, window +-128, vocab 262144, commit tau 2.0, slot read 8 slots x "
                      "4 labels (4 noise draws)"),
        "long_read": ("one canvas of 256 tokens over a 110,707-token cached prompt read cold, "
                      "d_model 256, 4 heads x 64, window +-128, vocab 2048; step + commit"),
        "ragged32": ("32 canvases of 256 tokens, prompts U{512..8192}, mask fractions U(0.1, 0.9), "
                     "d_model 256, 4 heads x 64, window +-16, vocab 2048; step + commit"),
        "reads512": ("512 canvases of 256 tokens, 1024-token prompts, a fixed skeleton with 4 slots, "
                     "k ~ U{2..26} labels, re-read above entropy 0.1 with 4 noise draws, d_model 256, "
                     "4 heads x 64, window +-16, vocab 2048; slot read"),
    }

    def __init__(self, name, hip, stream, lm_fp8=False, full_canvas=False, with_read=None,
                 lm_fp8_act=False):
        from slot_readout_amd import dg
        from slot_readout_amd.runtime import DeviceProblem
        from synth import config, make_inputs
        import torch
        self.name = name
        self.kind = "read" if name == "reads512" else "step"
        self.with_read = (name == "bf16_step") if with_read is None else with_read
        self.full_canvas = full_canvas
        self.cold = name == "long_read"
        self.hip, self.stream = hip, stream
        self.inp = make_inputs(config(name))
        self.dev = DeviceProblem(self.inp, device="cuda:0", with_lm_fp8=lm_fp8, lm_fp8_act=lm_fp8_act,
                                 with_embed_t=self.kind == "step")
        dev = self.dev
        self.so = dev.step_outputs(want_sc=True) if self.kind == "step" else None
        self.co = dev.commit_outputs() if self.kind == "step" else None
        self.ro = dev.slot_outputs()
        self.ws_step = (dev.workspace("step", dg.dg_denoise_step_workspace(dev.dims, dev.B, dev.max_prompt))
                        if self.kind == "step" else None)
        self.flush = None
        if self.cold:
            # a read sweep of 1 GiB evicts L2 and the 256 MB MALL without leaving
            # dirty lines behind, whose write-back would compete with the timed reads
            self.flush = torch.ones(1 << 27, dtype=torch.int64, device="cuda:0")
        torch.cuda.synchronize()

    def step(self, dbg=None, mark=lambda j: None):
        from slot_readout_amd import dg
        dev, inp, st = self.dev, self.inp, self.stream
        dm = inp["dims"]
        mark(0)
        if self.kind == "step":
            so, co = self.so, self.co
            dg.dg_denoise_step(dev.dims, dev.weights, dev.kv, dev.B, dev.canvas_ids, None,
                               inp["logit_scale"], None, so["conf"], so["entropy"], so["argmax"],
                               so["sc_out"], dbg, so["flags"], self.ws_step, st)
            mark(1)
            dg.dg_commit(dev.B, dev.C, dm.mask_id, dev.canvas_ids, so["conf"], so["entropy"],
                         so["argmax"], inp["tau"], co["mask"], co["out_ids"], co["n"], st)
            mark(2)
            if self.with_read:
                dev.slot_read(out=self.ro, stream=st, full_canvas=self.full_canvas)
        else:
            mark(1)
            mark(2)
            dev.slot_read(out=self.ro, stream=st, full_canvas=self.full_canvas)
        mark(3)

    def run(self, K, W, instrument=True):
        """W untimed steps, K timed steps (one event pair each), then, with
        instrument, K steps with per-stage events.  Returns the timing dict."""
        import numpy as np
        import torch
        from slot_readout_amd import dg
        hip, st = self.hip, self.stream
        n_st = 2 * dg.DG_N_STAGES
        span = Events(hip, 2 * K)
        for _ in range(W):
            if self.flush is not None:
                torch.amax(self.flush)
            self.step()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for k in range(K):
            if self.flush is not None:
                torch.amax(self.flush)
            span.record(2 * k, st)
            self.step()
            span.record(2 * k + 1, st)
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        per = [span.ms(2 * k, 2 * k + 1) for k in range(K)]
        if self.flush is not None:   # cache flushes sit between the steps: sum the steps
            total_ms = float(np.sum(per))
        else:
            total_ms = span.ms(0, 2 * K - 1)
        out = {"ms_per_step": total_ms / K, "ms_median": _pct(per, 50), "ms_p95": _pct(per, 95),
               "wall_s": wall, "steps": K}
        span.destroy()
        if instrument:
            marks = Events(hip, 4 * K)
            stage_ev = Events(hip, n_st * K)
            for k in range(K):
                if self.flush is not None:
                    torch.amax(self.flush)
                dbg = dg.make_debug(stage_events=stage_ev.sub(k * n_st)) if self.kind == "step" else None
                self.step(dbg, lambda j, k=k: marks.record(4 * k + j, st))
            torch.cuda.synchronize()
            out["step_ms"] = float(np.mean([marks.ms(4 * k, 4 * k + 1) for k in range(K)]))
            out["commit_ms"] = float(np.mean([marks.ms(4 * k + 1, 4 * k + 2) for k in range(K)]))
            out["read_ms"] = float(np.mean([marks.ms(4 * k + 2, 4 * k + 3) for k in range(K)]))
            if self.kind == "step":
                out["stages"] = {name: float(np.mean([stage_ev.ms(k * n_st + 2 * i, k * n_st + 2 * i + 1)
                                                      for k in range(K)]))
                                 for i, name in enumerate(dg.DG_STAGES)}
            marks.destroy()
            stage_ev.destroy()
        return out

    def release(self):
        import torch
        self.dev = self.so = self.co = self.ro = self.flush = None
        torch.cuda.empty_cache()


def kernel_work(w, lm_fp8=False, act=False):
    """(algorithmic bytes, flops) per launch of the step's main kernels."""
    inp, dm = w.inp, w.inp["dims"]
    B, C, V, d = inp["batch"], dm.canvas, dm.vocab, dm.d_model
    M, nvt = B * C, V // 256
    head_bytes = V * d + V * 4 if lm_fp8 else V * d * 2      # e4m3 codes + exponents
    h_bytes = M * d + M * 4 if act else M * d * 2             # e4m3 rows + exponents
    lm = (head_bytes + h_bytes + M * V * 2 + M * nvt * 16, 2.0 * M * V * d)
    sc = (d * V * 2 + M * V * 2 + M * nvt * 4 + M * d * 2, 2.0 * M * V * d)
    at = attention_work(inp)
    return {"lmhead": lm, "selfcond": sc, "attention": at[:2]}


KERNEL_NAMES = {"lmhead": "lmhead_kernel (S4+S5 tile statistics)",
                "selfcond": "scgemm_dma_kernel + sc_reduce4_kernel (S6)",
                "attention": "attn_kernel + attn_merge_kernel (S2)"}


def roofline_of(w, t, dominant=None, lm_fp8=False, act=False):
    """The dominant kernel's roofline from the instrumented stage times, and
    every stage's rate."""
    work = kernel_work(w, lm_fp8, act)
    st = t["stages"]
    dom = dominant or max(work, key=lambda k: st[k])
    nbytes, flops = work[dom]
    ms = st[dom]
    gbs = nbytes / (ms * 1e-3) / 1e9
    tflops = flops / (ms * 1e-3) / 1e12
    attn_bound = "hbm"
    roof = {"kernel": KERNEL_NAMES[dom], "bound": attn_bound, "achieved": round(gbs, 1),
            "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(gbs / HBM_PEAK_GBS, 4),
            "traffic": measured_traffic(dom, w.name),
            "algorithmic_bytes_per_launch": int(nbytes), "avg_launch_ms": round(ms, 4),
            "mfma_tflops": round(tflops, 1), "mfma_frac": round(tflops / BF16_PEAK_TFLOPS, 4)}
    if dom in DMA_KERNELS:
        roof["traffic_note"] = ("null: the kernel stages its operands with direct-to-LDS loads, for "
                                "which the plain-copy calibration of FETCH_SIZE does not hold")
    stages = {k: {"ms": round(st[k], 4), "GB/s": round(b / (st[k] * 1e-3) / 1e9, 1),
                  "TFLOP/s": round(f / (st[k] * 1e-3) / 1e12, 1)} for k, (b, f) in work.items()}
    return roof, stages


def leg_step_workload(name, hip, stream, K, W):
    """A step + commit workload with attention as its roofline kernel."""
    w = Workload(name, hip, stream)
    t = w.run(K, W)
    roof, stages = roofline_of(w, t, dominant="attention")
    B, C = w.inp["batch"], w.inp["dims"].canvas
    _, _, kv_bytes = attention_work(w.inp)
    out = {"workload": name + ": " + Workload.DESC[name], "metric": "canvas tokens/s",
           "value": round(B * C / (t["ms_per_step"] * 1e-3), 1),
           "ms_per_step": round(t["ms_per_step"], 4), "ms_median": t["ms_median"], "ms_p95": t["ms_p95"],
           "steps": K, "cold_cache": w.cold,
           "breakdown_ms": {"denoise_step": round(t["step_ms"], 4), "commit": round(t["commit_ms"], 4),
                            "stages": {k: round(v, 4) for k, v in t["stages"].items()}},
           "roofline": roof, "stage_roofline": stages,
           "prompt_kv_bytes": int(kv_bytes)}
    if name == "long_read":
        out["prefill"] = prefill_leg(w.dev, w.inp, stream)
    w.release()
    return out


def leg_reads512(hip, stream, K, W):
    """The 512-canvas structured read batch: slot reads per second.  The roofline
    is that of the whole read call (its kernels are not instrumented one by one;
    the per-kernel split is in the committed rocprofv3 summary) against HBM: the
    least traffic the call's work needs -- every prompt key and value once (the
    draws of a canvas differ from it only at the slots, so one pass over the
    prompt serves the first read and the draws), the base canvases' k and v at
    the rows within +-W of a slot, and the slot rows' q, o and the draws' slot
    k, v -- and the call's flops against the bf16 MFMA peak."""
    w = Workload("reads512", hip, stream)
    t = w.run(K, W)
    inp = w.inp
    B, S, nd = inp["batch"], inp["slot_pos"].shape[1], inp["n_draws"]
    du = w.ro["draws_used"]
    reread = int((du > 1).any(dim=1).sum().item())
    a1_bytes, a1_flops, kv = attention_work(inp, queries=S)
    dm = inp["dims"]
    hq, hkv = dm.n_q_heads * dm.head_dim, dm.n_kv_heads * dm.head_dim
    es = 2 if dm.dtype == "bf16" else 4
    ncv = B * (1 + (nd if reread else 0))
    # k, v are needed only at the canvas rows within +-W of a slot (once per
    # base canvas: the draws differ from it only at the slots); q and the output
    # projection at the slot rows of every canvas read
    import numpy as np
    sp = inp["slot_pos"]
    sp = sp.cpu().numpy() if hasattr(sp, "cpu") else np.asarray(sp)
    wnd = min(dm.window, dm.canvas - 1)
    pos = np.arange(dm.canvas)
    near = np.zeros((B, dm.canvas), dtype=bool)
    for s_ in range(S):
        q = sp[:, s_:s_ + 1]
        near |= (q >= 0) & (q < dm.canvas) & (np.abs(pos[None, :] - q) <= wnd)
    kv_rows = int(near.sum())
    passes_bytes = (kv + kv_rows * 2 * hkv * es + ncv * S * 2 * hq * es
                    + (B * nd * S * 2 * hkv * es if reread else 0))
    proj_flops = 2.0 * dm.d_model * (2 * hkv) * kv_rows + 4.0 * dm.d_model * hq * S * ncv
    head_flops = 2.0 * dm.vocab * dm.d_model * S * ncv
    flops = a1_flops * (1 + (nd if reread else 0)) + proj_flops + head_flops
    ms = t["ms_per_step"]
    gbs = passes_bytes / (ms * 1e-3) / 1e9
    tfl = flops / (ms * 1e-3) / 1e12
    out = {"workload": "reads512: " + Workload.DESC["reads512"], "metric": "slot reads/s",
           "value": round(B * S / (ms * 1e-3), 1), "ms_per_read_call": round(ms, 4),
           "ms_median": t["ms_median"], "ms_p95": t["ms_p95"], "steps": K,
           "canvases_reread": reread,
           "roofline": {"kernel": "dg_slot_read call (all kernels)", "bound": "hbm",
                        "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                        "frac": round(gbs / HBM_PEAK_GBS, 4), "traffic": None,
                        "algorithmic_bytes_per_call": int(passes_bytes), "kv_rows": kv_rows,
                        "mfma_tflops": round(tfl, 1), "mfma_frac": round(tfl / BF16_PEAK_TFLOPS, 4)}}
    w.release()
    return out


def leg_read_full_canvas(hip, stream, K, W):
    """The headline step with its read in the whole-canvas order."""
    w = Workload("bf16_step", hip, stream, full_canvas=True)
    t = w.run(K, W)
    B, C, S = w.inp["batch"], w.inp["dims"].canvas, w.dev.S
    out = {"ms_per_step": round(t["ms_per_step"], 4), "ms_median": t["ms_median"], "ms_p95": t["ms_p95"],
           "canvas_tokens_per_s": round(B * C / (t["ms_per_step"] * 1e-3), 1),
           "read_ms": round(t["read_ms"], 4),
           "slot_reads_per_s_of_read": round(B * S / (t["read_ms"] * 1e-3), 1)}
    w.release()
    return out


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--lm-fp8", action="store_true",
                    help="LM head from its e4m3 copy (weight-only FP8, bf16 activations)")
    ap.add_argument("--lm-fp8-act", action="store_true",
                    help="with --lm-fp8: FP8 activations too (per-row e4m3 h, FP8 matrix cores)")
    ap.add_argument("--no-legs", action="store_true",
                    help="the headline workload only (no secondary workloads or legs)")
    ap.add_argument("--workload", default=WORKLOAD,
                    choices=["bf16_step", "long_read", "ragged32", "reads512"],
                    help="profile one workload alone: bf16_step (default; step + commit + slot "
                         "read, then every leg), long_read and ragged32 (step + commit), "
                         "reads512 (slot read)")
    ap.add_argument("--full-canvas", action="store_true",
                    help="the read in the whole-canvas order (dg_slot_read_full_canvas)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="after the timed steps, copy 1 GiB device to device twice: a plain "
                         "copy of known size that scales the HBM byte counters of a "
                         "rocprofv3 --pmc FETCH_SIZE / WRITE_SIZE run")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU only: the hot path runs on a single GPU "
              "(the design document describes how it would shard); run with --gpus 1",
              file=sys.stderr)
        sys.exit(2)

    import torch
    from slot_readout_amd import dg

    dg.lib()   # fails loudly without the HIP library
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    torch.cuda.set_device(0)
    stream = torch.cuda.current_stream().cuda_stream
    hip = _hip()
    K, W = args.steps, args.warmup
    legs = not args.no_legs and args.workload == WORKLOAD

    if args.workload == "reads512":
        line = leg_reads512(hip, stream, K, W)
        print(json.dumps(line), flush=True)
        return

    t_in = time.perf_counter()
    args.lm_fp8 = args.lm_fp8 or args.lm_fp8_act
    w = Workload(args.workload, hip, stream, lm_fp8=args.lm_fp8, full_canvas=args.full_canvas,
                 lm_fp8_act=args.lm_fp8_act)
    setup_s = time.perf_counter() - t_in
    t = w.run(K, W)
    if args.copy_calibration:   # outside the timed region
        src = torch.ones(1 << 28, dtype=torch.float32, device="cuda:0")
        dst = torch.empty_like(src)
        for _ in range(2):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    inp, dev = w.inp, w.dev
    B, C, S = dev.B, dev.C, dev.S
    roof, stage_roof = roofline_of(w, t, lm_fp8=args.lm_fp8, act=args.lm_fp8_act)
    if args.lm_fp8:   # counters were taken with the bf16 head
        roof["traffic"] = None
    ms = t["ms_per_step"]
    _, _, kv_bytes = attention_work(inp)
    line = {
        "metric": "canvas tokens/s per denoise step + slot reads/s; % of MFMA/HBM roofline",
        "value": round(B * C / (ms * 1e-3), 1), "unit": "canvas tokens/s",
        "n_gpus": 1, "steps": K, "warmup": W, "ms_per_step": round(ms, 4),
        "ms_median": t["ms_median"], "ms_p95": t["ms_p95"],
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic (seeded; weights N(0,0.02), prompt K/V N(0,1))",
        "config": {"workload": args.workload + ": " + Workload.DESC[args.workload], "batch": B,
                   "canvas": C, "prompt": int(inp["max_prompt"]), "slots": S if w.with_read else 0,
                   "cold_cache": bool(w.cold),
                   "read_order": "whole canvas" if args.full_canvas else "slot rows",
                   "lm_head": ("e4m3 head and e4m3 activations, per-row power-of-two scales"
                               if args.lm_fp8_act else
                               "e4m3 codes, per-row power-of-two scales (weight-only FP8)")
                   if args.lm_fp8 else "bf16"},
        "slot_reads_per_s": round(B * S / (ms * 1e-3), 1) if w.with_read else None,
        "breakdown_ms": {"pass": "K further steps with per-stage HIP events, after the timed steps",
                         "denoise_step": round(t["step_ms"], 4), "commit": round(t["commit_ms"], 4),
                         "slot_read": round(t["read_ms"], 4),
                         "stages": {k: round(v, 4) for k, v in t["stages"].items()}},
        "roofline": roof,
        "stage_roofline": stage_roof,
        "attention_kv_read": {"kv_bytes": int(kv_bytes), "ms": round(t["stages"]["attention"], 4),
                              "hbm_frac": stage_roof["attention"]["GB/s"] / HBM_PEAK_GBS},
        "host_wall_s": round(t["wall_s"], 3), "setup_s": round(setup_s, 1),
    }
    if w.with_read:
        line["read_only"] = {"ms": round(t["read_ms"], 4),
                             "slot_reads_per_s": round(B * S / (t["read_ms"] * 1e-3), 1)}
    peaks = achievable_peaks()
    roof["achievable"] = dict(peaks, frac_of_copy=round(roof["achieved"] / peaks["copy_GBs"], 4),
                              mfma_frac_of_matmul=round(roof["mfma_tflops"] / peaks["matmul_bf16_TFLOPs"], 4))
    if legs:
        line["loop"] = loop_leg(dev, inp, stream)
        line["prefill"] = prefill_leg(dev, inp, stream)
        line["staged_read"] = staged_leg(dev, inp, stream)
    elif args.workload == "long_read" and not args.no_legs:
        line["prefill"] = prefill_leg(dev, inp, stream)
    cpu = None
    if legs and not args.no_cpu_baseline:
        cpu = cpu_baseline(inp)
    w.release()
    if legs:
        nl = min(K, LEG_STEPS)
        line["read_full_canvas"] = leg_read_full_canvas(hip, stream, nl, W)
        if not args.lm_fp8:
            line["fp8_head_step"] = fp8_leg(hip, stream, nl, W)
        line["workloads"] = {
            "long_read": leg_step_workload("long_read", hip, stream, nl, W),
            "ragged32": leg_step_workload("ragged32", hip, stream, nl, W),
            "reads512": leg_reads512(hip, stream, nl, W),
        }
    line["cpu_baseline"] = cpu
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
