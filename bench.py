"""Throughput of one full pass of the hot path on one MI355X.

A step = dg_denoise_step (attention, LM head, fused softmax/entropy, p.E
self-conditioning) + dg_commit + dg_slot_read (8 slots x 4 labels, first read
plus averaged noise draws) over one bf16 canvas of 256 tokens with a 2048-token
cached prompt: d_model 2816, 8 query / 2 KV heads x 512, window +-128, vocab
262,144.  Inputs are seeded and synthetic and already in HBM when timing
starts.  The K timed steps carry one HIP event pair each and no other
instrumentation; K further steps with per-stage HIP events give the stage
breakdown and the roofline kernel's launch duration.  Prints one JSON line.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline]
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
WORKLOAD = "bf16_step"


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


def attention_work(inp):
    """Algorithmic bytes and flops of the attention stage (all canvases)."""
    dm = inp["dims"]
    C, Hq, Hkv, hd, W = dm.canvas, dm.n_q_heads, dm.n_kv_heads, dm.head_dim, dm.window
    es = 2 if dm.dtype == "bf16" else 4
    lens = inp["prompt_lens"].astype("int64")
    kv_bytes = int(lens.sum()) * Hkv * hd * 2 * es
    canvas_bytes = len(lens) * C * (2 * Hq + 2 * Hkv) * hd * es      # q, o, canvas k, v
    win = sum(min(C, i + W + 1) - max(0, i - W) for i in range(C))    # visible canvas keys
    flops = 4.0 * Hq * hd * (C * float(lens.sum()) + len(lens) * win)
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
    path = os.path.join(ROOT, "profiles", f"counters_{workload}.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        c = json.load(f)
    if c.get("source_hash") != kernel_source_hash():
        return None
    k = c.get("kernels", {}).get(kernel)
    return None if k is None else k.get("hbm_bytes_per_launch")


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
        "sample": (f"the whole step of the same workload in float64 numpy: denoise step "
                   f"{t1 - t0:.2f} s + commit {t2 - t1:.3f} s + slot read of {S} slots "
                   f"({int(np.max(rd['draws_used']))} draws) {t3 - t2:.2f} s"),
        "seconds": round(total, 3),
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


def prefill_leg(dev, inp, stream, runs=5):
    """dg_prefill_kv of the workload's prompt tokens (seeded ids) into a scratch
    cache of the same shape, timed with HIP events after the step bench;
    median of `runs` calls after one warm-up call."""
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
    ts = []
    for i in range(runs + 1):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        dg.dg_prefill_kv(dev.dims, dev.weights, n, ids, k, v, None, stream)
        e1.record()
        torch.cuda.synchronize()
        if i:
            ts.append(e0.elapsed_time(e1))
    t = float(np.median(ts))
    return {"tokens": n, "ms": round(t, 4), "tokens_per_s": round(n / (t * 1e-3), 1)}


def staged_leg(dev, inp, stream, runs=5):
    """dg_slot_read_staged of the workload's slots: the first half in stage 0, the
    second half in stage 1, whose first slot is asked only if stage-0 slot 0
    answers label 0; median of `runs` calls after one warm-up call."""
    import numpy as np
    import torch
    S = dev.S
    stage = [0] * (S // 2) + [1] * (S - S // 2)
    ask, lab = [-1] * S, [0] * S
    if S >= 2:
        ask[S // 2] = 0
    out = dev.slot_outputs()
    ts = []
    for i in range(runs + 1):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        dev.slot_read_staged(stage, ask, lab, out=out, stream=stream)
        e1.record()
        torch.cuda.synchronize()
        if i:
            ts.append(e0.elapsed_time(e1))
    t = float(np.median(ts))
    return {"slots": S, "stages": 2, "ms": round(t, 4), "slot_reads_per_s": round(dev.B * S / (t * 1e-3), 1),
            "reads_per_slot": int(out["draws_used"].max().item()) + 1}


def fp8_leg(inp, stream, K=20, W=3):
    """The same step (step + commit + read) with the e4m3 copy of the LM head."""
    import numpy as np
    import torch
    from slot_readout_amd import dg
    from slot_readout_amd.runtime import DeviceProblem
    dev = DeviceProblem(inp, device="cuda:0", with_lm_fp8=True)
    dm = inp["dims"]
    so, co, ro = dev.step_outputs(want_sc=True), dev.commit_outputs(), dev.slot_outputs()
    ws = dev.workspace("step", dg.dg_denoise_step_workspace(dev.dims, dev.B, dev.max_prompt))

    def step():
        dg.dg_denoise_step(dev.dims, dev.weights, dev.kv, dev.B, dev.canvas_ids, None,
                           inp["logit_scale"], None, so["conf"], so["entropy"], so["argmax"],
                           so["sc_out"], None, so["flags"], ws, stream)
        dg.dg_commit(dev.B, dev.C, dm.mask_id, dev.canvas_ids, so["conf"], so["entropy"],
                     so["argmax"], inp["tau"], co["mask"], co["out_ids"], co["n"], stream)
        dev.slot_read(out=ro, stream=stream)

    for _ in range(W):
        step()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(K):
        step()
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / K
    del dev
    return {"lm_head": "e4m3 codes, per-row power-of-two scales", "ms_per_step": round(ms, 4),
            "canvas_tokens_per_s": round(dev_tokens(inp) / (ms * 1e-3), 1)}


def dev_tokens(inp):
    return inp["batch"] * inp["dims"].canvas


def achievable_peaks():
    """Measured ceilings on this GPU, beside the vendor peaks: a 1 GiB device-to-device
    copy (bytes read + written per second) and a bf16 8192^3 matrix product
    (contiguous operands).  Taken after the timed steps."""
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


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=30)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--lm-fp8", action="store_true",
                    help="LM head from its e4m3 copy (weight-only FP8, bf16 activations)")
    ap.add_argument("--no-loop", action="store_true",
                    help="skip the multi-step generation loop leg (measured after the timed steps)")
    ap.add_argument("--workload", default=WORKLOAD,
                    choices=["bf16_step", "long_read", "ragged32"],
                    help="bf16_step (default) times step + commit + slot read; long_read and "
                         "ragged32 time step + commit and report the attention stage")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="after the timed steps, copy 1 GiB device to device twice: a plain "
                         "copy of known size that scales the HBM byte counters of a "
                         "rocprofv3 --pmc FETCH_SIZE / WRITE_SIZE run")
    ap.add_argument("--cold", action="store_true",
                    help="evict the caches (read 1 GiB) before every timed step; the default "
                         "for long_read, whose prompt KV would otherwise sit in the 256 MB MALL")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU only: the hot path runs on a single GPU "
              "(the design document describes how it would shard); run with --gpus 1",
              file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch
    from slot_readout_amd import dg
    from slot_readout_amd.runtime import DeviceProblem
    from synth import config, make_inputs

    dg.lib()   # fails loudly without the HIP library
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    torch.cuda.set_device(0)
    workload = args.workload
    cold = args.cold or workload == "long_read"
    with_read = workload == "bf16_step"
    cfg = config(workload)
    t_in = time.perf_counter()
    inp = make_inputs(cfg)
    dev = DeviceProblem(inp, device="cuda:0", with_lm_fp8=args.lm_fp8)
    dm = inp["dims"]
    B, C, S, V, d = dev.B, dev.C, dev.S, dm.vocab, dm.d_model
    stream = torch.cuda.current_stream().cuda_stream
    so = dev.step_outputs(want_sc=True)
    co = dev.commit_outputs()
    ro = dev.slot_outputs()
    hip = _hip()
    K, W = args.steps, args.warmup
    n_st = 2 * dg.DG_N_STAGES
    # The metric's K steps carry one event pair each and nothing else; a second
    # pass of K steps records the per-stage events (each record adds about 3 us,
    # so they are kept out of the metric) for the breakdown and the roofline.
    span = Events(hip, 2 * K)
    marks = Events(hip, 4 * K)
    stage_ev = Events(hip, n_st * K)
    dbg_per_step = [dg.make_debug(stage_events=stage_ev.sub(k * n_st)) for k in range(K)]
    ws_step = dev.workspace("step", dg.dg_denoise_step_workspace(dev.dims, B, dev.max_prompt))

    flush = None
    if cold:
        # a read sweep of 1 GiB evicts L2 and the 256 MB MALL without leaving dirty
        # lines behind, whose write-back would otherwise compete with the timed reads
        flush = torch.ones(1 << 27, dtype=torch.int64, device="cuda:0")
        torch.cuda.synchronize()

    def one_step(k=None, instrumented=False):
        """k: the step's slot in the event blocks (None: warm-up)."""
        mark = (lambda j: marks.record(4 * k + j, stream)) if instrumented and k is not None else (lambda j: None)
        dbg = dbg_per_step[k] if instrumented and k is not None else None
        if flush is not None:
            torch.amax(flush)
        if k is not None and not instrumented:
            span.record(2 * k, stream)
        mark(0)
        dg.dg_denoise_step(dev.dims, dev.weights, dev.kv, B, dev.canvas_ids, None,
                           inp["logit_scale"], None, so["conf"], so["entropy"], so["argmax"],
                           so["sc_out"], dbg, so["flags"], ws_step, stream)
        mark(1)
        dg.dg_commit(B, C, dm.mask_id, dev.canvas_ids, so["conf"], so["entropy"], so["argmax"],
                     inp["tau"], co["mask"], co["out_ids"], co["n"], stream)
        mark(2)
        if with_read:
            dev.slot_read(out=ro, stream=stream)
        mark(3)
        if k is not None and not instrumented:
            span.record(2 * k + 1, stream)

    for _ in range(W):
        one_step()
    torch.cuda.synchronize()
    setup_s = time.perf_counter() - t_in
    t0 = time.perf_counter()
    for k in range(K):
        one_step(k)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    for k in range(K):   # instrumented pass, outside the metric
        one_step(k, instrumented=True)
    torch.cuda.synchronize()
    if args.copy_calibration:   # outside the timed region
        src = torch.ones(1 << 28, dtype=torch.float32, device="cuda:0")
        dst = torch.empty_like(src)
        for _ in range(2):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    if cold:   # cache flushes sit between the steps: sum the steps themselves
        ms_per_step = float(np.mean([span.ms(2 * k, 2 * k + 1) for k in range(K)]))
    else:
        ms_per_step = span.ms(0, 2 * K - 1) / K
    step_ms = float(np.mean([marks.ms(4 * k, 4 * k + 1) for k in range(K)]))
    commit_ms = float(np.mean([marks.ms(4 * k + 1, 4 * k + 2) for k in range(K)]))
    read_ms = float(np.mean([marks.ms(4 * k + 2, 4 * k + 3) for k in range(K)]))
    stages = {}
    for i, name in enumerate(dg.DG_STAGES):
        stages[name] = float(np.mean([stage_ev.ms(k * n_st + 2 * i, k * n_st + 2 * i + 1)
                                      for k in range(K)]))
    M = B * C
    nvt = V // 256
    # algorithmic work per launch of the two vocabulary-sized kernels
    head_bytes = V * d + V * 4 if args.lm_fp8 else V * d * 2      # e4m3 codes + exponents
    lm_bytes = head_bytes + M * d * 2 + M * V * 2 + M * nvt * 16
    lm_flops = 2.0 * M * V * d
    sc_bytes = d * V * 2 + M * V * 2 + M * nvt * 4 + M * d * 2
    sc_flops = 2.0 * M * V * d
    at_bytes, at_flops, kv_bytes = attention_work(inp)
    cand = {"lmhead": (stages["lmhead"], lm_bytes, lm_flops),
            "selfcond": (stages["selfcond"], sc_bytes, sc_flops),
            "attention": (stages["attention"], at_bytes, at_flops)}
    names = {"lmhead": "lmhead_kernel (S4+S5 tile statistics)",
             "selfcond": "scgemm_dma_kernel + sc_reduce_kernel (S6)",
             "attention": "attn_kernel + attn_merge_kernel (S2)"}
    dom = max(cand, key=lambda k: cand[k][0])
    t_ms, nbytes, flops = cand[dom]
    achieved_gbs = nbytes / (t_ms * 1e-3) / 1e9
    roofline = {"kernel": names[dom],
                "bound": "hbm", "achieved": round(achieved_gbs, 1), "peak": HBM_PEAK_GBS,
                "unit": "GB/s", "frac": round(achieved_gbs / HBM_PEAK_GBS, 4),
                "traffic": measured_traffic(dom, workload),
                "algorithmic_bytes_per_launch": int(nbytes), "avg_launch_ms": round(t_ms, 4),
                "mfma_tflops": round(flops / (t_ms * 1e-3) / 1e12, 1),
                "mfma_frac": round(flops / (t_ms * 1e-3) / 1e12 / BF16_PEAK_TFLOPS, 4)}
    stage_roof = {}
    for name, (tm, nb, fl) in cand.items():
        stage_roof[name] = {"ms": round(tm, 4), "GB/s": round(nb / (tm * 1e-3) / 1e9, 1),
                            "TFLOP/s": round(fl / (tm * 1e-3) / 1e12, 1)}

    value = M / (ms_per_step * 1e-3)
    wl_desc = {
        "bf16_step": (f"bf16_step: one canvas of 256 tokens, 2048-token cached prompt, d_model 2816, "
                      f"8q/2kv heads x 512, window +-128, vocab 262144, commit tau 2.0, slot read "
                      f"8 slots x 4 labels (4 noise draws)"),
        "long_read": ("long_read: one canvas of 256 tokens over a 110,707-token cached prompt read "
                      "cold, d_model 256, 4 heads x 64, window +-128, vocab 2048; step + commit"),
        "ragged32": ("ragged32: 32 canvases of 256 tokens, prompts U{512..8192}, d_model 256, "
                     "4 heads x 64, window +-16, vocab 2048; step + commit"),
    }[workload]
    line = {
        "metric": "canvas tokens/s per denoise step + slot reads/s; % of MFMA/HBM roofline",
        "value": round(value, 1), "unit": "canvas tokens/s",
        "n_gpus": 1, "steps": K, "warmup": W, "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic (seeded; weights N(0,0.02), prompt K/V N(0,1))",
        "config": {"workload": wl_desc, "batch": B, "canvas": C,
                   "prompt": int(inp["max_prompt"]), "slots": S if with_read else 0,
                   "cold_cache": bool(cold),
                   "lm_head": "e4m3 codes, per-row power-of-two scales (weight-only FP8)"
                   if args.lm_fp8 else "bf16"},
        "slot_reads_per_s": round(B * S / (ms_per_step * 1e-3), 1) if with_read else None,
        "breakdown_ms": {"pass": "K further steps with per-stage HIP events, after the timed steps",
                         "denoise_step": round(step_ms, 4), "commit": round(commit_ms, 4),
                         "slot_read": round(read_ms, 4),
                         "stages": {k: round(v, 4) for k, v in stages.items()}},
        "roofline": roofline,
        "stage_roofline": stage_roof,
        "attention_kv_read": {"kv_bytes": int(kv_bytes), "ms": round(stages["attention"], 4),
                              "GB/s": round(at_bytes / (stages["attention"] * 1e-3) / 1e9, 1),
                              "hbm_frac": round(at_bytes / (stages["attention"] * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)},
        "host_wall_s": round(wall, 3), "setup_s": round(setup_s, 1),
    }
    marks.destroy()
    span.destroy()
    if args.lm_fp8:   # counters were taken with the bf16 head
        line["roofline"]["traffic"] = None
    peaks = achievable_peaks()
    roof = line["roofline"]
    roof["achievable"] = dict(peaks, frac_of_copy=round(roof["achieved"] / peaks["copy_GBs"], 4),
                              mfma_frac_of_matmul=round(roof["mfma_tflops"] / peaks["matmul_bf16_TFLOPs"], 4))
    if not args.no_loop and workload == WORKLOAD:
        line["loop"] = loop_leg(dev, inp, stream)
    if workload in ("bf16_step", "long_read"):
        line["prefill"] = prefill_leg(dev, inp, stream)
    if workload == WORKLOAD:
        line["staged_read"] = staged_leg(dev, inp, stream)
        if not args.lm_fp8:
            line["fp8_head_step"] = fp8_leg(inp, stream)
    stage_ev.destroy()
    if not args.no_cpu_baseline and workload == WORKLOAD:
        line["cpu_baseline"] = cpu_baseline(inp)
    else:
        line["cpu_baseline"] = None
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
