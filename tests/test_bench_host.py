"""bench.py's host-side contract, without a GPU: one GPU only, and HBM traffic
taken from the committed counter summaries only while they describe the
current kernel sources."""
import json
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)


def test_more_than_one_gpu_is_refused_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


def test_traffic_only_for_the_current_kernel_sources():
    import bench
    h = bench.kernel_source_hash()
    assert len(h) == 16 and h == bench.kernel_source_hash()
    for w in ("long_read", "ragged32"):
        path = os.path.join(ROOT, "profiles", f"counters_{w}.json")
        with open(path) as f:
            c = json.load(f)
        for kern in c["kernels"]:
            got = bench.measured_traffic(kern, w)
            if kern in bench.DMA_KERNELS:
                # direct-to-LDS loads: the copy calibration does not apply
                assert got is None
            elif c["source_hash"] == h:
                assert got == c["kernels"][kern]["hbm_bytes_per_launch"] and got > 0
            else:
                assert got is None
    # the vocabulary GEMMs stage through direct-to-LDS loads: never a calibrated figure
    for kern in ("lmhead", "selfcond"):
        assert kern in bench.DMA_KERNELS and bench.measured_traffic(kern, "bf16_step") is None
    assert bench.measured_traffic("no_such_kernel", "bf16_step") is None
    assert bench.measured_traffic("selfcond", "no_such_workload") is None


def test_attention_work_counts():
    """Algorithmic attention work of the long read: 110,707 prompt keys and
    values read once (bf16, 4 kv heads x 64), q/o and canvas k/v of 256 rows,
    and 4 flops per (query, key, head, dim) for QK^T and PV over the prompt
    plus the +-128 window."""
    import bench
    from synth import config, make_inputs
    inp = make_inputs(config("long_read"), prompt_override=("fixed", 110707))
    nbytes, flops, kv = bench.attention_work(inp)
    assert kv == 110707 * 4 * 64 * 2 * 2
    assert nbytes == kv + 256 * (2 * 4 + 2 * 4) * 64 * 2
    win = sum(min(256, i + 129) - max(0, i - 128) for i in range(256))
    assert flops == 4.0 * 4 * 64 * (256 * 110707 + win)
