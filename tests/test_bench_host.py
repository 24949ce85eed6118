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
    for w in ("bf16_step", "long_read", "ragged32"):
        path = os.path.join(ROOT, "profiles", f"counters_{w}.json")
        with open(path) as f:
            c = json.load(f)
        kern = next(iter(c["kernels"]))
        got = bench.measured_traffic(kern, w)
        if c["source_hash"] == h:
            assert got == c["kernels"][kern]["hbm_bytes_per_launch"] and got > 0
        else:
            assert got is None
    assert bench.measured_traffic("no_such_kernel", "bf16_step") is None
    assert bench.measured_traffic("selfcond", "no_such_workload") is None
