"""Compile the gfx950 HIP kernels and the C-ABI layer into slot_readout_amd/libdg.so.

Usage: python -m slot_readout_amd.build   (or build() from Python)
"""
import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
OUT = os.path.join(PKG, "libdg.so")
BUILD_DIR = os.path.join(ROOT, "_build")

SOURCES = ["gemm.hip", "attention.hip", "vocab_commit.hip", "slot.hip", "encode.hip", "noalloc.hip",
           "plan.cpp", "dg_api.cpp"]
ARCH = "gfx950"


def hipcc():
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found (ROCm is required to build the HIP library)")


def common_flags():
    return [f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", f"-I{INCLUDE}",
            # packed fp32 vector ops are kept out of the generated code
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            # MFMA results stay in VGPRs (no AGPR round trips when the accumulators
            # are also touched by vector ALU code, e.g. the softmax rescale)
            "-mllvm", "-amdgpu-mfma-vgpr-form",
            "-Wall", "-Wno-unused-result"]


def _compile(src):
    obj = os.path.join(BUILD_DIR, os.path.basename(src) + ".o")
    cmd = [hipcc()] + common_flags() + ["-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    msgs = "\n".join(l for l in (r.stdout + r.stderr).splitlines()
                     if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"compiling {src} failed:\n{msgs}")
    return obj, msgs


def build(verbose: bool = False) -> str:
    """Compile every source and link libdg.so; returns the library path."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    with ThreadPoolExecutor(max_workers=min(len(SOURCES), os.cpu_count() or 4)) as ex:
        results = list(ex.map(_compile, SOURCES))
    for _, msgs in results:
        if verbose and msgs.strip():
            print(msgs)
    tmp = OUT + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp] + [o for o, _ in results]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"linking libdg.so failed:\n{r.stdout}{r.stderr}")
    os.replace(tmp, OUT)
    if verbose:
        print(f"built {OUT}")
    return OUT


if __name__ == "__main__":
    build(verbose="-q" not in sys.argv)
