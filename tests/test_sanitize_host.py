"""The C-ABI's host code built with AddressSanitizer and UndefinedBehaviorSanitizer
(host only: hipcc --offload-host-only, each -fsanitize after -Xarch_host), with
the kernel launchers replaced by counting stubs, then run on the CPU:
tests/sanitize/host_checks.cpp drives the argument checks, workspace queries
(monotone, and extreme sizes), status strings, per-thread error messages, and
every entry point with arguments it must reject before launching anything.
Any sanitizer report or failed check fails the test."""
import hashlib
import os
import re
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "slot_readout_amd", "csrc")
OUT = os.path.join(ROOT, "_build", "sanitize")
HOST_SOURCES = ["dg_api.cpp", "plan.cpp"]


def _hipcc():
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    return None


def _stubs():
    """A stub for every launcher declared in kernels.h: counts the call and
    returns hipErrorNotSupported."""
    src = open(os.path.join(CSRC, "kernels.h")).read()
    src = re.sub(r"//[^\n]*", "", src)
    decls = re.findall(r"hipError_t\s+(launch_\w+)\s*\(([^;]*?)\)\s*;", src, flags=re.S)
    assert decls, "no launcher declarations found"
    body = ['#include "kernels.h"', "static int g_launches = 0;",
            'extern "C" int dg_stub_launches(void) { return g_launches; }', "namespace dg {"]
    for name, args in decls:
        args = " ".join(args.split())
        body.append(f"hipError_t {name}({args}) {{ ++g_launches; return hipErrorNotSupported; }}")
    body.append("}  // namespace dg")
    return "\n".join(body) + "\n"


def _flags():
    return ["-x", "hip", "--offload-host-only", "-O1", "-g", "-fno-omit-frame-pointer", "-std=c++17",
            f"-I{os.path.join(ROOT, 'include')}", f"-I{CSRC}",
            "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
            "-Xarch_host", "-fno-sanitize-recover=undefined"]


def test_host_code_under_address_and_undefined_sanitizers():
    hipcc = _hipcc()
    if hipcc is None:
        pytest.skip("hipcc not available")
    os.makedirs(OUT, exist_ok=True)
    stub = os.path.join(OUT, "stubs.cpp")
    with open(stub, "w") as f:
        f.write(_stubs())
    srcs = [os.path.join(CSRC, s) for s in HOST_SOURCES] + [
        stub, os.path.join(ROOT, "tests", "sanitize", "host_checks.cpp")]
    h = hashlib.sha256()
    for s in srcs + [os.path.join(CSRC, "kernels.h"), os.path.join(CSRC, "common.h"),
                     os.path.join(ROOT, "include", "dg.h")]:
        h.update(open(s, "rb").read())
    exe = os.path.join(OUT, "host_checks_" + h.hexdigest()[:12])
    if not os.path.exists(exe):
        objs = []
        for s in srcs:
            o = os.path.join(OUT, os.path.basename(s) + ".o")
            r = subprocess.run([hipcc] + _flags() + ["-c", s, "-o", o], capture_output=True, text=True)
            assert r.returncode == 0, f"compiling {s}:\n{r.stderr[-3000:]}"
            objs.append(o)
        r = subprocess.run([hipcc, "--offload-host-only", "-Xarch_host", "-fsanitize=address",
                            "-Xarch_host", "-fsanitize=undefined", "-o", exe] + objs + ["-lpthread"],
                           capture_output=True, text=True)
        assert r.returncode == 0, f"linking:\n{r.stderr[-3000:]}"
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0:halt_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1", LSAN_OPTIONS="")
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=300)
    out = r.stdout + r.stderr
    assert "runtime error" not in out, out[-4000:]
    assert "AddressSanitizer" not in out and "LeakSanitizer" not in out, out[-4000:]
    assert r.returncode == 0, out[-4000:]
    assert "host checks passed" in out
