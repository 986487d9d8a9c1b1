"""The library's host code under AddressSanitizer and UndefinedBehaviorSanitizer, on the
CPU: argument validation of every entry point (no launch on a refused call), the
saved-image header parser on truncated and corrupted images (Issue #67 "Path F format
v3: persist per-head INT8 KV scales", section Phased plan: the reader tells the
versions apart and refuses one without scales for int8), and the streamed window's
planner and map (random requests, refused arguments, a failed copy rolled back).

The host translation units are compiled host-only with the sanitizers and linked with
tests/host_sanitize/host_checks.cpp, which stubs the kernel launchers.  Runs only where
no GPU is visible (the driver hands fake pointers to the runtime's copy calls)."""
import hashlib
import os
import shutil
import subprocess

import pytest

ROOT = os.path.abspath(os.path.join(os.path.dirname(__file__), ".."))
CSRC = os.path.join(ROOT, "quantized_kv_cache_q8_amd", "csrc")
DRIVER = os.path.join(ROOT, "tests", "host_sanitize", "host_checks.cpp")
OUT = os.path.join(ROOT, "_build", "host_sanitize")
SOURCES = [os.path.join(CSRC, "api.hip"), os.path.join(CSRC, "window.hip")]


def _hipcc():
    for c in (shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if c and os.path.exists(c):
            return c
    pytest.skip("hipcc not found")


def _build():
    h = hashlib.sha256()
    for f in SOURCES + [DRIVER, os.path.join(CSRC, "kvq8_internal.h"),
                        os.path.join(ROOT, "include", "kvq8.h")]:
        h.update(open(f, "rb").read())
    exe = os.path.join(OUT, "host_checks_" + h.hexdigest()[:12])
    if os.path.exists(exe):
        return exe
    os.makedirs(OUT, exist_ok=True)
    hipcc = _hipcc()
    # host-only compilation; every sanitizer flag applies to the host side only
    san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
           "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", "-g", "-O1"]
    objs = []
    for src in SOURCES:
        obj = os.path.join(OUT, os.path.basename(src) + ".o")
        cmd = [hipcc, "-x", "hip", "--cuda-host-only", "-std=c++17", *san, "-c", src, "-o", obj]
        r = subprocess.run(cmd, capture_output=True, text=True)
        assert r.returncode == 0, r.stderr
        objs.append(obj)
    cmd = [hipcc, "-x", "hip", "--cuda-host-only", "-std=c++17", *san, DRIVER, "-x", "none",
           *objs, "-o", exe]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    return exe


@pytest.mark.skipif(os.path.exists("/dev/kfd"), reason="a GPU node is visible")
def test_host_code_under_sanitizers():
    exe = _build()
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=600)
    print(r.stdout[-4000:])
    if r.returncode == 3:
        pytest.skip("a GPU is visible to the HIP runtime")
    assert r.returncode == 0, r.stdout[-3000:] + r.stderr[-6000:]
    assert "ALL OK" in r.stdout
    assert "failed copy rolled back" in r.stdout
