"""Host-only AddressSanitizer run of the C ABI's validation layer.

The library sources are compiled with AddressSanitizer on their host code only (the device
code for gfx950 is built as usual and never runs), linked with tests/asan/abi_driver.cpp, and
run: every entry point is called with invalid
arguments (rejected before any HIP call) and the host-only entry points run in full.  A
read past an argument (e.g. a layer pattern) or any other memory error fails the run."""
import os
import subprocess
from concurrent.futures import ThreadPoolExecutor

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "dsa_lightning_indexer_scores_amd", "csrc")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

pytestmark = pytest.mark.skipif(not os.path.exists(HIPCC), reason="hipcc not available")


def test_abi_validation_under_address_sanitizer(tmp_path):
    srcs = sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith(".hip"))
    def compile_one(s):
        o = str(tmp_path / (os.path.basename(s) + ".o"))
        cmd = [HIPCC, "--offload-arch=gfx950", "-O1", "-g", "-std=c++17", "-fPIC", "-Xarch_host", "-fsanitize=address",
               "-fno-omit-frame-pointer", "-fno-honor-nans", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
               "-I", os.path.join(ROOT, "include"), "-c", s, "-o", o]
        r = subprocess.run(cmd, capture_output=True, text=True)
        assert r.returncode == 0, r.stderr[-3000:]
        return o

    with ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = list(ex.map(compile_one, srcs))
    exe = str(tmp_path / "abi_driver")
    cmd = [HIPCC, "--offload-arch=gfx950", "-O1", "-g", "-std=c++17", "-Xarch_host", "-fsanitize=address",
           "-fno-omit-frame-pointer",
           "-I", os.path.join(ROOT, "include"), "-x", "c++", os.path.join(ROOT, "tests", "asan", "abi_driver.cpp"),
           "-x", "none", *objs, "-o", exe]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-3000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0")
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=120)
    assert r.returncode == 0, r.stdout + r.stderr[-5000:]
    assert "all calls returned the expected status" in r.stdout
