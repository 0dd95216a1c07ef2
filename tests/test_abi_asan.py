"""CPU tier: the C ABI's host code under AddressSanitizer and
UndefinedBehaviorSanitizer.

Every library source is compiled (device code unchanged) with
-fsanitize=address,undefined placed after -Xarch_host, linked with
tests/abi_asan_driver.cpp, and run: every validation path with bad pointers,
alignments, enums, shapes and workspaces, the workspace queries at the edges
of their ranges (including sizes near 2^40 that must not overflow), the delta
cache's bookkeeping, and valid calls that reach a launch and fail for want of
a device.  The run must report no sanitizer error and every status must be
the expected one."""
import concurrent.futures as cf
import glob
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HIPCC = "/opt/rocm/bin/hipcc"


def test_abi_host_code_under_asan_and_ubsan(tmp_path):
    if not os.path.exists(HIPCC):
        pytest.skip("hipcc not available")
    san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
           "-Xarch_host", "-fno-omit-frame-pointer", "-Xarch_host", "-fno-sanitize-recover=undefined"]
    srcs = sorted(glob.glob(os.path.join(ROOT, "tenant_fine_tune_amd", "csrc", "*.hip")) +
                  glob.glob(os.path.join(ROOT, "tenant_fine_tune_amd", "csrc", "*.cpp")))
    srcs.append(os.path.join(ROOT, "tests", "abi_asan_driver.cpp"))

    def comp(src):
        obj = str(tmp_path / (os.path.basename(src) + ".o"))
        r = subprocess.run([HIPCC, "-O1", "-g", "-std=c++17", "-fPIC", "-x", "hip",
                            "--offload-arch=gfx950", *san, "-I", os.path.join(ROOT, "include"), "-c", src, "-o", obj],
                           capture_output=True, text=True, timeout=600)
        assert r.returncode == 0, r.stderr[-3000:]
        return obj

    with cf.ThreadPoolExecutor(max_workers=min(8, os.cpu_count() or 1)) as ex:
        objs = list(ex.map(comp, srcs))
    exe = str(tmp_path / "abi_driver")
    r = subprocess.run([HIPCC, "--offload-arch=gfx950", *san, *objs, "-o", exe], capture_output=True, text=True,
                       timeout=600)
    assert r.returncode == 0, r.stderr[-3000:]
    env = {**os.environ, "ASAN_OPTIONS": "detect_leaks=0:abort_on_error=0:halt_on_error=1",
           "UBSAN_OPTIONS": "halt_on_error=1:print_stacktrace=1"}
    run = subprocess.run([exe], capture_output=True, text=True, timeout=600, env=env)
    out = run.stdout + run.stderr
    assert "AddressSanitizer" not in out and "runtime error" not in out, out[-4000:]
    assert run.returncode == 0, out[-4000:]
    assert "abi driver: 0 failures" in run.stdout
