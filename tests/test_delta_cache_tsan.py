"""CPU tier: the delta cache under ThreadSanitizer.

tests/cache_stress.cpp drives the cache from 8 threads (hits, misses, joins
of in-flight loads, evictions, refused requests and loader failures) with a
host-side fake loader; it is built with g++ -fsanitize=thread together with
the cache's source and must finish with no race report and every acquired
slot holding its variant's bytes.  A second scenario (three variants, one
slot, a loader that never fails) makes callers that joined a successful load
often find the variant evicted again when they wake; none may report a
failure.  Host code only: nothing here touches a GPU.
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_delta_cache_has_no_data_race(tmp_path):
    if shutil.which("g++") is None or not os.path.exists("/opt/rocm/include/hip/hip_runtime.h"):
        pytest.skip("g++ or the HIP headers are not available")
    exe = str(tmp_path / "cache_stress")
    build = subprocess.run(
        ["g++", "-std=c++17", "-O1", "-g", "-fsanitize=thread", "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include",
         "-I" + os.path.join(ROOT, "include"), os.path.join(ROOT, "tests", "cache_stress.cpp"),
         os.path.join(ROOT, "tenant_fine_tune_amd", "csrc", "delta_cache.cpp"), "-L/opt/rocm/lib", "-lamdhip64",
         "-Wl,-rpath,/opt/rocm/lib", "-lpthread", "-o", exe],
        capture_output=True, text=True, timeout=300)
    assert build.returncode == 0, build.stderr[-2000:]
    for args in ([], ["join"]):
        run = subprocess.run([exe, *args], capture_output=True, text=True, timeout=300,
                             env={**os.environ, "TSAN_OPTIONS": "halt_on_error=1"})
        assert "ThreadSanitizer" not in run.stderr, run.stderr[-4000:]
        assert run.returncode == 0, run.stdout + run.stderr[-2000:]
        assert "bad 0" in run.stdout
