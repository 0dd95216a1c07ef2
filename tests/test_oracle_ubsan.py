"""CPU tier: the oracle built with UndefinedBehaviorSanitizer passes every pin.

A copy of oracle/bitdelta_oracle.c is compiled with gcc -fsanitize=undefined
-fno-sanitize-recover (so any undefined behaviour aborts the process) and the
pins of tests/pins.py run against it in a child process."""
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_oracle_pins_under_ubsan(tmp_path):
    if shutil.which("gcc") is None:
        pytest.skip("gcc is not available")
    lib = str(tmp_path / "liboracle_ubsan.so")
    build = subprocess.run(["gcc", "-O1", "-g", "-fopenmp", "-ffp-contract=off", "-std=c11", "-shared", "-fPIC",
                            "-fsanitize=undefined", "-fno-sanitize-recover=all",
                            os.path.join(ROOT, "oracle", "bitdelta_oracle.c"), "-o", lib, "-lm"],
                           capture_output=True, text=True, timeout=300)
    assert build.returncode == 0, build.stderr[-2000:]
    code = ("import oracle\nfrom tests import pins\no = oracle.Oracle(%r)\n"
            "for p in pins.ALL:\n    p(o)\nprint('pins', len(pins.ALL))\n" % lib)
    run = subprocess.run([sys.executable, "-c", code], cwd=ROOT, capture_output=True, text=True, timeout=600,
                         env={**os.environ, "PYTHONPATH": ROOT})
    assert run.returncode == 0 and "runtime error" not in run.stderr, run.stderr[-4000:]
    assert run.stdout.strip().startswith("pins")
