import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: long CPU case (still part of the default CPU tier)")
    # Host-side checkers are cheap to build; build them only when nothing is built yet.
    need = [p for p in ("oracle/liboracle.so", "synth/libsynth.so") if not os.path.exists(os.path.join(ROOT, p))]
    if need:
        subprocess.run([sys.executable, "-c", "import __graft_entry__ as g; g._build_host_libs()"],
                       cwd=ROOT, check=True)


@pytest.fixture(scope="session")
def orc():
    import oracle

    return oracle.default()
