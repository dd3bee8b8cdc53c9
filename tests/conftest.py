import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an AMD GPU (MI355X / gfx950) and the built HIP library")
    config.addinivalue_line("markers", "slow: long CPU test")
    config.addinivalue_line("markers", "gpu_fullsize: every element of a full-size workload against the oracle "
                                       "(minutes; run on request with -m gpu_fullsize, not part of -m gpu)")


@pytest.fixture(scope="session", autouse=True)
def _built_cpu_libs():
    """Build the oracle and generator once per session if they are not built yet."""
    import oracle
    import synth
    if not os.path.exists(os.path.join(ROOT, "oracle", "liboracle.so")):
        oracle.build()
    if not os.path.exists(os.path.join(ROOT, "synth", "libsynth.so")):
        synth.build()
    yield
