import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) and the built HIP library")
    # Host-only libraries are cheap to build; build them if a fresh checkout lacks them.
    need = [os.path.join(ROOT, "synth", "libsynth.so"), os.path.join(ROOT, "oracle", "liboracle.so")]
    if not all(os.path.exists(p) for p in need):
        import synth.build
        import oracle.build
        synth.build.build()
        oracle.build.build()


@pytest.fixture(scope="session")
def orc():
    import oracle
    return oracle.default()
