import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)
HERE = os.path.dirname(os.path.abspath(__file__))
if HERE not in sys.path:
    sys.path.insert(0, HERE)


def _ensure_built():
    """Build the oracle and the GPU library once if they are missing (a fresh
    checkout); an existing build is used as it is."""
    import oracle
    if not os.path.exists(os.path.join(ROOT, "oracle", "liboracle.so")):
        oracle.build(force=False)
    if not os.path.exists(os.path.join(ROOT, "block_scaled_precision_05_amd", "libbsg.so")):
        from block_scaled_precision_05_amd import build
        build.build(force=False)


_ensure_built()


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU")
    config.addinivalue_line("markers", "slow: long-running CPU test")


@pytest.fixture(scope="session")
def orc():
    import oracle
    oracle._load()
    return oracle
