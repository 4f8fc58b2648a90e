import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: takes more than a few seconds on the CPU")


def _ensure_built():
    """Build the C libraries only when nothing is built yet (build() always rebuilds)."""
    from oracle import build as ob
    from synth import build as sb
    if not os.path.exists(ob.LIB) and "MOE_ORACLE_LIB" not in os.environ:
        ob.build()
    if not os.path.exists(sb.LIB):
        sb.build()


_ensure_built()


@pytest.fixture(scope="session")
def gpu_available():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    return True
