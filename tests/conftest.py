import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def _ensure_built():
    """Build the HIP library (cross-compiled for gfx950) and the oracle when
    missing, so a fresh checkout can run the CPU suite directly."""
    lib = os.path.join(ROOT, "int8_weight_quantized_amd", "libqw.so")
    if not os.path.exists(lib) and os.path.exists("/opt/rocm/bin/hipcc"):
        from int8_weight_quantized_amd import build as qwbuild
        qwbuild.build()


def pytest_configure(config):
    _ensure_built()
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: takes more than a few seconds on the CPU")


@pytest.fixture(scope="session")
def orc():
    import oracle
    return oracle.default()
