import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an AMD GPU (MI355X, gfx950) and the built HIP library")
    config.addinivalue_line("markers", "slow: full-size cases (still run by default)")


def _gpu_available() -> bool:
    try:
        import torch
        return bool(torch.cuda.is_available())
    except Exception:
        return False


def pytest_collection_modifyitems(config, items):
    if _gpu_available():
        return
    skip = pytest.mark.skip(reason="no GPU visible to torch")
    for item in items:
        if "gpu" in item.keywords:
            item.add_marker(skip)


@pytest.fixture
def qmm_override():
    """Set launch-plan overrides in the loaded library for one test (they are
    removed afterwards): ``qmm_override("QMM_GEMM_TILE_M", 64)``."""
    import gemm_qmm_gemv_amd as qmm
    names = []

    def set_override(name, value):
        qmm.qmm_set_override(name, int(value))
        names.append(name)

    yield set_override
    for name in names:
        qmm.qmm_set_override(name, -1)
