import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU")
    config.addinivalue_line("markers", "slow: long-running check")


def _ensure_built():
    """Build the host-side libraries when nothing is built yet (the GPU
    libraries are built by __graft_entry__.build() and never here)."""
    import oracle
    import sdm_inputs

    if not os.path.exists(oracle.LIB):
        oracle.build()
    if not os.path.exists(sdm_inputs.HOST_LIB):
        sdm_inputs.build()


_ensure_built()


def gpu_available() -> bool:
    try:
        import torch

        return torch.cuda.is_available()
    except Exception:  # pragma: no cover
        return False


def pytest_collection_modifyitems(config, items):
    if gpu_available():
        return
    skip = pytest.mark.skip(reason="no GPU in this environment")
    for it in items:
        if "gpu" in it.keywords:
            it.add_marker(skip)
