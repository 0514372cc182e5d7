import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU; parity tests against the oracle")
    config.addinivalue_line("markers", "slow: CPU test that takes more than a few seconds")


def gpu_available() -> bool:
    try:
        import torch

        return torch.cuda.is_available()
    except Exception:
        return False


def pytest_sessionstart(session):
    # A fresh checkout has no libgqa.so (it is built, not committed).  Without a GPU, build
    # it here (hipcc cross-compiles gfx950) so that the ABI tests run.  With a GPU it must
    # already be built, and a missing library fails the tests that load it.
    lib = os.path.join(ROOT, "transformer_attention_07_amd", "libgqa.so")
    if not os.path.exists(lib) and not gpu_available():
        from transformer_attention_07_amd.build import build_library

        build_library()


def pytest_collection_modifyitems(config, items):
    if gpu_available():
        return
    skip = pytest.mark.skip(reason="no GPU in this environment")
    for item in items:
        if "gpu" in item.keywords:
            item.add_marker(skip)
