import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: long-running (large sizes)")


@pytest.fixture(scope="session")
def gpu_lib():
    """The HIP library through its Python binding; fails loudly when it is
    missing or there is no GPU, so a GPU test can never pass on a fallback."""
    import torch
    if not torch.cuda.is_available():
        pytest.fail("GPU test collected but no GPU is visible")
    import exact_lloyd_means_flashassign_amd as fk
    fk.load()  # raises if libfk.so is missing
    return fk


@pytest.fixture(autouse=True, scope="module")
def _release_cached_memory():
    """After each test module, hand back what the caches hold: the binding's
    per-device workspace, torch's cached device blocks and its cached pinned
    host blocks (a module that streams a 50 GB pinned array would otherwise
    keep it pinned for the rest of the session)."""
    yield
    import gc
    import sys as _sys
    torch = _sys.modules.get("torch")
    if torch is None or not torch.cuda.is_initialized():
        return
    fk = _sys.modules.get("exact_lloyd_means_flashassign_amd")
    gc.collect()
    torch.cuda.synchronize()
    if fk is not None:
        fk._ws_cache.clear()
    torch.cuda.empty_cache()
    torch._C._host_emptyCache()
