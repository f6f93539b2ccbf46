import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: full-size workloads (minutes of CPU time)")


def _gpu_available():
    try:
        import torch
        return torch.cuda.is_available()
    except Exception:  # pragma: no cover
        return False


def pytest_collection_modifyitems(config, items):
    if _gpu_available():
        return
    skip = pytest.mark.skip(reason="no GPU visible")
    for item in items:
        if "gpu" in item.keywords:
            item.add_marker(skip)


@pytest.fixture
def lib_env():
    """Set the library's debug variables (MOSAIC_TUNE, MOSAIC_CHECK_IDX) for one test.

    The library reads them once per process, so each change is followed by
    mosaic_debug_reload_env(), and so is restoring them when the test ends."""
    from mask_only_logits_amd import mosaic
    saved = {}

    def set_env(name, value=None):
        saved.setdefault(name, os.environ.get(name))
        if value is None:
            os.environ.pop(name, None)
        else:
            os.environ[name] = value
        mosaic.mosaic_debug_reload_env()

    yield set_env
    for k, v in saved.items():
        if v is None:
            os.environ.pop(k, None)
        else:
            os.environ[k] = v
    mosaic.mosaic_debug_reload_env()
