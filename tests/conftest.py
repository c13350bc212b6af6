import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: long-running statistical or full-size check")


@pytest.fixture(scope="session")
def clm_gpu():
    """The GPU binding, loaded; skips nothing silently - a missing library or
    GPU is an error for tests marked gpu."""
    import torch
    if not torch.cuda.is_available():
        pytest.fail("test marked gpu but no GPU is visible")
    import codec_language_model_amd as clm
    clm.load()
    return clm
