import os
import sys

import pytest

try:  # import torch at collection time (slow on a cold box), not inside a timed test
    import torch  # noqa: F401
except Exception:  # pragma: no cover
    pass

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


@pytest.fixture(scope="session")
def gpu_lib():
    """The loaded C-ABI library on a GPU; the tests marked gpu fail loudly
    when either the device or the built library is missing."""
    import torch
    assert torch.cuda.is_available(), "GPU test run without a visible GPU"
    from gguf_quant_block_amd import binding
    return binding.lib()
