import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) and the built HIP library")


@pytest.fixture(scope="session")
def gpu_lib():
    """The HIP library bound for GPU tests; fails loudly when it is not built or no GPU is present."""
    import torch
    if not torch.cuda.is_available():
        pytest.fail("GPU test collected without a visible GPU")
    import stream_audio_video_amd as h3
    h3.load_library()
    return h3
