import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

# Every input, however small, takes the library's early-exit rounds unless it
# asks for log Z (which reads every row): the GPU tests then run both ways on
# every case (tests/gpu_helpers.run_gpu) instead of rounds on large inputs only.
os.environ.setdefault("SPECV_ROUNDS_MIN_BYTES", "0")


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) and the built HIP library")
    config.addinivalue_line("markers", "slow: long-running CPU test")


@pytest.fixture(scope="session")
def gpu_lib():
    """The HIP path, loaded; skips only when no GPU is visible at all."""
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    import speculative_sampling_verify_spec_amd as sv
    sv.load()          # raises if the built library is missing: never a silent fallback
    return sv
