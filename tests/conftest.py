import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: long-running (full-size model) test")


@pytest.fixture(scope="session")
def weights_7b():
    """Seeded Mistral-7B-shaped bf16 weights (seed 0), generated once per session."""
    import synth
    print("7B: generating weights", flush=True)
    return synth.make_weights(synth.MISTRAL7B)


@pytest.fixture(scope="session")
def device_weights_7b(weights_7b):
    import continuous_batching_decode_step_amd as cbd
    return cbd.upload_weights(weights_7b)
