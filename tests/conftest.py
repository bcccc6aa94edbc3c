import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs a gfx950 GPU (runs the HIP library)")
    config.addinivalue_line("markers", "slow: large full-size parity cases")


def gpu_available() -> bool:
    try:
        import torch
        return torch.cuda.is_available()
    except Exception:
        return False


@pytest.fixture(scope="session")
def oracle_lib():
    import oracle
    oracle.build(force=not os.path.exists(oracle._LIB_PATH))
    return oracle


@pytest.fixture(scope="session")
def synth_lib():
    import synth
    synth.build(force=not os.path.exists(synth._LIB_PATH))
    return synth


@pytest.fixture
def tune():
    """tune(**knobs): tuning overrides of the library (lsa_set_tuning) for the
    calling thread, undone when the test ends."""
    import lookahead_chunk_sparse_amd as lsa
    held = []

    def set_knobs(**knobs):
        cm = lsa.tuning(**knobs)
        cm.__enter__()
        held.append(cm)

    yield set_knobs
    for cm in reversed(held):
        cm.__exit__(None, None, None)
