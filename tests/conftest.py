import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: full-size workloads (minutes of CPU oracle time)")


@pytest.fixture(scope="session")
def gpu_lib():
    """The HIP library through its binding; skips when no GPU is visible."""
    import torch

    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    from paged_kv_decode_02_amd import pa

    pa.load()  # raises if the built library is missing
    return pa


def pytest_collection_finish(session):
    """Start the oracle's worker processes (spawned interpreters that never
    touch a GPU) before any test initialises the GPU, when GPU tests will
    run on a machine that has one.  (Counting devices does not initialise
    the runtime.)"""
    if not any(item.get_closest_marker("gpu") for item in session.items):
        return
    import torch

    if torch.cuda.device_count() > 0:
        from oracle import parallel

        n = parallel.start_pool()
        print(f"[conftest] oracle worker processes: {n}", file=sys.stderr, flush=True)


def pytest_unconfigure(config):
    from oracle import parallel

    parallel.stop_pool()
