import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)
HERE = os.path.dirname(os.path.abspath(__file__))
if HERE not in sys.path:
    sys.path.insert(0, HERE)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: long-running CPU test")


@pytest.fixture(scope="session")
def gpu():
    """(torch, binding module) with the HIP library loaded; skips without a GPU."""
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from drafter_vocab_top_amd import topk_cols as T
    T.load()   # fails loudly if the library is missing
    return torch, T
