import os
import sys

import numpy as np
import pytest
import torch

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built libpa.so")
    config.addinivalue_line("markers", "slow: full-size workloads")


def raw(t: torch.Tensor) -> np.ndarray:
    """Raw storage of a CPU tensor in the oracle's conventions (bf16 -> uint16 bits, fp8 -> uint8 codes)."""
    t = t.detach().cpu().contiguous()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    if t.dtype == torch.float8_e4m3fn:
        return t.view(torch.uint8).numpy()
    return t.numpy()


@pytest.fixture
def to_raw():
    return raw
