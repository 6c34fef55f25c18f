import os
import sys

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


def f64(t):
    """Exact upcast of a torch tensor (any float dtype, any device) to float64 numpy."""
    import torch
    if isinstance(t, np.ndarray):
        return t.astype(np.float64)
    return t.detach().to("cpu", torch.float64).numpy()


def i64(t):
    if isinstance(t, np.ndarray):
        return t.astype(np.int64)
    return t.detach().cpu().numpy().astype(np.int64)


@pytest.fixture(scope="session")
def golden_dir():
    return os.path.join(ROOT, "tests", "golden")
