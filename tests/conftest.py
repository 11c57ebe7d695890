import os
import sys

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


def golden_lines(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return [ln.strip() for ln in f if ln.strip() and not ln.startswith("#")]


@pytest.fixture(scope="session")
def orc():
    import oracle
    oracle.lib()
    return oracle


@pytest.fixture(scope="session")
def bsq_gpu():
    """The HIP library through its Python binding, on cuda:0."""
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import block_scaled_precision_bsq_amd as bsq
    return bsq


def bf16(a):
    from workloads import f32_to_bf16_bits
    return f32_to_bf16_bits(np.asarray(a, np.float32))
