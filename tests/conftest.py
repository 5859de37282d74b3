"""Shared test helpers: markers and plain tensor -> numpy plumbing for the oracle."""

import os
import sys

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


def to_oracle_pool(pt):
    """PagedTensors -> oracle.OraclePool holding exactly the stored bytes (no arithmetic)."""
    import torch
    from oracle import OraclePool

    data = pt.data.detach().cpu()
    if pt.dtype == "bf16":
        data = data.view(torch.int16).numpy().view(np.uint16)
    else:
        data = data.numpy()
    scale = None if pt.scale is None else pt.scale.detach().cpu().numpy()
    return OraclePool(data=data, dtype=pt.dtype, dim=pt.dim, ratio=pt.ratio,
                      block_table=pt.block_table.detach().cpu().numpy(), scale=scale)


def to_f64(t):
    """Stored tensor (f32 / bf16) -> float64 numpy (exact widening)."""
    import torch
    return t.detach().cpu().to(torch.float64).numpy()


@pytest.fixture(scope="session")
def gpu_lib():
    """The built HIP library on a GPU; skips if no GPU is visible."""
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    import sparse_attention_hyb_amd as hyb
    hyb.load()
    return hyb
