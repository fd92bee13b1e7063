"""Shared pytest setup: markers, import path and on-demand builds.

Tests marked ``gpu`` need an MI355X (gfx950) and the built HIP library; every
other test runs on the CPU.
"""
import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: full-size workloads (seconds to a minute each)")


@pytest.fixture(scope="session")
def oracle_mod():
    import oracle

    if not os.path.exists(oracle.LIB_PATH):
        oracle.build()
    return oracle


@pytest.fixture(scope="session")
def gpu_lib():
    """The HIP library, loaded through the product binding; skips nothing.

    A GPU test that cannot load the library fails loudly: there is no CPU
    fallback for the product path.
    """
    import torch

    if not torch.cuda.is_available():
        pytest.fail("gpu test collected on a machine without a GPU")
    from gqa_kv_cache_decode_amd import _lib

    return _lib.load()
