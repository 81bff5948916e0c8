import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: long-running (large workloads)")


def _ensure_cpu_libs():
    """The generator and the oracle are plain C; build them if nothing is built yet."""
    from local_sparse_attention_amd import _build
    import oracle

    if not os.path.exists(_build.SYNTH_LIB):
        _build.build_synth()
    if not os.path.exists(oracle._LIBPATH):
        oracle.build()


_ensure_cpu_libs()


@pytest.fixture(scope="session")
def dsa3d_gpu():
    """The HIP binding on cuda:0 (tests marked gpu only)."""
    import torch

    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from local_sparse_attention_amd import dsa3d

    dsa3d.load()  # raises if the library is missing: no CPU fallback exists
    return dsa3d
