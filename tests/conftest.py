import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


@pytest.fixture(scope="session")
def orc():
    import oracle
    oracle.build()
    oracle.lib()
    return oracle


@pytest.fixture(scope="session")
def dsv4():
    """The HIP library's binding (built in-tree first if it is missing)."""
    lib = os.path.join(ROOT, "sparse_mla_attention_combine_amd", "_lib", "libdsv4.so")
    if not os.path.exists(lib):
        from sparse_mla_attention_combine_amd import build as _b
        _b.build()
    import sparse_mla_attention_combine_amd as m
    return m
