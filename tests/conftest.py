import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU")


import pytest  # noqa: E402


@pytest.fixture(scope="session")
def ra_lib():
    """libra.so loaded through the binding; built in-tree first if it is missing."""
    from blockwise_ring_attention_amd import _binding
    if not os.path.exists(_binding.LIB_PATH):
        from blockwise_ring_attention_amd.csrc import build
        build.build()
    return _binding.load()
