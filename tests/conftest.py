import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (runs the HIP path through the C ABI)")
    config.addinivalue_line("markers", "slow: long CPU work (full-size oracle runs)")


def pytest_collection_modifyitems(session, config, items):
    """Full-size parity runs after every other test (a -x stop there hides nothing
    else); the allocation-free entry point's module, named to sort last, stays last."""
    def key(item):
        mod = item.module.__name__.rsplit(".", 1)[-1]
        return (mod.startswith("test_zz_"), mod == "test_gpu_fullsize")
    items.sort(key=key)
