import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)
TESTS = os.path.dirname(os.path.abspath(__file__))
if TESTS not in sys.path:
    sys.path.insert(0, TESTS)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: full-size workloads")


def pytest_collection_modifyitems(config, items):
    # run the GPU suite in a fixed order: layout probes, stages, parity, full size,
    # and the allocation-free entry point last
    order = {"test_gpu_layout": 0, "test_gpu_stages": 1, "test_gpu_parity": 2,
             "test_gpu_decay": 3, "test_gpu_anchors": 3,
             "test_gpu_batched": 3, "test_gpu_prep": 3, "test_gpu_fullsize": 4,
             "test_zz_no_alloc": 9}

    def key(item):
        mod = item.module.__name__.rsplit(".", 1)[-1]
        return order.get(mod, -1)
    items.sort(key=key)
