import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_addoption(parser):
    parser.addoption("--seed-offset", type=int, default=0,
                     help="add this to the seed of every synthetic workload (re-runs the parity tests on "
                          "other seeded inputs; both sides read the same generator)")


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: full-size parity case (minutes of CPU oracle work)")
    offset = config.getoption("--seed-offset")
    if offset:
        from synth import workloads

        init = workloads.Workload.__init__

        def shifted(self, *args, **kwargs):
            init(self, *args, **kwargs)
            self.seed = self.seed + offset

        workloads.Workload.__init__ = shifted


def _has_gpu():
    try:
        import torch
        return torch.cuda.is_available()
    except Exception:
        return False


def pytest_collection_modifyitems(config, items):
    if _has_gpu():
        return
    skip = pytest.mark.skip(reason="no GPU visible")
    for item in items:
        if "gpu" in item.keywords:
            item.add_marker(skip)
