import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: full-size workload, minutes of CPU or GPU time")


def pytest_sessionstart(session):
    # tests load the built library; build it once if it is not there yet
    lib = os.path.join(ROOT, "expert_routing_grouped_route_amd", "libmoe.so")
    if not os.path.exists(lib):
        from expert_routing_grouped_route_amd.build import build_library
        build_library()
