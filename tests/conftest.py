import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: CPU test that takes more than a few seconds")


def pytest_sessionfinish(session, exitstatus):
    # the per-step parity metrics the GPU tests recorded (nothing on a CPU-only run)
    from tests import gpu_harness
    gpu_harness.write_report()
