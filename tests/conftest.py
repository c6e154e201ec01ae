import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)
# the mutation check runs the oracle pins against a planted-mistake copy of the
# oracle placed in this directory
_override = os.environ.get("SPA_ORACLE_UNDER_TEST")
if _override:
    sys.path.insert(0, _override)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: full-size workload, minutes of CPU work")
