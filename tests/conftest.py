import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: long-running CPU test")
    from tests import live
    live._CONFIG = config


def pytest_sessionfinish(session, exitstatus):
    # the whole-tensor references' worker pool, if a test started it
    mod = sys.modules.get("tests.oracle_par")
    if mod is not None:
        mod.shutdown()
