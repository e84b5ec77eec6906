import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: full-size cases (minutes of host work)")


def pytest_collection_modifyitems(config, items):
    """Tests marked slow (minutes of host work on all cores) run only when
    MOE_RUN_SLOW=1 is set; otherwise they are reported as skipped."""
    if os.environ.get("MOE_RUN_SLOW") == "1":
        return
    skip = pytest.mark.skip(reason="slow: set MOE_RUN_SLOW=1 to run")
    for item in items:
        if "slow" in item.keywords:
            item.add_marker(skip)
