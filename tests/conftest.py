import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU")
    config.addinivalue_line("markers", "slow: full-size workload (minutes of host work)")


def _ensure_built():
    """Build the native pieces only when nothing is built yet."""
    import __graft_entry__ as ge
    need = [os.path.join(ROOT, "oracle", "liboracle.so"),
            os.path.join(ROOT, "synthetic", "libsynth.so")]
    if not all(os.path.exists(p) for p in need):
        ge.build()


_ensure_built()
