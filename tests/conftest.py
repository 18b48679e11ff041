import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: full-size configuration test")


def _ensure_library():
    """Build libpagedattn.so when it is missing (tests load what is built)."""
    from attention_paged_kv_varlen_amd import build as _build
    if not os.path.exists(_build.LIB):
        _build.build()


def pytest_sessionstart(session):
    _ensure_library()
