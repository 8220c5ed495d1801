import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)
HERE = os.path.dirname(os.path.abspath(__file__))
if HERE not in sys.path:
    sys.path.insert(0, HERE)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: long-running CPU test")


def _ensure_built():
    """Load what is built; build only when nothing is (CPU cross-compile)."""
    lib = os.path.join(ROOT, "importance_aware_kv_amd", "libhikv.so")
    if not os.path.exists(lib):
        from importance_aware_kv_amd import build as b
        b.build()
    ref = os.path.join(ROOT, "oracle", "libhikv_ref.so")
    if not os.path.exists(ref):
        from oracle import build as ob
        ob.build()


_ensure_built()
