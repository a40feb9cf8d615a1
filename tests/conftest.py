import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)
HERE = os.path.dirname(os.path.abspath(__file__))
if HERE not in sys.path:
    sys.path.insert(0, HERE)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (runs through the C-ABI library)")


def pytest_sessionstart(session):
    # Build the seeded-input fillers if this checkout has none yet (gcc + hipcc, seconds).
    from switchffn_synth import _native
    if not (os.path.exists(_native.HOST_LIB) and os.path.exists(_native.DEV_LIB)):
        from switchffn_synth.build import build
        build()
