import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)
TESTS = os.path.dirname(os.path.abspath(__file__))
if TESTS not in sys.path:
    sys.path.insert(0, TESTS)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the HIP library")
    config.addinivalue_line("markers", "slow: full-size case that takes tens of seconds")
    # Build the host-side libraries only when nothing is built yet.
    for sub, lib in (("oracle", "libmoe_ref.so"), ("synth", "libsynth_host.so")):
        if not os.path.exists(os.path.join(ROOT, sub, lib)):
            import importlib
            importlib.import_module(f"{sub}.build").build()
