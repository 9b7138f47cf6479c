"""pytest configuration: the `gpu` marker and import paths.

Tests marked `gpu` need an MI355X (gfx950) and the built GPU library; everything
else runs on a CPU-only host. Run the CPU suite with `pytest -m "not gpu"`.
"""
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)
TESTS = os.path.dirname(os.path.abspath(__file__))
if TESTS not in sys.path:
    sys.path.insert(0, TESTS)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X GPU and the built HIP library")
