"""pytest configuration: the `gpu` marker and import paths.

Tests marked `gpu` need an MI355X (gfx950) and the built HIP library; everything else
runs on a CPU-only host (`pytest -m "not gpu"`).
"""
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
TESTS = os.path.dirname(os.path.abspath(__file__))
for p in (ROOT, TESTS):
    if p not in sys.path:
        sys.path.insert(0, p)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an AMD Instinct GPU (gfx950) and the HIP library")
