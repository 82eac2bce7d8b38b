import pytest


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: runs HIP kernels; needs an MI355X (gfx950) device")
