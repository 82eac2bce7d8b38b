import pytest


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: runs HIP kernels; needs an MI355X (gfx950) device")


@pytest.fixture(scope="session")
def built_lib():
    """The engine library, built in-tree only if it is not there yet."""
    import co_activation_amd
    if not co_activation_amd.is_built():
        from co_activation_amd.build import build
        build()
    return co_activation_amd.lib()
