import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line(
        "markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


import pytest  # noqa: E402


@pytest.fixture(autouse=True)
def _library_options_follow_environment():
    """After each test (and after monkeypatch has restored the environment,
    since autouse fixtures are torn down last) the library re-reads its
    PAGEDATTN_* overrides, so no test inherits another's."""
    yield
    import paged_kv_cache_reshape_amd as pa
    if pa._lib is not None:
        pa.reload_options()
