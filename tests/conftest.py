import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


def ensure_library():
    """Load the built library; build it only if nothing is built yet."""
    lib = os.path.join(ROOT, "paged_kv_cache_amd", "libpkv.so")
    if not os.path.exists(lib):
        import importlib.util
        spec = importlib.util.spec_from_file_location(
            "pkv_build", os.path.join(ROOT, "paged_kv_cache_amd", "build.py"))
        mod = importlib.util.module_from_spec(spec)
        spec.loader.exec_module(mod)
        mod.build()
    import paged_kv_cache_amd  # noqa: F401  (raises ImportError if unusable)
    return lib


@pytest.fixture(scope="session")
def pkv():
    ensure_library()
    import paged_kv_cache_amd
    return paged_kv_cache_amd
