import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU; runs the HIP path")


@pytest.fixture(scope="session")
def oracle_mod():
    import oracle
    oracle._load()
    return oracle


def pytest_sessionstart(session):
    # the libraries are git-ignored build products: build them here if a
    # fresh checkout has none (this compiles; it never runs GPU code)
    lib = os.path.join(ROOT, "gemm_collective_tile_amd", "libiris_local.so")
    if not os.path.exists(lib):
        import importlib.util
        spec = importlib.util.spec_from_file_location(
            "_iris_build", os.path.join(ROOT, "gemm_collective_tile_amd", "build.py"))
        mod = importlib.util.module_from_spec(spec)
        spec.loader.exec_module(mod)
        mod.build()
    import oracle.build as ob
    if not os.path.exists(ob.LIB):
        ob.build()
