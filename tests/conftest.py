import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line(
        "markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


@pytest.fixture(scope="session", autouse=True)
def _gpu_library_is_current(request):
    """Once per session that runs GPU tests: the HIP library about to be
    used was built from the sources in this tree (load() rebuilds or raises
    otherwise), so a green GPU run speaks for these sources."""
    if not any(item.get_closest_marker("gpu") for item in request.session.items):
        return
    from exact_io_aware_05_amd import _lib, build
    lib = _lib.load()
    got = lib.fa_source_hash().decode()
    assert got == build.source_hash(), "libfa.so does not match csrc/"
    print(f"\nlibfa.so source hash {got[:16]} matches the sources", flush=True)
