import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU")
    # Use what is built; build only what is missing.
    from bit_quantized_all_amd import build as hip_build
    if not os.path.exists(hip_build.LIB):
        hip_build.build()
    if not all(os.path.exists(f) for f in (hip_build.TEST_HELPER_LIB, hip_build.SMALL_GRID_LIB,
                                           hip_build.ABI_CHECK_BIN)):
        hip_build.build_test_helpers()


@pytest.fixture(scope="session")
def oracle():
    import oracle as _oracle
    return _oracle.default()
