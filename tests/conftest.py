import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: long-running test")


@pytest.fixture(scope="session", autouse=True)
def _host_libs():
    """Make sure the host-side helper libraries (generator, oracle) exist.
    With GDN_HOST_ASAN_DIR set (tests/host_asan.sh), load the sanitizer builds
    of the oracle, the generator and libgdn from that directory instead."""
    import oracle
    import synth

    asan = os.environ.get("GDN_HOST_ASAN_DIR")
    if asan:
        import gated_delta_rule_scan_amd as gdn

        synth._SO = os.path.join(asan, "libsynth.so")
        oracle._SO = os.path.join(asan, "liboracle.so")
        gdn.LIB_PATH = os.path.join(asan, "libgdn.so")
        gdn._lib = None
    synth._load()
    oracle._load()
