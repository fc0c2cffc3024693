import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line(
        "markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    # MNB_HOST_LIB names a host-only build of the library (the sanitizer
    # test builds the front end with stand-ins for the HIP side); the ABI
    # tests then load it in place of libmnb.so.
    host_lib = os.environ.get("MNB_HOST_LIB")
    if host_lib:
        import block_wise_int4_matmulnbits_amd as mnb
        mnb.LIB_PATH = host_lib


@pytest.fixture(scope="session")
def oracle_mod():
    # MNB_ORACLE_ROOT names a directory holding another copy of the oracle
    # package (the mutation test plants one mistake in such a copy and runs
    # the pins against it).
    alt = os.environ.get("MNB_ORACLE_ROOT")
    if alt:
        sys.path.insert(0, alt)
    import oracle
    if alt:
        assert os.path.dirname(os.path.dirname(os.path.abspath(oracle.__file__))) == \
            os.path.abspath(alt), oracle.__file__
    oracle.build(force=False)
    return oracle
