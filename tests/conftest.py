import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: runs HIP kernels on an MI355X (gfx950) device")


# The host-only build of the library (the C ABI layer and the planner compiled by a plain C++ compiler,
# with sanitizers, and linked against kernel-launch stubs: tests/test_host_build.py) stands in for the HIP
# library in the CPU tests of argument checking and planning when this variable names it.
_HOST_LIB = os.environ.get("AAH_TEST_HOST_LIB")
if _HOST_LIB:
    from head_causal_local_amd import _lib as _aah_lib
    _aah_lib.LIB_PATH = _HOST_LIB
