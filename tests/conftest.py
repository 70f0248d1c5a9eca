import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_addoption(parser):
    parser.addoption("--kda-library", default=None,
                     help="path of another build of libkda.so to test (e.g. the host AddressSanitizer build)")
    parser.addoption("--oracle-library", default=None,
                     help="path of another build of the oracle's shared library")


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: long-running CPU test")
    lib = config.getoption("--kda-library")
    if lib:
        from chunked_gated_delta_13_amd import _lib
        _lib.LIB_PATH = os.path.abspath(lib)
    ora = config.getoption("--oracle-library")
    if ora:
        import oracle
        oracle._LIB_PATH = os.path.abspath(ora)
