import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


# Set by tests/test_host_sanitizers.py for the child pytest it runs: the host-only
# ASan / UBSan build of the library to bind in place of libkda.so.
SANITIZED_LIB_ENV = "KDA_TEST_SANITIZED_LIB"


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU")
    path = os.environ.get(SANITIZED_LIB_ENV)
    if path:
        from gated_delta_rule_68_amd import _lib
        _lib._lib = _lib.bind(path)


def pytest_collection_modifyitems(config, items):
    # GPU tests last within the collected order is not required; nothing to reorder.
    return
