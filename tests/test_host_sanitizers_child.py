"""Run by tests/test_host_sanitizers.py in its sanitized child process only:
the library the binding loaded there is the sanitizer build, and the
sanitizer runtime is live."""

from __future__ import annotations

import ctypes
import os

import pytest

from position_extrapolation_amd import api

pytestmark = pytest.mark.skipif("DCA_LIBRARY" not in os.environ, reason="only in the sanitized child process")


def test_the_sanitized_library_is_the_one_loaded():
    assert api.LIB_PATH == os.environ["DCA_LIBRARY"]
    api.lib()
    maps = open("/proc/self/maps").read()
    assert os.path.basename(os.environ["DCA_LIBRARY"]) in maps
    # the AddressSanitizer runtime is mapped and answers
    asan = ctypes.CDLL(None)
    assert hasattr(asan, "__asan_init")
