"""The library's host code under AddressSanitizer and UndefinedBehaviorSanitizer
(CPU, no GPU): api.cpp -- argument validation, workspace layout, overlap
checks, stage sequencing -- is compiled with g++ -fsanitize=address,undefined
and linked with launchers that report "no device" (tests/
sanitizer_host_stubs.cpp); the C-ABI tests (tests/test_abi_cpu.py) then run
against that build in a child process with the sanitizer runtime preloaded.
Any sanitizer report fails the child (halt_on_error) and this test."""

from __future__ import annotations

import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
OUT = os.path.join(ROOT, "_build", "sanitize")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")


def _gxx(*args):
    cmd = ["g++", "-std=c++17", "-O1", "-g", "-fPIC", "-fno-omit-frame-pointer", "-D__HIP_PLATFORM_AMD__",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined", f"-I{ROCM}/include",
           f"-I{ROOT}/include", f"-I{ROOT}/position_extrapolation_amd/csrc", *args]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, " ".join(cmd) + "\n" + r.stdout + r.stderr


def _runtime(name):
    path = subprocess.run(["g++", f"-print-file-name={name}"], capture_output=True, text=True).stdout.strip()
    return path if os.path.isabs(path) and os.path.exists(path) else None


@pytest.fixture(scope="module")
def asan_lib():
    if _runtime("libasan.so") is None:
        pytest.skip("g++ has no AddressSanitizer runtime here")
    os.makedirs(OUT, exist_ok=True)
    objs = []
    for src in (os.path.join(ROOT, "position_extrapolation_amd", "csrc", "api.cpp"),
                os.path.join(ROOT, "tests", "sanitizer_host_stubs.cpp")):
        obj = os.path.join(OUT, os.path.splitext(os.path.basename(src))[0] + ".o")
        _gxx("-c", src, "-o", obj)
        objs.append(obj)
    lib = os.path.join(OUT, "libdca_host_sanitized.so")
    _gxx("-shared", *objs, "-o", lib, f"-L{ROCM}/lib", "-lamdhip64", f"-Wl,-rpath,{ROCM}/lib")
    return lib


def test_abi_tests_under_address_and_undefined_sanitizers(asan_lib):
    env = dict(os.environ)
    env["DCA_LIBRARY"] = asan_lib
    pre = [_runtime("libasan.so"), _runtime("libubsan.so")]
    env["LD_PRELOAD"] = ":".join([p for p in pre if p] + ([env["LD_PRELOAD"]] if env.get("LD_PRELOAD") else []))
    # leaks: the Python interpreter and torch keep allocations alive at exit
    env["ASAN_OPTIONS"] = "detect_leaks=0:halt_on_error=1:verify_asan_link_order=0"
    env["UBSAN_OPTIONS"] = "halt_on_error=1:print_stacktrace=1"
    cmd = [sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider", "-m", "not gpu",
           os.path.join(ROOT, "tests", "test_abi_cpu.py"),
           os.path.join(ROOT, "tests", "test_host_sanitizers_child.py")]
    r = subprocess.run(cmd, capture_output=True, text=True, env=env, cwd=ROOT, timeout=600)
    out = r.stdout + r.stderr
    assert "AddressSanitizer" not in out and "runtime error:" not in out, out[-4000:]
    assert r.returncode == 0, out[-4000:]
    assert " passed" in out
