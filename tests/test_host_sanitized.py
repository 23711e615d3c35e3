"""The library's host-side argument checks, prefill workspace layout, decode
plan and per-block selection, built for the host with AddressSanitizer and
UndefinedBehaviorSanitizer and swept over valid and hostile arguments (CPU
only).

``tests/native/abi_check_driver.cpp`` includes the very headers the library
compiles (``spa_check.h``, ``spa_plan.h``, ``spa_select.h``): every call must
return a defined status, every accepted call must describe shapes the kernels
assume and a workspace whose regions hold their data, and the selection
network and the 2:4 tournament must agree with the rank rule.  Any sanitizer
report (an overflow, an out-of-bounds access, a leak) fails the test.
"""
import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)


@pytest.fixture(scope="module")
def driver(tmp_path_factory):
    cxx = shutil.which("g++")
    if cxx is None:
        pytest.skip("no host C++ compiler")
    exe = str(tmp_path_factory.mktemp("asan") / "abi_check_driver")
    cmd = [cxx, "-std=c++17", "-O1", "-g", "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined",
           "-fno-omit-frame-pointer", "-Wall", "-Wno-unknown-pragmas", "-I", os.path.join(ROOT, "include"),
           "-I", os.path.join(ROOT, "activation_sparsification_amd", "csrc"),
           os.path.join(HERE, "native", "abi_check_driver.cpp"), "-o", exe]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0 and "sanitizer" in r.stderr.lower():
        pytest.skip("no sanitizer runtime for the host compiler")
    assert r.returncode == 0, r.stderr
    return exe


def test_host_checks_under_sanitizers(driver):
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    r = subprocess.run([driver], capture_output=True, text=True, env=env, timeout=300)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "runtime error" not in r.stderr and "AddressSanitizer" not in r.stderr, r.stderr
    words = r.stdout.split()
    assert words[0] == "ok", r.stdout
    # the sweep reaches accepted calls of both kinds, not only rejections
    decode, prefill = int(words[4]), int(words[7])
    assert decode > 10000 and prefill > 10000, r.stdout
