"""The host-only sources of the library (no HIP calls) built with g++ under AddressSanitizer and
UBSan, and again under ThreadSanitizer, and driven through every host entry point (and the thread
team the offloaded step keeps for its chunks) by tests/sanitize/host_driver.cpp."""

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "zero_partition_plan_amd", "csrc")


@pytest.mark.skipif(shutil.which("g++") is None, reason="needs g++")
def test_host_entry_points_under_asan_and_ubsan(tmp_path):
    exe = tmp_path / "host_driver"
    cmd = ["g++", "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer", "-ffp-contract=off",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined", "-pthread",
           "-I", os.path.join(ROOT, "include"), "-I", CSRC,
           os.path.join(ROOT, "tests", "sanitize", "host_driver.cpp"),
           os.path.join(CSRC, "zero_host.cpp"), os.path.join(CSRC, "zero_host_adam.cpp"),
           "-o", str(exe)]
    build = subprocess.run(cmd, capture_output=True, text=True)
    assert build.returncode == 0, build.stderr[-3000:]
    env = {**os.environ, "ASAN_OPTIONS": "detect_leaks=1:abort_on_error=0",
           "UBSAN_OPTIONS": "print_stacktrace=1"}
    run = subprocess.run([str(exe)], capture_output=True, text=True, env=env, timeout=300)
    assert run.returncode == 0, (run.stdout + run.stderr)[-4000:]
    assert "host driver ok" in run.stdout
    assert "AddressSanitizer" not in run.stderr and "runtime error" not in run.stderr


@pytest.mark.skipif(shutil.which("g++") is None, reason="needs g++")
def test_host_threads_under_tsan(tmp_path):
    """The host update's per-call threads and the offloaded step's thread team (its job hand-off
    under a mutex and condition variables) with ThreadSanitizer: no data race reported."""
    exe = tmp_path / "host_driver_tsan"
    cmd = ["g++", "-std=c++17", "-O1", "-g", "-ffp-contract=off", "-fsanitize=thread", "-pthread",
           "-I", os.path.join(ROOT, "include"), "-I", CSRC,
           os.path.join(ROOT, "tests", "sanitize", "host_driver.cpp"),
           os.path.join(CSRC, "zero_host.cpp"), os.path.join(CSRC, "zero_host_adam.cpp"),
           "-o", str(exe)]
    build = subprocess.run(cmd, capture_output=True, text=True)
    assert build.returncode == 0, build.stderr[-3000:]
    env = {**os.environ, "TSAN_OPTIONS": "halt_on_error=1:second_deadlock_stack=1"}
    run = subprocess.run([str(exe)], capture_output=True, text=True, env=env, timeout=600)
    assert run.returncode == 0, (run.stdout + run.stderr)[-4000:]
    assert "host driver ok" in run.stdout
    assert "ThreadSanitizer" not in run.stderr
