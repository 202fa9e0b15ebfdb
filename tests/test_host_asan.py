"""The library's host code (csrc/onela_host.cpp) built with g++ under AddressSanitizer and UndefinedBehavior-
Sanitizer, without a GPU: tests/host_asan/ holds a host stand-in for the HIP runtime calls and the kernel
launchers (each touches exactly the buffer extents its kernel reads and writes, and records what it wrote per
kind of buffer) and a driver that walks the C ABI's state machine: errors before a context, steps to capacity,
reset, a bad parent and its sticky flag, a failed launch, prefill, device mismatch, beam-selection argument
checks and the allocation-free selection's size limit, for every dispatch path.  The run fails on any
sanitizer report, failed check, or workspace regions written over each other."""

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HERE = os.path.join(ROOT, "tests", "host_asan")


@pytest.mark.skipif(shutil.which("g++") is None, reason="g++ not available")
def test_host_state_machine_under_sanitizers(tmp_path):
    exe = str(tmp_path / "driver")
    cmd = ["g++", "-std=c++17", "-g", "-O1", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
           "-fno-sanitize-recover=all", "-I", HERE, "-I", os.path.join(ROOT, "include"),
           "-I", os.path.join(ROOT, "linear_attention_beam_amd", "csrc"),
           os.path.join(ROOT, "linear_attention_beam_amd", "csrc", "onela_host.cpp"),
           os.path.join(HERE, "stub_device.cpp"), os.path.join(HERE, "driver.cpp"), "-o", exe]
    build = subprocess.run(cmd, capture_output=True, text=True, timeout=300)
    assert build.returncode == 0, build.stdout + build.stderr
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0", UBSAN_OPTIONS="print_stacktrace=1")
    run = subprocess.run([exe], capture_output=True, text=True, timeout=300, env=env)
    assert run.returncode == 0, run.stdout + run.stderr
    assert "all checks passed" in run.stdout
