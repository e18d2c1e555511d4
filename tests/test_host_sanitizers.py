"""libserq's host code under the compiler's sanitizers (CPU only).

calibrate.cpp (calibration, GPTQ, MXFP4, the permutation helper, the bf6
prepack; host threads) and serq_abi.cpp (every argument validator) are
built with g++ together with tests/host/sanitizer_driver.cpp, whose stubs
stand in for the device launchers. That program runs the offline calls on
random layers with every output buffer exactly its documented size, and the
online validators with valid and invalid arguments. AddressSanitizer +
UndefinedBehaviorSanitizer (aborting on the first report), then
ThreadSanitizer for the calibration threads and the GPTQ barrier.
"""

from __future__ import annotations

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "w4a4_linear_layers_amd", "csrc")
SOURCES = [os.path.join(ROOT, "tests", "host", "sanitizer_driver.cpp"), os.path.join(CSRC, "calibrate.cpp"),
           os.path.join(CSRC, "serq_abi.cpp")]
ROCM_INCLUDE = "/opt/rocm/include"


def _build_and_run(tmp_path, flags):
    if shutil.which("g++") is None or not os.path.isdir(ROCM_INCLUDE):
        pytest.skip("g++ and the ROCm headers are needed")
    exe = str(tmp_path / "driver")
    cmd = (["g++", "-std=c++17", "-g", "-O1", "-fno-omit-frame-pointer"] + flags
           + ["-D__HIP_PLATFORM_AMD__", "-I", ROCM_INCLUDE, "-I", os.path.join(ROOT, "include"), "-I", CSRC]
           + SOURCES + ["-o", exe, "-lpthread"])
    b = subprocess.run(cmd, capture_output=True, text=True, timeout=300)
    assert b.returncode == 0, b.stderr[-3000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=1:verify_asan_link_order=0", UBSAN_OPTIONS="print_stacktrace=1",
               TSAN_OPTIONS="halt_on_error=1")
    r = subprocess.run([exe], capture_output=True, text=True, timeout=300, env=env)
    assert r.returncode == 0, (r.stdout[-2000:], r.stderr[-4000:])
    assert "all checks passed" in r.stdout


def test_host_code_under_address_and_ub_sanitizers(tmp_path):
    _build_and_run(tmp_path, ["-fsanitize=address,undefined", "-fno-sanitize-recover=all"])


def test_host_code_under_thread_sanitizer(tmp_path):
    _build_and_run(tmp_path, ["-fsanitize=thread"])
