"""The C ABI's argument validation and host-side size arithmetic under
AddressSanitizer and UndefinedBehaviorSanitizer.

The library's sources are built with both sanitizers on their host code and
linked into a plain C program (tests/host_sanitize/abi_driver.c) that calls
every entry point of qlora.h with arguments its validation must reject
before any device work, and runs the size queries over the benchmark
workloads' layers and at the edge of the 2^31 index range. Any sanitizer
report aborts the program; every status must match. It runs without a GPU
(no device is made visible to it) and never launches a kernel.
"""

import os
import subprocess

import pytest

from quantized_frozen_weight_amd import build_lib

HERE = os.path.dirname(os.path.abspath(__file__))
DRIVER = os.path.join(HERE, "host_sanitize", "abi_driver.c")


@pytest.mark.timeout(600)
def test_abi_validation_under_host_sanitizers(tmp_path):
    exe = build_lib.build_host_sanitized(DRIVER, str(tmp_path / "abi_driver"))
    env = dict(os.environ)
    # no device for the driver, whatever the machine has
    env["HIP_VISIBLE_DEVICES"] = ""
    env["ROCR_VISIBLE_DEVICES"] = ""
    env["ASAN_OPTIONS"] = "detect_leaks=0:abort_on_error=1"
    env["UBSAN_OPTIONS"] = "print_stacktrace=1:halt_on_error=1"
    proc = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=120)
    out = proc.stdout + proc.stderr
    assert proc.returncode == 0, out[-4000:]
    assert " 0 failures" in out, out[-4000:]
    assert "ERROR: AddressSanitizer" not in out and "runtime error:" not in out, out[-4000:]
