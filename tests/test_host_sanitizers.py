"""The C ABI's host code under AddressSanitizer and UndefinedBehaviorSanitizer
(CPU only).

Builds every library source together with tests/host_sanitizer_driver.cpp,
with the sanitizers on the host side only (the device code is compiled as
usual and never runs: there is no GPU here), and runs the driver: argument
validation, workspace sizes and carving, dispatch-size arithmetic and the
log-probability checks, for the same bad arguments as test_boundary.py and
for valid calls that go as far as the launch.

The valid calls carry made-up device addresses: with a GPU present they would
launch kernels on memory that does not exist.  So the test is skipped where a
GPU device node exists, and the driver itself refuses to run (exit 77) when
HIP reports a device.
"""
import os
import subprocess
import tempfile

import pytest

from attention_sink_fwd_amd.build import CSRC, HIPCC, ROOT, SOURCES

pytestmark = [
    pytest.mark.slow,
    pytest.mark.skipif(os.path.exists("/dev/kfd"), reason="needs a machine without a GPU (made-up device addresses)"),
]

SANITIZE = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
            "-Xarch_host", "-fno-sanitize-recover=undefined", "-fno-gpu-sanitize"]


def test_host_code_is_clean_under_asan_and_ubsan():
    driver = os.path.join(ROOT, "tests", "host_sanitizer_driver.cpp")
    with tempfile.TemporaryDirectory() as d:
        exe = os.path.join(d, "driver")
        cmd = [HIPCC, "--offload-arch=gfx950", "-O1", "-g", "-std=c++17",
               "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", *SANITIZE,
               "-I", os.path.join(ROOT, "include"), "-I", CSRC,
               *[os.path.join(CSRC, s) for s in SOURCES], driver, "-o", exe]
        r = subprocess.run(cmd, capture_output=True, text=True)
        assert r.returncode == 0, r.stderr[-3000:]
        env = dict(os.environ)
        env["ASAN_OPTIONS"] = "detect_leaks=0:abort_on_error=1"
        env["UBSAN_OPTIONS"] = "halt_on_error=1:print_stacktrace=1"
        env.pop("SINK_ATTN_DKDV_HEADS", None)
        env.pop("SINK_ATTN_PACK_HEADS", None)
        env.pop("SINK_ATTN_VALIDATE", None)
        env["SINK_ATTN_TRACE"] = "1"  # the trace path formats every launch's line
        r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=300)
        out = r.stdout + r.stderr
        if r.returncode == 77 and "skipped: a GPU is visible" in out:
            pytest.skip("a GPU is visible: the driver's made-up device addresses must not reach a launch")
        assert r.returncode == 0, out[-4000:]
        assert "host checks passed" in out, out[-4000:]
        assert "runtime error" not in out and "AddressSanitizer" not in out, out[-4000:]
