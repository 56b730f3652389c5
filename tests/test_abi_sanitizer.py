"""The C ABI's validation paths under AddressSanitizer and UBSan (host code
only), on a machine without a GPU: the library sources and
tests/abi_sanitizer_driver.cpp are built with the sanitizers on the host
side, and the driver runs every argument error of idattn_forward and
idattn_decode_step plus the workspace query over every supported shape.  No
call reaches a HIP launch."""
import os
import subprocess
import tempfile

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "fixed_state_ssm_amd", "csrc")
from fixed_state_ssm_amd.build import SOURCES  # noqa: E402
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")


@pytest.mark.skipif(not os.path.exists(HIPCC), reason="hipcc not available")
def test_abi_validation_under_host_sanitizers():
    with tempfile.TemporaryDirectory() as td:
        exe = os.path.join(td, "abi_driver")
        cmd = [HIPCC, "--offload-arch=gfx950", "-O1", "-std=c++17",
               "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
               "-Xarch_host", "-fno-omit-frame-pointer", "-Xarch_host", "-fno-sanitize-recover=all",
               "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
               "-I", os.path.join(ROOT, "include"),
               *[os.path.join(CSRC, s) for s in SOURCES],
               os.path.join(ROOT, "tests", "abi_sanitizer_driver.cpp"), "-o", exe]
        build = subprocess.run(cmd, capture_output=True, text=True)
        assert build.returncode == 0, build.stderr[-3000:]
        env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:halt_on_error=1", UBSAN_OPTIONS="halt_on_error=1")
        run = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=120)
        assert run.returncode == 0, run.stdout[-3000:] + run.stderr[-3000:]
        assert "0 failed" in run.stdout, run.stdout
