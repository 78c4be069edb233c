"""The C ABI's host code under AddressSanitizer, on the CPU (no GPU is touched).

Builds the library sources with the sanitizer on the host side only (device code is compiled as
usual) together with tests/asan/host_checks.cpp, and runs that program: every validation and error
path, and an init that must fail cleanly without a device, with leak checking on."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "dispatch_fp8_grouped_amd", "csrc")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")


@pytest.mark.skipif(not os.path.exists(HIPCC), reason="hipcc not installed")
def test_host_abi_under_address_sanitizer(tmp_path):
    srcs = [os.path.join(CSRC, f) for f in ("host.hip", "route.hip", "fill.hip", "gemm.hip", "combine.hip",
                                            "pack.hip")]
    exe = str(tmp_path / "host_checks")
    cmd = [HIPCC, "--offload-arch=gfx950", "-O1", "-g", "-std=c++17",
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
           "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fno-omit-frame-pointer",
           os.path.join(ROOT, "tests", "asan", "host_checks.cpp"), *srcs, "-o", exe]
    res = subprocess.run(cmd, capture_output=True, text=True)
    assert res.returncode == 0, res.stderr[-4000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0", HIP_VISIBLE_DEVICES="",
               ROCR_VISIBLE_DEVICES="")
    run = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=300)
    assert run.returncode == 0 and "host checks ok" in run.stdout, (run.stdout + run.stderr)[-6000:]
