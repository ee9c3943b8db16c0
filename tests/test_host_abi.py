"""The C ABI's host layer under AddressSanitizer and UndefinedBehaviorSanitizer,
without a GPU: tests/host/abi_host_test.cpp compiles api.cpp with g++ next to
stub kernel launchers and stub HIP runtime calls, and checks every refusal
(status, message, nothing launched), accepted calls (one launch, split buffers
inside the caller's workspace), plan/call agreement, the epoch generator's
wrap past 0 and random arguments."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.skipif(shutil.which("g++") is None or not os.path.isdir("/opt/rocm/include"),
                    reason="needs g++ and the ROCm headers")
def test_host_abi_under_sanitizers(tmp_path):
    exe = tmp_path / "abi_host_test"
    cmd = ["g++", "-std=c++20", "-O1", "-g", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
           "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include", "-I", os.path.join(ROOT, "include"),
           "-I", os.path.join(ROOT, "fp8_paged_kv_amd", "csrc"),
           os.path.join(ROOT, "tests", "host", "abi_host_test.cpp"), "-o", str(exe)]
    r = subprocess.run(cmd, capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, r.stderr[-4000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:verify_asan_link_order=0",
               UBSAN_OPTIONS="print_stacktrace=1")
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=300, env=env)
    assert r.returncode == 0 and "ALL OK" in r.stdout, (r.stdout[-4000:] + r.stderr[-4000:])
