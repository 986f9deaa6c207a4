"""The C ABI's host code (validation, workspace layout, dispatch) built with
the host C++ compiler under AddressSanitizer and UndefinedBehaviorSanitizer,
with stub launchers in place of the GPU kernels, and driven through valid and
invalid argument sets (tests/host/abi_driver.cpp).  CPU only."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "shared_kv_attention_amd", "csrc")
HOST = os.path.join(ROOT, "tests", "host")


@pytest.mark.skipif(shutil.which("g++") is None or not os.path.isdir("/opt/rocm/include"),
                    reason="needs g++ and the ROCm headers")
def test_abi_host_code_under_sanitizers(tmp_path):
    exe = tmp_path / "abi_driver"
    cmd = ["g++", "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
           "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include",
           os.path.join(CSRC, "abi.cpp"), os.path.join(CSRC, "plan.cpp"),
           os.path.join(HOST, "stub_launch.cpp"), os.path.join(HOST, "abi_driver.cpp"),
           "-o", str(exe)]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-4000:]
    # a library preloaded by the environment may come before the sanitizer
    # runtime: let it (the link-order check is the only thing that objects)
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:verify_asan_link_order=0",
               UBSAN_OPTIONS="print_stacktrace=1")
    r = subprocess.run([str(exe)], capture_output=True, text=True, env=env, timeout=120)
    assert r.returncode == 0, (r.stdout + r.stderr)[-4000:]
    assert "all checks passed" in r.stdout
