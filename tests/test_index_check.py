"""The kernels' index arithmetic (shared_kv_attention_amd/csrc/index_map.hpp:
workgroup maps, key spans, LDS swizzles, staging slots and fragment offsets,
decode splits and lane offsets) built for the host with YOCO_CHECK_BOUNDS
(every helper asserts its preconditions) under AddressSanitizer and
UndefinedBehaviorSanitizer, and enumerated over every workgroup, lane and
slot of a set of launch shapes (tests/host/index_check.cpp).  CPU only."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "shared_kv_attention_amd", "csrc")
HOST = os.path.join(ROOT, "tests", "host")


@pytest.mark.skipif(shutil.which("g++") is None or not os.path.isdir("/opt/rocm/include"),
                    reason="needs g++ and the ROCm headers")
def test_index_arithmetic_enumerated_with_bounds_checks(tmp_path):
    exe = tmp_path / "index_check"
    cmd = ["g++", "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
           "-DYOCO_CHECK_BOUNDS", "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include", "-I", CSRC,
           os.path.join(HOST, "index_check.cpp"), os.path.join(CSRC, "plan.cpp"),
           "-o", str(exe)]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-4000:]
    # a library preloaded by the environment may come before the sanitizer
    # runtime: let it (the link-order check is the only thing that objects)
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:verify_asan_link_order=0",
               UBSAN_OPTIONS="print_stacktrace=1")
    r = subprocess.run([str(exe)], capture_output=True, text=True, env=env, timeout=300)
    assert r.returncode == 0, (r.stdout + r.stderr)[-4000:]
    assert "all index checks passed" in r.stdout
