"""Build libyoco.so (the gfx950 HIP kernels + C ABI) in-tree with hipcc.

Usage: python -m shared_kv_attention_amd.build [--jobs N]
Objects go to _build/ at the repository root; the library is written next to
this file so the Python binding (and any C caller) finds it.
"""
import argparse
import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libyoco.so")

SOURCES = ["attn_fwd.hip", "decode.hip", "kv_proj.hip", "linear.hip", "fp8_quant.hip", "gret.hip", "peak.hip", "noalloc.hip", "plan.cpp", "abi.cpp"]

HIPCC = os.environ.get("HIPCC", shutil.which("hipcc") or "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
CFLAGS = [
    "-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
    # keep the compiler from forming packed-FP32 VALU instructions
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument",
    "-I", os.path.join(ROOT, "include"),
]


def _compile(src):
    obj = os.path.join(BUILD, src + ".o")
    cmd = [HIPCC, *CFLAGS, "-c", os.path.join(CSRC, src), "-o", obj]
    if src.endswith(".cpp"):
        cmd[1:1] = ["-x", "hip"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stderr}")
    return obj


# A test-only library over decode.hip (tests/gpu_lib): runs the decode kernels
# with an explicit split plan and K-load form, for the test that compares the
# two forms bitwise.  Built with the product so that GPU runs need no compiler.
TEST_LIB = os.path.join(ROOT, "tests", "gpu_lib", "libyoco_decode_forms.so")
TEST_SRC = os.path.join(ROOT, "tests", "gpu_lib", "decode_forms.hip")


def build_test_lib(verbose=True):
    obj = os.path.join(BUILD, "decode_forms.hip.o")
    r = subprocess.run([HIPCC, *CFLAGS, "-c", TEST_SRC, "-o", obj], capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {TEST_SRC}:\n{r.stderr}")
    objs = [obj, os.path.join(BUILD, "decode.hip.o"), os.path.join(BUILD, "plan.cpp.o")]
    tmp = TEST_LIB + ".tmp"
    r = subprocess.run([HIPCC, "-shared", "-fPIC", f"--offload-arch={ARCH}", *objs, "-o", tmp],
                       capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, TEST_LIB)
    if verbose:
        print(f"built {TEST_LIB}")
    return TEST_LIB


def build(jobs=None, verbose=True):
    """Compile every source for gfx950 and link libyoco.so (and the test-only
    decode-form library); returns libyoco.so's path."""
    os.makedirs(BUILD, exist_ok=True)
    jobs = jobs or min(len(SOURCES), os.cpu_count() or 4, 8)
    with cf.ThreadPoolExecutor(jobs) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, "-shared", "-fPIC", f"--offload-arch={ARCH}", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    build_test_lib(verbose)
    return LIB


if __name__ == "__main__":
    ap = argparse.ArgumentParser()
    ap.add_argument("--jobs", type=int, default=None)
    args = ap.parse_args()
    try:
        build(args.jobs)
    except RuntimeError as e:
        print(e, file=sys.stderr)
        sys.exit(1)
