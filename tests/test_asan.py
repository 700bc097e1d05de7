"""The host side of the library (plan builder, C ABI, argument checks, plan
cache) under AddressSanitizer, on the CPU.

Builds a copy of libfsa whose host code carries -fsanitize=address (the
device code is built as usual; nothing is launched without a GPU) into
_build/, then runs the
plan and ABI test modules in a child process that loads it, with the
sanitizer runtime preloaded into the interpreter. Any invalid read or write,
use after free or double free in the host code fails the child.
"""
import glob
import os
import subprocess
import sys

import pytest

from frame_aligned_block_amd import build as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
OUT = os.path.join(ROOT, "_build", "libfsa_asan.so")


def asan_runtime():
    hits = sorted(glob.glob("/opt/rocm/lib/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    return hits[-1] if hits else None


@pytest.fixture(scope="module")
def asan_lib():
    rt = asan_runtime()
    if rt is None:
        pytest.skip("no clang AddressSanitizer runtime in this image")
    os.makedirs(os.path.dirname(OUT), exist_ok=True)
    srcs = []
    for s in B.SOURCES:
        srcs += ["-x", "hip", os.path.join(B.CSRC, s)]
    cmd = [B.hipcc(), f"--offload-arch={B.ARCH}", "-O1", "-g", "-std=c++17", "-fPIC", "-shared",
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
           "-mllvm", "-amdgpu-mfma-vgpr-form=1",
           "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fno-omit-frame-pointer",
           "-I", B.INCLUDE, *srcs, "-o", OUT]
    res = subprocess.run(cmd, capture_output=True, text=True)
    assert res.returncode == 0, res.stdout + res.stderr
    return rt


def test_host_code_under_asan(asan_lib):
    env = dict(os.environ, FSA_LIBRARY=OUT, LD_PRELOAD=asan_lib,
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=1:halt_on_error=1")
    res = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                          "-m", "not gpu", "tests/test_plan.py", "tests/test_abi.py"],
                         cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    out = res.stdout + res.stderr
    assert "AddressSanitizer" not in out, out[-4000:]
    assert res.returncode == 0, out[-4000:]
    assert " passed" in out


PLANTED = """
import ctypes, numpy as np
from frame_aligned_block_amd import fsa
p = fsa.fsa_plan_create(fsa.make_shape(1, 1, 5, 48, 64, 1, 0, 0, 0, fsa.FSA_F32))
nq, nnz = ctypes.c_int32(), ctypes.c_int64()
fsa.lib().fsa_plan_export(p, None, None, None, None, ctypes.byref(nq), ctypes.byref(nnz))
small = np.zeros(int(nnz.value) // 2, np.int32)      # half the tile list: the copy overruns it
fsa.lib().fsa_plan_export(p, None, small.ctypes.data, None, None, None, None)
"""


def test_sanitizer_is_live(asan_lib):
    """Control: the same build and preload catch a planted host overrun (the
    caller hands fsa_plan_export an array half the tile list's size)."""
    env = dict(os.environ, FSA_LIBRARY=OUT, LD_PRELOAD=asan_lib, PYTHONPATH=ROOT,
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=1:halt_on_error=1")
    res = subprocess.run([sys.executable, "-c", PLANTED], cwd=ROOT, env=env, capture_output=True,
                         text=True, timeout=120)
    assert "AddressSanitizer: heap-buffer-overflow" in res.stdout + res.stderr
    assert res.returncode != 0
