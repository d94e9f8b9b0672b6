"""Host sanitizer build (CPU only): the C-ABI layer (fb_abi.cpp) and the host SVD (fb_svd.cpp)
compiled for the host alone with AddressSanitizer and UndefinedBehaviorSanitizer, the kernel
launchers replaced by stubs (tests/native/launch_stubs.cpp), and driven by
tests/native/abi_sanitize.cpp: argument validation of the entry points, workspace sizes and the
truncated SVD on matrices with chosen singular values.  Any memory error or undefined behaviour
aborts the driver."""
import glob
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "attention_additive_rank_amd", "csrc")
NATIVE = os.path.join(ROOT, "tests", "native")


def _host_clang():
    for c in ("/opt/rocm/lib/llvm/bin/clang++", shutil.which("clang++") or ""):
        if c and os.path.exists(c):
            return c
    return None


CXX = _host_clang()


@pytest.mark.skipif(CXX is None or not glob.glob("/opt/rocm/include/hip/hip_runtime_api.h"),
                    reason="needs a host clang++ and the HIP headers")
def test_abi_and_svd_under_asan_ubsan(tmp_path):
    exe = tmp_path / "abi_sanitize"
    srcs = [os.path.join(CSRC, "fb_abi.cpp"), os.path.join(CSRC, "fb_svd.cpp"),
            os.path.join(NATIVE, "launch_stubs.cpp"), os.path.join(NATIVE, "abi_sanitize.cpp")]
    # host code only (-x c++ names no device source): the sanitizers instrument the host
    cmd = [CXX, "-x", "c++", "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-D__HIP_PLATFORM_AMD__",
           "-I/opt/rocm/include", "-I", CSRC, "-I", os.path.join(ROOT, "include")] + srcs + \
          ["-x", "none", "-o", str(exe), "-lpthread"]
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True, timeout=600)
    assert r.returncode == 0, r.stdout[-4000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    r = subprocess.run([str(exe)], stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True, timeout=300, env=env)
    print(r.stdout[-4000:])
    assert r.returncode == 0, r.stdout[-4000:]
    assert "ok: 0 failed checks" in r.stdout
