"""The C ABI's host side (csrc/uf_api.cpp) under AddressSanitizer and UndefinedBehaviorSanitizer.

The host source is built with g++ against launch stubs (tests/host_stub/launch_stub.cpp), which
check the launch parameters and launch nothing, and tests/test_host_abi.py then runs against
that build in a child process: every validation path, the window bookkeeping and, through the
stubs, every valid call's host path.  A sanitizer report fails the child and this test.
"""
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "windowed_attention_amd", "csrc")
OUT = os.path.join(ROOT, "_build", "libuf_host_sanitized.so")


def _asan_runtime():
    if not shutil.which("g++"):
        return None
    path = subprocess.run(["g++", "-print-file-name=libasan.so"], capture_output=True, text=True).stdout.strip()
    return path if os.path.isabs(path) and os.path.exists(path) else None


@pytest.mark.skipif(_asan_runtime() is None or not os.path.exists("/opt/rocm/include/hip/hip_runtime_api.h"),
                    reason="needs g++ with libasan and the HIP headers")
def test_host_side_under_sanitizers():
    os.makedirs(os.path.dirname(OUT), exist_ok=True)
    san = ["-fsanitize=address", "-fsanitize=undefined", "-fno-sanitize-recover=undefined"]
    cmd = ["g++", "-std=c++17", "-fPIC", "-shared", "-g", "-O1", "-fno-omit-frame-pointer", *san,
           "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include", "-I" + os.path.join(ROOT, "include"), "-I" + CSRC,
           os.path.join(CSRC, "uf_api.cpp"), os.path.join(ROOT, "tests", "host_stub", "launch_stub.cpp"),
           "-L/opt/rocm/lib", "-Wl,-rpath,/opt/rocm/lib", "-lamdhip64", "-o", OUT]
    subprocess.run(cmd, check=True)
    env = dict(os.environ, UF_LIBRARY_PATH=OUT, LD_PRELOAD=_asan_runtime(),
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=1", UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    res = subprocess.run([sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider",
                          os.path.join(ROOT, "tests", "test_host_abi.py")],
                         cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    print(res.stdout[-3000:], res.stderr[-3000:])
    assert res.returncode == 0
    assert "passed" in res.stdout and "skipped" not in res.stdout   # the stub-only test ran too
    assert "ERROR: AddressSanitizer" not in res.stderr and "runtime error" not in res.stderr
