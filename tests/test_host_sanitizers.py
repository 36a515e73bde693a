"""The C ABI's host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

api.cpp -- every argument check, size query and workspace carving -- is compiled with g++
and -fsanitize=address,undefined into a shared library that takes the kernels' launchers
from the in-tree libqlinear.so, and tests/test_abi.py runs against it in a child process
(ASan runtime preloaded, leak checking off: the interpreter itself is not instrumented).
The argument-error tests launch nothing, so no GPU is needed; any sanitizer report fails.
"""
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PKG = os.path.join(ROOT, "quantized_linear_layers_block_amd")


def test_abi_checks_under_host_sanitizers(tmp_path):
    if not os.path.exists(os.path.join(PKG, "libqlinear.so")):
        pytest.skip("libqlinear.so is not built")
    gxx = shutil.which("g++")
    if gxx is None or not os.path.isdir("/opt/rocm/include"):
        pytest.skip("g++ or the ROCm headers are missing")
    asan = subprocess.run([gxx, "-print-file-name=libasan.so"], capture_output=True, text=True).stdout.strip()
    if not os.path.exists(asan):
        pytest.skip("no host AddressSanitizer runtime")
    lib = tmp_path / "libqlinear_api_sanitized.so"
    build = [gxx, "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
             "-fno-sanitize-recover=undefined", "-shared", "-fPIC", "-D__HIP_PLATFORM_AMD__",
             "-I/opt/rocm/include", "-I" + os.path.join(ROOT, "include"), os.path.join(PKG, "csrc", "api.cpp"),
             "-o", str(lib), "-Wl,-Bsymbolic", "-L" + PKG, "-l:libqlinear.so", "-Wl,-rpath," + PKG]
    r = subprocess.run(build, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-4000:]
    env = dict(os.environ, QLINEAR_LIB=str(lib), QLINEAR_NO_TORCH="1", LD_PRELOAD=asan,
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_abi.py")],
                       env=env, capture_output=True, text=True, timeout=600, cwd=ROOT)
    report = r.stdout[-4000:] + r.stderr[-4000:]
    assert r.returncode == 0, report
    assert "AddressSanitizer" not in r.stderr and "runtime error" not in r.stderr, report
    assert " passed" in r.stdout, report
