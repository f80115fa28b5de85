"""The host planner under AddressSanitizer and UndefinedBehaviorSanitizer.

fia_api.cpp (argument validation, shape / stride / offset arithmetic, work
planning and workspace layout) is built host-only with g++ against
stand-ins for the HIP runtime and the kernel launchers
(tests/hostcheck/hip_host_stubs.cpp), and the C-ABI phase-1 tests of
test_abi_cpu.py run against that build in a child process with the ASan
runtime loaded first.  Any sanitizer report fails the child, and with it this
test."""
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "attention_online_softmax_flash_amd", "csrc")


def _build(gxx, out):
    cmd = [gxx, "-std=c++17", "-O1", "-g", "-fPIC", "-shared", "-fno-omit-frame-pointer",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
           "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include", "-I", os.path.join(ROOT, "include"),
           "-I", CSRC, os.path.join(CSRC, "fia_api.cpp"),
           os.path.join(ROOT, "tests", "hostcheck", "hip_host_stubs.cpp"), "-o", out]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-4000:]


def test_phase1_under_asan_and_ubsan(tmp_path):
    gxx = shutil.which("g++")
    if gxx is None or not os.path.isdir("/opt/rocm/include"):
        pytest.skip("needs g++ and the ROCm headers")
    libasan = subprocess.run([gxx, "-print-file-name=libasan.so"], capture_output=True,
                             text=True).stdout.strip()
    if not os.path.isabs(libasan) or not os.path.exists(libasan):
        pytest.skip("libasan is not available")
    lib = str(tmp_path / "libfia_hostcheck.so")
    _build(gxx, lib)
    # the build is instrumented: it calls the ASan and UBSan report hooks
    syms = subprocess.run(["nm", "-D", lib], capture_output=True, text=True).stdout
    assert "__asan_report_load" in syms and "__ubsan_handle_" in syms
    env = dict(os.environ)
    env["FIA_HOSTCHECK_LIB"] = lib
    # The ASan runtime must come first among the preloaded libraries.
    env["LD_PRELOAD"] = libasan + (":" + env["LD_PRELOAD"] if env.get("LD_PRELOAD") else "")
    env["ASAN_OPTIONS"] = "detect_leaks=0:abort_on_error=0:halt_on_error=1:exitcode=23"
    env["UBSAN_OPTIONS"] = "print_stacktrace=1:halt_on_error=1:exitcode=24"
    r = subprocess.run([sys.executable, "-m", "pytest", os.path.join(ROOT, "tests", "test_abi_cpu.py"),
                        "-q", "-x", "-m", "not gpu", "-p", "no:cacheprovider"],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    tail = (r.stdout + r.stderr)[-6000:]
    assert r.returncode == 0, tail
    assert "passed" in r.stdout and "ERROR: AddressSanitizer" not in tail and "runtime error" not in tail, tail
