"""The library's host side (argument validation, planning, workspace sizes;
aq_api.cpp and aq_plan.cpp) built with AddressSanitizer and
UndefinedBehaviorSanitizer by the host C++ compiler, with stand-in kernel
launchers, and run without a GPU: every entry point rejects invalid
arguments before any launch, and a launch failure forced from the host
comes back as AQ_ERR_HIP (tests/sanitize/)."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.timeout(600)
def test_host_side_under_asan_ubsan(tmp_path):
    cxx = shutil.which("g++")
    if cxx is None:
        pytest.skip("no host C++ compiler")
    exe = str(tmp_path / "abi_host_check")
    src = [os.path.join(ROOT, "mixed_precision_int_amd", "csrc", "aq_api.cpp"),
           os.path.join(ROOT, "mixed_precision_int_amd", "csrc", "aq_plan.cpp"),
           os.path.join(ROOT, "tests", "sanitize", "launch_stubs.cpp"),
           os.path.join(ROOT, "tests", "sanitize", "abi_host_check.cpp")]
    cmd = [cxx, "-std=c++17", "-O1", "-g", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
           "-fno-omit-frame-pointer", "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include",
           "-I" + os.path.join(ROOT, "include"), *src, "-o", exe]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-4000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0", UBSAN_OPTIONS="print_stacktrace=1")
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=300)
    assert r.returncode == 0 and "host ABI check: ok" in r.stdout, (r.stdout[-4000:], r.stderr[-4000:])
