"""AddressSanitizer + UndefinedBehaviorSanitizer builds of the host code, on the CPU: the C oracle
(tests/oracle_check.c: round trips, random bytes through every decoder, calibration, coverage,
attention) and the host half of the C ABI (api.cpp with the kernel launchers stubbed,
tests/abi_host_check.cpp: parameter validation, sizes, admission and argument errors of every
entry point).  Any out-of-bounds access, leak or undefined behaviour aborts the program."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", "-g", "-O1"]
ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=1", UBSAN_OPTIONS="print_stacktrace=1")


def _run(exe):
    res = subprocess.run([str(exe)], capture_output=True, text=True, timeout=300, env=ENV)
    assert res.returncode == 0 and res.stdout.startswith("ok"), (res.returncode, res.stdout[-2000:], res.stderr[-4000:])


def test_oracle_under_asan_ubsan(tmp_path):
    exe = tmp_path / "oracle_check"
    subprocess.check_call(["gcc", *SAN, "-std=c11", os.path.join(ROOT, "oracle", "kvc_oracle.c"),
                           os.path.join(ROOT, "tests", "oracle_check.c"), "-o", str(exe), "-lm"])
    _run(exe)


@pytest.mark.skipif(not os.path.isdir("/opt/rocm/include"), reason="needs the HIP host headers")
def test_abi_host_code_under_asan_ubsan(tmp_path):
    exe = tmp_path / "abi_host_check"
    inc = ["-I", os.path.join(ROOT, "include"), "-I", os.path.join(ROOT, "decode_attention_calibrate_amd", "csrc"),
           "-I", "/opt/rocm/include", "-D__HIP_PLATFORM_AMD__"]
    subprocess.check_call(["g++", *SAN, "-std=c++17", *inc,
                           os.path.join(ROOT, "decode_attention_calibrate_amd", "csrc", "api.cpp"),
                           os.path.join(ROOT, "tests", "abi_launch_stubs.cpp"),
                           os.path.join(ROOT, "tests", "abi_host_check.cpp"),
                           "-L/opt/rocm/lib", "-lamdhip64", "-Wl,-rpath,/opt/rocm/lib", "-o", str(exe)])
    _run(exe)
