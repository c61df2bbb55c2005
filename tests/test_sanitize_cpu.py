"""Host code under the address and undefined-behaviour sanitizers (no GPU):
the oracle (oracle/oracle.c, and its binary32 twin oracle32.c) on every
entry point with edge and special values, and the C ABI's validation, workspace queries and launch planning
(mb_abi.cpp, mb_plan.cpp) with hostile arguments, linked against launch
stand-ins. Any out-of-bounds access, signed overflow, misaligned or invalid
operation aborts the program and fails the test."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HERE = os.path.join(ROOT, "tests", "sanitize_c")
CSRC = os.path.join(ROOT, "transformer_elementwise_epilogues_amd", "csrc")
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", "-g", "-O1"]
ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=1", UBSAN_OPTIONS="print_stacktrace=1")


def run(cmd, exe):
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-4000:]
    r = subprocess.run([exe], capture_output=True, text=True, timeout=300, env=ENV)
    assert r.returncode == 0 and r.stdout.strip().endswith("ok"), (r.stdout + r.stderr)[-4000:]


def test_oracle_sanitized(tmp_path):
    if not shutil.which("gcc"):
        pytest.skip("gcc not found")
    exe = str(tmp_path / "oracle_san")
    run(["gcc", "-std=c11", "-ffp-contract=off", "-fno-fast-math", *SAN, os.path.join(ROOT, "oracle", "oracle.c"),
         os.path.join(HERE, "oracle_driver.c"), "-o", exe, "-lm"], exe)


def test_oracle32_sanitized(tmp_path):
    if not shutil.which("gcc"):
        pytest.skip("gcc not found")
    exe = str(tmp_path / "oracle32_san")
    run(["gcc", "-std=c11", "-ffp-contract=off", "-fno-fast-math", *SAN, os.path.join(ROOT, "oracle", "oracle.c"),
         os.path.join(ROOT, "oracle", "oracle32.c"), os.path.join(HERE, "oracle32_driver.c"), "-o", exe, "-lm"], exe)


def test_abi_host_code_sanitized(tmp_path):
    if not shutil.which("g++") or not os.path.exists("/opt/rocm/lib/libamdhip64.so"):
        pytest.skip("g++ or the HIP runtime library not found")
    exe = str(tmp_path / "abi_san")
    run(["g++", "-std=c++17", *SAN, "-D__HIP_PLATFORM_AMD__", "-I", os.path.join(ROOT, "include"), "-I", CSRC,
         "-isystem", "/opt/rocm/include", os.path.join(CSRC, "mb_abi.cpp"), os.path.join(CSRC, "mb_plan.cpp"),
         os.path.join(HERE, "abi_stubs.cpp"), os.path.join(HERE, "abi_driver.cpp"), "-o", exe,
         "-L/opt/rocm/lib", "-lamdhip64", "-Wl,-rpath,/opt/rocm/lib"], exe)
