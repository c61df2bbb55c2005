"""The boundary from C and C++: include/mb.h compiles as C11 and as C++17, a
program linked against libmb.so calls it, and the calls that need no GPU
(version, status names, validation, workspace queries) behave as declared."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LIBDIR = os.path.join(ROOT, "transformer_elementwise_epilogues_amd")
SRC = os.path.join(ROOT, "tests", "abi_c", "caller.c")


@pytest.mark.parametrize("compiler,std", [("gcc", ["-x", "c", "-std=c11"]), ("g++", ["-x", "c++", "-std=c++17"])])
def test_c_caller(tmp_path, compiler, std):
    if not shutil.which(compiler):
        pytest.skip(f"{compiler} not found")
    if not os.path.exists(os.path.join(LIBDIR, "libmb.so")):
        pytest.skip("libmb.so not built")
    exe = tmp_path / "caller"
    cmd = [compiler, *std, "-Wall", "-Wextra", "-Werror", "-D__HIP_PLATFORM_AMD__", "-I", os.path.join(ROOT, "include"),
           "-isystem", "/opt/rocm/include", SRC, "-o", str(exe), "-L", LIBDIR, "-lmb", f"-Wl,-rpath,{LIBDIR}"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=60)
    assert r.returncode == 0 and r.stdout.strip().endswith("ok"), r.stdout + r.stderr
