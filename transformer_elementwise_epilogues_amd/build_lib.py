"""Builds libmb.so (the HIP kernels and the C ABI) in-tree with hipcc for gfx950.

    python -m transformer_elementwise_epilogues_amd.build_lib

Every HIP translation unit is compiled with packed-fp32 instructions disabled
(``-target-feature -packed-fp32-ops``): the kernels are written as scalar
fp32 code and must not be turned into v_pk_* FMA forms.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build", "libmb")
LIB = os.path.join(PKG, "libmb.so")
# the benchmark's streaming-ceiling kernel: a library of its own, outside the ABI
STREAM_SOURCES = ["mb_stream.hip"]
STREAM_LIB = os.path.join(PKG, "libmb_stream.so")

SOURCES = ["mb_gelu.hip", "mb_bda.hip", "mb_glu.hip", "mb_reduce.hip", "mb_ln.hip", "mb_sqrelu.hip", "mb_noalloc.hip",
           "mb_plan.cpp", "mb_abi.cpp"]
ARCH = "gfx950"


def hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found: the fused-epilogue library needs ROCm's hipcc to build")


def common_flags(extra=()):
    return ["-O3", "-std=c++17", "-fPIC", "-Wall", "-Wno-unused-function", f"--offload-arch={ARCH}",
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            "-I", INCLUDE, "-I", CSRC, *extra]


def _compile(src: str, extra) -> str:
    obj = os.path.join(BUILD, os.path.basename(src) + ".o")
    cmd = [hipcc(), *common_flags(extra), "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{r.stdout}\n{r.stderr}")
    return obj


def build(extra_flags=(), out: str = LIB, verbose: bool = False, sources=SOURCES) -> str:
    """Compile every source and link libmb.so (always rebuilds)."""
    os.makedirs(BUILD, exist_ok=True)
    with ThreadPoolExecutor(len(sources)) as ex:
        objs = list(ex.map(lambda s: _compile(s, extra_flags), sources))
    tmp = out + ".tmp%d" % os.getpid()
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, out)
    if verbose:
        print("built", out)
    return out


def build_stream(extra_flags=(), verbose: bool = False) -> str:
    """The benchmark's streaming-ceiling library, libmb_stream.so."""
    return build(extra_flags, out=STREAM_LIB, verbose=verbose, sources=STREAM_SOURCES)


if __name__ == "__main__":
    build(extra_flags=sys.argv[1:], verbose=True)
    build_stream(extra_flags=sys.argv[1:], verbose=True)
