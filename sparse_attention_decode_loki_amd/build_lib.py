"""Build libloki.so in-tree for gfx950 with hipcc (no GPU needed).

    python -m sparse_attention_decode_loki_amd.build_lib
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
OBJ = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libloki.so")

ARCH = os.environ.get("LOKI_OFFLOAD_ARCH", "gfx950")
HIP_SOURCES = ["decode_kernels.hip", "fused_kernels.hip", "append_kernels.hip", "probe_kernels.hip",
               "api.hip"]
CXX_SOURCES = ["calibrate.cpp"]
# Packed-FP32 instructions are disabled for all device code.
HIPCC_FLAGS = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}", "-Wall",
               "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
               "-I", os.path.join(ROOT, "include")]
CXX_FLAGS = ["-O2", "-std=c++17", "-fPIC", "-Wall", "-I", os.path.join(ROOT, "include")]


C_CLIENT_SRC = os.path.join(ROOT, "tests", "host", "c_client.c")
C_CLIENT = os.path.join(ROOT, "tests", "host", "c_client")


def build_c_client() -> str:
    """The plain-C test client of the ABI (tests/host/c_client.c), linked
    against the in-tree libloki.so and the HIP runtime."""
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    _run(["gcc", "-std=c99", "-O2", "-Wall", "-D__HIP_PLATFORM_AMD__",
          "-I", os.path.join(rocm, "include"), "-I", os.path.join(ROOT, "include"), C_CLIENT_SRC,
          "-L", PKG, "-lloki", "-L", os.path.join(rocm, "lib"), "-lamdhip64", "-lm",
          "-Wl,-rpath,$ORIGIN/../../sparse_attention_decode_loki_amd:" + os.path.join(rocm, "lib"),
          "-o", C_CLIENT])
    return C_CLIENT


def _hipcc() -> str:
    for c in (shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found")


def _run(cmd):
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("build step failed:\n" + " ".join(cmd) + "\n" + r.stdout + r.stderr)
    return r


def build(verbose: bool = False) -> str:
    os.makedirs(OBJ, exist_ok=True)
    hipcc = _hipcc()
    jobs = []
    for src in HIP_SOURCES:
        obj = os.path.join(OBJ, src + ".o")
        jobs.append([hipcc, *HIPCC_FLAGS, "-c", os.path.join(CSRC, src), "-o", obj])
    for src in CXX_SOURCES:
        obj = os.path.join(OBJ, src + ".o")
        jobs.append(["g++", *CXX_FLAGS, "-c", os.path.join(CSRC, src), "-o", obj])
    with ThreadPoolExecutor(len(jobs)) as ex:
        for r in ex.map(_run, jobs):
            if verbose and (r.stdout or r.stderr):
                print(r.stdout + r.stderr, file=sys.stderr)
    objs = [j[-1] for j in jobs]
    tmp = LIB + ".tmp"
    _run([hipcc, "-shared", f"--offload-arch={ARCH}", "-o", tmp, *objs])
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
    print(build_c_client())
