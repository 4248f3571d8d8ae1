"""Builds liblsa.so (the HIP kernels and the C ABI) for gfx950 with hipcc.

Every source is compiled in its own process, then linked; packed-fp32 VALU
instructions are disabled for all device code.  Device code is compiled
assuming no NaNs (float min/max then need no operand canonicalisation): the
library's contract leaves results for non-finite inputs unspecified, and no
memory access depends on a float value.
"""
from __future__ import annotations

import concurrent.futures
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "liblsa.so")
SOURCES = ["summarize.hip", "route.hip", "tree.hip", "attend.hip", "decode.hip", "lsa_api.hip"]
ARCH = os.environ.get("LSA_OFFLOAD_ARCH", "gfx950")

FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Xarch_device", "-fno-honor-nans",
    "-Wall", "-Wno-unused-result", "-I", INCLUDE, "-I", CSRC,
]


def _hipcc():
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    return os.path.join(rocm, "bin", "hipcc")


def build(verbose: bool = False) -> str:
    objdir = os.path.join(PKG, "_build")
    os.makedirs(objdir, exist_ok=True)

    def compile_one(src):
        obj = os.path.join(objdir, src + ".o")
        cmd = [_hipcc(), *FLAGS, "-c", os.path.join(CSRC, src), "-o", obj]
        r = subprocess.run(cmd, capture_output=True, text=True)
        noise = "packed-fp32-ops"  # the host pass does not know the feature
        err = "\n".join(l for l in r.stderr.splitlines() if noise not in l)
        if r.returncode != 0:
            raise RuntimeError(f"hipcc failed on {src}:\n{err}")
        if verbose and err.strip():
            print(err, file=sys.stderr)
        return obj

    with concurrent.futures.ThreadPoolExecutor(max_workers=len(SOURCES)) as ex:
        objs = list(ex.map(compile_one, SOURCES))
    tmp = LIB + ".tmp"
    subprocess.check_call([_hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs,
                           "-o", tmp])
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
