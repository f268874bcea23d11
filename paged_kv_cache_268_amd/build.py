"""Build libpkv.so in-tree with hipcc for gfx950.

    python -m paged_kv_cache_268_amd.build

Every HIP source is compiled with packed-fp32 instructions turned off
(-Xclang -target-feature -Xclang -packed-fp32-ops); hipcc's host pass warns
that it does not know that feature, which is harmless.
"""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libpkv.so")
ARCH = os.environ.get("PKV_OFFLOAD_ARCH", "gfx950")

SOURCES = ["pkv_decode.hip", "pkv_append.hip", "pkv_tier.hip", "pkv_fp8.hip", "pkv_prefill.hip", "pkv_noalloc.hip",
           "pkv_probe.hip", "pkv_host.cpp"]
HIP_FLAGS = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
             "-Wall", "-Wno-unused-function", f"-I{os.path.join(ROOT, 'include')}"]


def _run(cmd):
    print(" ".join(cmd), flush=True)
    subprocess.check_call(cmd)


def build(verbose: bool = True) -> str:
    objdir = os.path.join(ROOT, "_build")
    os.makedirs(objdir, exist_ok=True)
    objs = []
    for src in SOURCES:
        path = os.path.join(CSRC, src)
        obj = os.path.join(objdir, src + ".o")
        if src.endswith(".hip"):
            _run(["hipcc", *HIP_FLAGS, "-x", "hip", "-c", path, "-o", obj])
        else:   # host-only C++ against the HIP runtime API
            _run(["hipcc", "-O2", "-std=c++17", "-fPIC", "-Wall", "-x", "c++", "-D__HIP_PLATFORM_AMD__",
                  "-I/opt/rocm/include",
                  f"-I{os.path.join(ROOT, 'include')}", "-c", path, "-o", obj])
        objs.append(obj)
    tmp = LIB + ".tmp"
    _run(["hipcc", f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp])
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    build()
    sys.exit(0)
