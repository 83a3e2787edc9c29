"""Compile librskv.so (HIP for gfx950) in-tree.

Every translation unit is compiled with hipcc for gfx950 only, with packed
fp32 instructions disabled, and linked into ``routed_sparse_kv_amd/lib``.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIBDIR = os.path.join(HERE, "lib")
LIB = os.path.join(LIBDIR, "librskv.so")
SOURCES = ["segment.hip", "summary.hip", "factor.hip", "route.hip", "attend.hip", "retrieval.hip",
           "window.hip", "static_ws.hip", "api.cpp", "retrieval_api.cpp", "window_api.cpp"]
ARCH = "gfx950"


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def _flags():
    return ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            "-Wall", "-Wno-unused-result", "-I", os.path.join(HERE, "..", "include")]


# Per-source flags.  factor.hip: its kernels call non-inlined phase functions,
# so the compiler cannot rule out accumulation registers being needed and
# picks the accumulation-register form of the fp64 MFMA, copying the Gram
# tiles' accumulators there and back around every K step; the vector-register
# form keeps them in place.
EXTRA_FLAGS = {"factor.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form=1"]}


def build(verbose: bool = False, jobs: int = 8) -> str:
    """Compile every source and link the shared library; return its path."""
    objdir = os.path.join(LIBDIR, "obj")
    os.makedirs(objdir, exist_ok=True)
    cc = hipcc()

    def compile_one(src):
        obj = os.path.join(objdir, os.path.splitext(src)[0] + ".o")
        lang = ["-x", "hip"] if src.endswith(".hip") else []
        cmd = [cc, *_flags(), *EXTRA_FLAGS.get(src, []), *lang, "-c", os.path.join(CSRC, src), "-o", obj]
        r = subprocess.run(cmd, capture_output=True, text=True)
        if verbose or r.returncode != 0:
            sys.stderr.write(" ".join(cmd) + "\n" + r.stdout + _filter(r.stderr))
        if r.returncode != 0:
            raise RuntimeError(f"hipcc failed on {src}")
        return obj

    with ThreadPoolExecutor(max(1, jobs)) as ex:
        objs = list(ex.map(compile_one, SOURCES))
    tmp = LIB + ".tmp"
    cmd = [cc, "-shared", "-fPIC", f"--offload-arch={ARCH}", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(" ".join(cmd) + "\n" + r.stdout + r.stderr)
        raise RuntimeError("link of librskv.so failed")
    os.replace(tmp, LIB)
    return LIB


def _filter(stderr: str) -> str:
    # hipcc's host pass does not know the device-only target feature.
    return "".join(line + "\n" for line in stderr.splitlines()
                   if "packed-fp32-ops" not in line)


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
