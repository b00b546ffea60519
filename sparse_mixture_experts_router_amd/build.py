"""Build libmoe.so (HIP kernels + C ABI) for gfx950 with hipcc, in-tree.

Usage: ``python -m sparse_mixture_experts_router_amd.build`` or ``build()``.
Every call recompiles all sources; objects go to ``_build/`` next to this file
and the library to ``libmoe.so`` beside it.
"""

from __future__ import annotations

import concurrent.futures
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(os.path.dirname(HERE), "include")
OBJ_DIR = os.path.join(HERE, "_build")
LIB_PATH = os.path.join(HERE, "libmoe.so")

SOURCES = ["route.hip", "permute.hip", "grouped_gemm.hip", "expert_gemm.hip", "combine.hip",
           "backward.hip", "moe_api.hip"]

ARCH = "gfx950"
FLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-Wall",
    "-Wno-unused-function",
    # packed fp32 VALU forms stay off: hipcc must not emit them from float code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    f"-I{INCLUDE}",
    f"-I{CSRC}",
]


def _hipcc() -> str:
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    path = os.path.join(rocm, "bin", "hipcc")
    return path if os.path.exists(path) else (shutil.which("hipcc") or "hipcc")


def _run(cmd):
    res = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    # the host pass does not know the packed-fp32 feature and says so; drop that line
    out = "\n".join(l for l in res.stdout.splitlines()
                    if "packed-fp32-ops' is not a recognized feature" not in l)
    return res.returncode, out


def build(verbose: bool = False, jobs: int = 8) -> str:
    """Compile every source and link libmoe.so; returns the library path."""
    os.makedirs(OBJ_DIR, exist_ok=True)
    hipcc = _hipcc()
    cmds = []
    for src in SOURCES:
        obj = os.path.join(OBJ_DIR, os.path.splitext(src)[0] + ".o")
        cmds.append([hipcc, *FLAGS, "-c", os.path.join(CSRC, src), "-o", obj])
    with concurrent.futures.ThreadPoolExecutor(max_workers=max(1, min(jobs, len(cmds)))) as ex:
        results = list(ex.map(_run, cmds))
    for cmd, (rc, out) in zip(cmds, results):
        if out.strip() and (verbose or rc != 0):
            print(out, file=sys.stderr)
        if rc != 0:
            raise RuntimeError(f"hipcc failed for {cmd[-3]}")
    objs = [c[-1] for c in cmds]
    tmp = LIB_PATH + ".tmp"
    rc, out = _run([hipcc, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs])
    if rc != 0:
        print(out, file=sys.stderr)
        raise RuntimeError("link of libmoe.so failed")
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
