"""Build libtreewy.so (HIP kernels + C ABI) for gfx950 with hipcc, in-tree.

Every HIP source is compiled with packed fp32 instructions disabled
(``-Xclang -target-feature -Xclang -packed-fp32-ops``); the host pass warns that
it does not know the feature, which is harmless.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG_DIR)
CSRC = os.path.join(PKG_DIR, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD_DIR = os.path.join(ROOT, "_build")
LIB_PATH = os.path.join(PKG_DIR, "libtreewy.so")
ARCH = "gfx950"

HIP_SOURCES = ["verify.hip", "verify_fused.hip", "verify_pool.hip", "verify_pool_trees.hip",
               "verify_s16.hip", "verify_s16_pool.hip", "verify_s16_pool_trees.hip", "commit.hip",
               "store_all.hip", "prefill.hip", "scratch.hip"]
HOST_SOURCES = ["api.cpp", "tree_meta.cpp"]
COMMON = ["-O3", "-std=c++17", "-fPIC", "-Wall", "-I", INCLUDE, "-I", CSRC]
NO_PK_FP32 = ["-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


def _hipcc() -> str:
    env = os.environ.get("HIPCC")
    if env:
        return env
    found = shutil.which("hipcc")
    return found or "/opt/rocm/bin/hipcc"


def _run(cmd):
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(l for l in r.stdout.splitlines() if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"command failed ({r.returncode}): {' '.join(cmd)}\n{out}")
    return out


def build(verbose: bool = False, jobs: int = 8) -> str:
    """Compile every source and link the shared library; returns its path."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    hipcc = _hipcc()
    cmds, objs = [], []
    for src in HIP_SOURCES:
        obj = os.path.join(BUILD_DIR, src + ".o")
        cmds.append([hipcc, "-x", "hip", f"--offload-arch={ARCH}", *COMMON, *NO_PK_FP32,
                     "-c", os.path.join(CSRC, src), "-o", obj])
        objs.append(obj)
    for src in HOST_SOURCES:
        obj = os.path.join(BUILD_DIR, src + ".o")
        cmds.append([hipcc, *COMMON, "-c", os.path.join(CSRC, src), "-o", obj])
        objs.append(obj)
    with cf.ThreadPoolExecutor(max_workers=jobs) as ex:
        for out in ex.map(_run, cmds):
            if verbose and out.strip():
                print(out)
    tmp = LIB_PATH + ".tmp"
    _run([hipcc, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp])
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
