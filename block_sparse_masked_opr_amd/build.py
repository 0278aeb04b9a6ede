"""Build libopr.so (HIP kernels + C ABI) in-tree for gfx950 with hipcc.

    python -m block_sparse_masked_opr_amd.build        # or build() from Python

Objects go to <repo>/_build/, the library to block_sparse_masked_opr_amd/libopr.so.
build(debug=True) builds the checked library instead (-DOPR_DEBUG: the kernels
test the invariants their indexing relies on, read by opr_debug_errors):
objects in <repo>/_build_debug/, library libopr_debug.so.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libopr.so")
BUILD_DEBUG = os.path.join(ROOT, "_build_debug")
LIB_DEBUG = os.path.join(PKG, "libopr_debug.so")
ARCH = "gfx950"

SOURCES = ["opr_api.cpp", "layout.hip", "attn_prologue.hip", "attn_fwd.hip", "attn_bwd.hip", "attn_dq.hip",
           "token_ce.hip", "kpass_plan.cpp", "gemm.cpp", "block.hip"]

HIPCC_FLAGS = [
    "-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
    # no packed fp32 arithmetic (v_pk_* f32) in device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-result",
]


def _hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libopr)")


def _compile(src: str, extra, build_dir: str = BUILD) -> str:
    obj = os.path.join(build_dir, os.path.basename(src) + ".o")
    cmd = [_hipcc(), *HIPCC_FLAGS, *extra, "-I", INCLUDE, "-I", CSRC, "-c", os.path.join(CSRC, src), "-o", obj]
    if src.endswith(".cpp"):
        cmd[1:1] = ["-x", "hip"]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{res.stdout}\n{res.stderr}")
    return obj


def build(verbose: bool = False, extra_flags=(), debug: bool = False) -> str:
    """Compile every source and link libopr.so (libopr_debug.so with
    debug=True); returns the library path."""
    build_dir, lib = (BUILD_DEBUG, LIB_DEBUG) if debug else (BUILD, LIB)
    flags = list(extra_flags) + (["-DOPR_DEBUG"] if debug else [])
    os.makedirs(build_dir, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=min(8, len(SOURCES))) as ex:
        objs = list(ex.map(lambda s: _compile(s, flags, build_dir), SOURCES))
    tmp = lib + ".tmp"
    cmd = [_hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs,
           "-L/opt/rocm/lib", "-lhipblaslt", "-Wl,-rpath,/opt/rocm/lib", "-Wl,--no-undefined"]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{res.stdout}\n{res.stderr}")
    os.replace(tmp, lib)
    if verbose:
        print(f"built {lib}")
    return lib


if __name__ == "__main__":
    args = sys.argv[1:]
    build(verbose=True, extra_flags=[a for a in args if a != "--debug"], debug="--debug" in args)
