"""The host code of the C ABI (opr_api.cpp: argument validation, workspace
carving, the no-allocation scratch lookup; kpass_plan.cpp: the K-pass
planner) built with AddressSanitizer and UndefinedBehaviorSanitizer, and run
through tests/sanitize/abi_checks.cpp: every entry point's validation paths
with fake device pointers (no HIP call is reached: the attention launchers and
the GEMM are stand-ins that abort if called, tests/sanitize/stubs.cpp) and the
planner on random and limit-sized conversations.  The sanitizers act on host
code only (-Xarch_host); device code is built as usual."""
import concurrent.futures as cf
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "block_sparse_masked_opr_amd", "csrc")
HERE = os.path.join(ROOT, "tests", "sanitize")
OUT = os.path.join(ROOT, "_build", "sanitize")
SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
       "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer"]
BASE = ["-O1", "-g", "-std=c++17", "-fPIC", "--offload-arch=gfx950",
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", "-Wno-unused-result",
        "-I", os.path.join(ROOT, "include"), "-I", CSRC]


def _hipcc():
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    return None


def _compile(args):
    src, sanitize = args
    obj = os.path.join(OUT, os.path.basename(src) + ".o")
    cmd = [_hipcc(), *BASE, *(SAN if sanitize else []), "-x", "hip", "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, f"{' '.join(cmd)}\n{r.stderr[-3000:]}"
    return obj


def test_abi_host_code_under_asan_and_ubsan():
    if _hipcc() is None:
        pytest.skip("hipcc not available")
    os.makedirs(OUT, exist_ok=True)
    jobs = [(os.path.join(CSRC, "opr_api.cpp"), True), (os.path.join(CSRC, "kpass_plan.cpp"), True),
            (os.path.join(HERE, "abi_checks.cpp"), True), (os.path.join(HERE, "stubs.cpp"), True),
            # size functions and their own launchers, built as usual
            (os.path.join(CSRC, "layout.hip"), False), (os.path.join(CSRC, "token_ce.hip"), False),
            (os.path.join(CSRC, "block.hip"), False)]
    with cf.ThreadPoolExecutor(max_workers=len(jobs)) as ex:
        objs = list(ex.map(_compile, jobs))
    exe = os.path.join(OUT, "abi_checks")
    cmd = [_hipcc(), "--offload-arch=gfx950", *SAN, "-o", exe, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, f"{' '.join(cmd)}\n{r.stderr[-3000:]}"
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=600)
    print(r.stdout, r.stderr[-3000:])
    assert r.returncode == 0, r.stderr[-3000:]
    assert "checks passed" in r.stdout
