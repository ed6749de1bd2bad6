"""Builds the lane library libws.so in-tree with hipcc for gfx950.

    python -m post_processing_amd.build

Also builds the host-only test driver of the planning code (g++, no HIP)
when asked to (see tests/test_host_logic.py).
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libws.so")
SOURCES = ["ws_preprocess.hip", "ws_topk.hip", "ws_detect.hip", "ws_runtime.hip",
           "ws_noalloc.hip"]
ARCH = "gfx950"


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build the lane library)")


LIB_MARKS = os.path.join(PKG, "libws_marks.so")


def lib_command(out: str, marks: bool = False) -> list[str]:
    return [
        hipcc(), *(["-DWS_CLOCK_MARKS"] if marks else []), f"--offload-arch={ARCH}", "-O3",
        "-std=c++17", "-fPIC", "-shared",
        "-Wall", "-Wno-unused-command-line-argument",
        # keep the compiler from forming packed FP32 instructions
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        # IEEE binary32 division and square root (detection decisions rely on it)
        "-fhip-fp32-correctly-rounded-divide-sqrt",
        # leading scalar and pointer kernel arguments arrive in scalar
        # registers at wave launch (gfx950 kernarg preloading)
        "-mllvm", "-amdgpu-kernarg-preload-count=16",
        "-I", INCLUDE, "-I", CSRC,
        "-o", out,
    ] + [os.path.join(CSRC, s) for s in SOURCES]


def build_lib(verbose: bool = False, marks: bool = False) -> str:
    """Build libws.so, or with `marks` the clock-mark instrumented
    libws_marks.so (phase timing only; never loaded by default)."""
    lib = LIB_MARKS if marks else LIB
    tmp = lib + ".tmp"
    cmd = lib_command(tmp, marks)
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError(f"hipcc failed with exit code {res.returncode}")
    os.replace(tmp, lib)
    return lib


def build_host_test(out: str, sanitize: bool = False) -> str:
    """g++ build of the planning code's host-only test driver (no HIP);
    with `sanitize`, instrumented by AddressSanitizer and
    UndefinedBehaviorSanitizer, any report aborting the run."""
    src = os.path.join(ROOT, "tests", "host", "ws_plan_test.cpp")
    cmd = ["g++", "-std=c++17", "-O1", "-Wall", "-Werror", "-I", INCLUDE, "-I", CSRC]
    if sanitize:
        cmd += ["-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
                "-fno-sanitize-recover=all"]
    cmd += ["-o", out, src]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError("g++ failed:\n" + res.stdout + res.stderr)
    return out


if __name__ == "__main__":
    print(build_lib(verbose=True, marks="--marks" in sys.argv[1:]))
