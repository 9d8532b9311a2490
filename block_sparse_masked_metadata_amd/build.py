"""Compile libbsm.so in-tree for gfx950.

Host planner (C++17) with g++; HIP sources with hipcc --offload-arch=gfx950.
All HIP code is built with packed fp32 instructions disabled.
Run:  python -m block_sparse_masked_metadata_amd.build
"""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
OUT_DIR = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libbsm.so")
PROBE_LIB = os.path.join(HERE, "libbsm_probe.so")  # MFMA rate / clock probe for bench.py
ARCH = os.environ.get("BSM_ARCH", "gfx950")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
HIP_FLAGS = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
             "-I", INCLUDE, "-I", CSRC]
HOST_FLAGS = ["-O3", "-std=c++17", "-fPIC", "-pthread", "-Wall", "-I", INCLUDE, "-I", CSRC]

HIP_SOURCES = ["fwd.hip", "bwd.hip", "capi.hip"]
HOST_SOURCES = ["planner.cpp", "calls.cpp"]


def _run(cmds):
    procs = [(c, subprocess.Popen(c, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True))
             for c in cmds]
    ok = True
    for c, p in procs:
        out, _ = p.communicate()
        lines = [ln for ln in out.splitlines()
                 if "packed-fp32-ops" not in ln and ln.strip()]
        if p.returncode != 0:
            ok = False
            sys.stderr.write("FAILED: " + " ".join(c) + "\n" + out + "\n")
        elif lines and os.environ.get("BSM_BUILD_VERBOSE"):
            sys.stderr.write("\n".join(lines) + "\n")
    return ok


def build(verbose: bool = False) -> str:
    os.makedirs(OUT_DIR, exist_ok=True)
    objs = []
    cmds = []
    for s in HOST_SOURCES:
        o = os.path.join(OUT_DIR, s + ".o")
        objs.append(o)
        cmds.append(["g++", *HOST_FLAGS, "-c", os.path.join(CSRC, s), "-o", o])
    for s in HIP_SOURCES:
        o = os.path.join(OUT_DIR, s + ".o")
        objs.append(o)
        cmds.append([HIPCC, *HIP_FLAGS, "-c", os.path.join(CSRC, s), "-o", o])
    if not _run(cmds):
        raise RuntimeError("libbsm compile failed")
    tmp = LIB + ".tmp"
    if not _run([[HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-pthread", *objs, "-o", tmp]]):
        raise RuntimeError("libbsm link failed")
    os.replace(tmp, LIB)
    tmp = PROBE_LIB + ".tmp"
    if not _run([[HIPCC, *HIP_FLAGS, "-shared", os.path.join(CSRC, "probe.hip"), "-o", tmp]]):
        raise RuntimeError("libbsm_probe build failed")
    os.replace(tmp, PROBE_LIB)
    if verbose:
        print("built", LIB, "and", os.path.basename(PROBE_LIB))
    return LIB


if __name__ == "__main__":
    build(verbose=True)
