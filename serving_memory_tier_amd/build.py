"""Builds ``libhisparse.so`` in-tree for gfx950 (MI355X) with hipcc."""

from __future__ import annotations

import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
SOURCES = ["resolve.hip", "copy.hip", "fetch.hip", "touch.hip", "attend.hip", "api.hip"]
ARCH = "gfx950"

# Packed-FP32 instructions are switched off for all HIP code (hipcc's host pass
# warns that it does not know the feature; that warning is harmless).
FLAGS = ["-O3", "-std=c++17", "-fPIC", "-shared", f"--offload-arch={ARCH}",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-Wall", "-Wno-unused-function"]


POLICY_SRC = os.path.join(HERE, "csrc", "policy.cpp")
POLICY_LIB = os.path.join(HERE, "libhs_policy.so")


def build_policy() -> str:
    """The host-only residency policy library (no HIP), with g++."""
    tmp = POLICY_LIB + ".tmp"
    cmd = ["g++", "-O2", "-std=c++17", "-fPIC", "-shared", "-Wall", "-I",
           os.path.join(ROOT, "include"), "-o", tmp, POLICY_SRC]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError("g++ failed:\n" + res.stdout + res.stderr)
    os.replace(tmp, POLICY_LIB)
    return POLICY_LIB


def build(verbose: bool = False) -> str:
    build_policy()
    out = os.path.join(HERE, "libhisparse.so")
    tmp = out + ".tmp"
    cmd = (["hipcc"] + FLAGS + ["-I", os.path.join(ROOT, "include"), "-o", tmp] +
           [os.path.join(HERE, "csrc", s) for s in SOURCES])
    res = subprocess.run(cmd, capture_output=True, text=True)
    noise = "packed-fp32-ops' is not a recognized feature"
    msgs = [ln for ln in (res.stdout + res.stderr).splitlines() if noise not in ln]
    if res.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + "\n".join(msgs))
    if verbose and msgs:
        print("\n".join(msgs))
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build(verbose=True))
