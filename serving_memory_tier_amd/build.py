"""Builds ``libhisparse.so`` in-tree for gfx950 (MI355X) with hipcc."""

from __future__ import annotations

import os
import re
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
SOURCES = ["resolve.hip", "copy.hip", "fetch.hip", "touch.hip", "attend.hip", "api.hip"]
ARCH = "gfx950"

# Packed-FP32 instructions are switched off for all HIP code (hipcc's host pass
# warns that it does not know the feature; that warning is harmless).  The
# fused resolve-and-fill kernels exceed the AMDGPU inliner's default limit on
# a caller's basic blocks; a device function left out of line there costs a
# call frame in scratch memory for every lane, so the limit is raised.
FLAGS = ["-O3", "-std=c++17", "-fPIC", "-shared", f"--offload-arch={ARCH}",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-mllvm", "-amdgpu-inline-max-bb=2000",
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


PROBE_SRC = "probe.hip"
PROBE_LIB = os.path.join(HERE, "libhs_probe.so")


def _hipcc(args, what):
    res = subprocess.run(["hipcc"] + args, capture_output=True, text=True)
    noise = "packed-fp32-ops' is not a recognized feature"
    msgs = [ln for ln in (res.stdout + res.stderr).splitlines() if noise not in ln]
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({what}):\n" + "\n".join(msgs))
    return msgs


def _scratch_users(msgs):
    """Kernels whose resource remarks report scratch memory per lane (a
    spill or an out-of-line call): none may, as every kernel here is tuned
    to keep its working set in registers and LDS."""
    users, name = [], None
    for ln in msgs:
        m = re.search(r"Function Name: (\S+)", ln)
        if m:
            name = m.group(1)
        m = re.search(r"ScratchSize \[bytes/lane\]: (\d+)", ln)
        if m and int(m.group(1)) > 0:
            users.append(f"{name}: {m.group(1)} bytes/lane")
    return users


def build(verbose: bool = False) -> str:
    """Compiles every source to an object (in parallel), links the library,
    and builds the measurement library beside it."""
    import tempfile
    from concurrent.futures import ThreadPoolExecutor

    build_policy()
    out = os.path.join(HERE, "libhisparse.so")
    tmp = out + ".tmp"
    inc = ["-I", os.path.join(ROOT, "include")]
    compile_flags = [f for f in FLAGS if f != "-shared"] + ["-Rpass-analysis=kernel-resource-usage"]
    with tempfile.TemporaryDirectory(prefix="hs_build_") as objdir:
        def compile_one(src):
            obj = os.path.join(objdir, src.replace(".hip", ".o"))
            return _hipcc(compile_flags + inc + ["-c", os.path.join(HERE, "csrc", src), "-o", obj],
                          src), obj
        jobs = min(len(SOURCES) + 1, max(1, os.cpu_count() or 1))
        with ThreadPoolExecutor(jobs) as ex:
            results = list(ex.map(compile_one, SOURCES + [PROBE_SRC]))
        msgs = [m for r in results for m in r[0]]
        scratch = _scratch_users(msgs)
        if scratch:
            raise RuntimeError("kernels using scratch memory:\n" + "\n".join(scratch))
        msgs = [m for m in msgs if "kernel-resource-usage" not in m]
        objs = [r[1] for r in results]
        msgs += _hipcc(FLAGS + ["-o", tmp] + objs[:-1], "link")
        msgs += _hipcc(FLAGS + ["-o", PROBE_LIB + ".tmp", objs[-1]], "link probe")
    if verbose and msgs:
        print("\n".join(msgs))
    os.replace(tmp, out)
    os.replace(PROBE_LIB + ".tmp", PROBE_LIB)
    return out


if __name__ == "__main__":
    print(build(verbose=True))
