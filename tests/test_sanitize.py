"""The host-side C++ under AddressSanitizer and UndefinedBehaviorSanitizer.

The CPU oracle (oracle/hisparse_oracle.cpp) and the residency policy
(serving_memory_tier_amd/csrc/policy.cpp) are compiled with g++ together with
a small native driver (tests/native/sanitize_driver.cpp) that runs the
hand-worked resolve example and random tiny cases of every oracle function
(tables pointing outside the pools, every entry kind, the largest stamp) and
policy runs under pressure.  Any out-of-bounds access, use after free, leak
or undefined operation ends the run with a sanitizer report.  CPU only.
"""

from __future__ import annotations

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.skipif(shutil.which("g++") is None, reason="needs g++")
def test_oracle_and_policy_sanitized(tmp_path):
    exe = str(tmp_path / "sanitize_driver")
    cmd = ["g++", "-std=c++17", "-O1", "-g", "-fsanitize=address,undefined",
           "-fno-sanitize-recover=all", "-fno-omit-frame-pointer",
           "-I", os.path.join(ROOT, "include"),
           os.path.join(ROOT, "tests", "native", "sanitize_driver.cpp"),
           os.path.join(ROOT, "oracle", "hisparse_oracle.cpp"),
           os.path.join(ROOT, "serving_memory_tier_amd", "csrc", "policy.cpp"), "-o", exe]
    res = subprocess.run(cmd, capture_output=True, text=True)
    assert res.returncode == 0, res.stdout + res.stderr
    # the environment is passed on as it is; a preloaded library ahead of the
    # sanitizer runtime is allowed (verify_asan_link_order=0)
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:verify_asan_link_order=0",
               UBSAN_OPTIONS="print_stacktrace=1")
    run = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=300)
    assert run.returncode == 0, run.stdout + run.stderr
    assert "runtime error" not in run.stderr and "ERROR: AddressSanitizer" not in run.stderr
    assert "clean" in run.stdout
