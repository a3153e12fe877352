"""Host-side checks of the benchmark's bookkeeping (no GPU): the kernel source
hash that ties measured traffic to the sources it was taken on, the committed
counter summary being current, the CPU baseline's passes, and the one-GPU
guard."""

from __future__ import annotations

import os
import shutil
import subprocess
import sys

import bench
import hs_gen

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _hash_of(tmp_root):
    old = bench.ROOT
    try:
        bench.ROOT = str(tmp_root)
        return bench.kernel_source_hash()
    finally:
        bench.ROOT = old


def test_source_hash_ignores_comments_not_code(tmp_path):
    src = os.path.join(ROOT, "serving_memory_tier_amd", "csrc")
    dst = tmp_path / "serving_memory_tier_amd" / "csrc"
    shutil.copytree(src, dst)
    h0 = _hash_of(tmp_path)
    assert h0 == bench.kernel_source_hash()
    f = dst / "copy.hip"
    text = f.read_text()
    f.write_text("// a note\n" + text.replace("\n", "\n  \n", 3) + "\n/* another\n note */\n")
    assert _hash_of(tmp_path) == h0
    f.write_text(text.replace("kCommitEPW = 16", "kCommitEPW = 32"))
    assert _hash_of(tmp_path) != h0


def test_committed_counters_match_the_sources():
    # the headline's HBM traffic comes from profiles/counters_mixed_decode.md,
    # valid only while the kernel sources hash to the value recorded there
    v = bench.measured_traffic("resolve_fill", "mixed_decode")
    assert v is not None and v > 80_000_000
    assert bench.measured_traffic("resolve_fill", "no_such_workload") is None


def test_cpu_baseline_runs_passes_until_its_budget():
    wl = hs_gen.tiny(steps=3)
    done, passes, spent = bench._oracle_run(wl, 0.05, 1)
    assert spent >= 0.05 and done >= len(wl.steps) * (passes - 1) + 1
    assert passes >= 1


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120, cwd=ROOT)
    assert r.returncode == 2
    assert "one GPU" in (r.stdout + r.stderr)
