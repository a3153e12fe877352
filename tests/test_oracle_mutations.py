"""The pins are strong enough: each plausible mistake planted in a copy of the
oracle (on the CPU, never in the product) makes at least one pin fail.

Each mutant is compiled from the oracle source with one edit, and the fast
pins of test_oracle.py run against it in a subprocess (HS_ORACLE_LIB); the
mutant must make that run fail.
"""

from __future__ import annotations

import os
import subprocess
import sys
import tempfile

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "hisparse_oracle.cpp")

MUTANTS = {
    "victims_most_recent_first": ("if (stp[a] != stp[b]) return stp[a] < stp[b];",
                                  "if (stp[a] != stp[b]) return stp[a] > stp[b];"),
    "victim_tie_break_reversed": ("    return a < b;\n  });", "    return a > b;\n  });"),
    "hits_not_refreshed": ("if (ukind[k] == U_HIT) stp[uslot[k]] = stamp;",
                           "if (ukind[k] == U_HIT) (void)stamp;"),
    "misses_assigned_descending": ("const int32_t u = misses[j];",
                                   "const int32_t u = misses[M - 1 - j];"),
    "wrong_host_row_offset": ("const int64_t src_row = (int64_t)hbt[u / page] * page + u % page;",
                              "const int64_t src_row = (int64_t)hbt[u / page] * page + (u + 1) % page;"),
    "resident_row_drops_offset": ("rows[i] = b * page + t % page;", "rows[i] = b * page;"),
    "ctx_bound_off_by_one": ("t >= ctx || t / page >= max_pages", "t > ctx || t / page >= max_pages"),
    "missing_host_copy_ignored": ("if (hb < 0 || hb >= host_blocks) {\n        ukind[k] = U_INVALID;",
                                  "if (false) {\n        ukind[k] = U_INVALID;"),
    "hit_slot_not_excluded": ("if (!is_hit_slot[q] && slot_ok(q)) V.push_back(q);",
                              "if (slot_ok(q)) V.push_back(q);"),
    "new_token_not_recorded": ("    tok[q] = u;\n", "    (void)u;\n"),
    "gather_before_copies": ("  // Step 8: the gather reads the pool after every copy of the call.\n  if (gather_out) gather_rows(lay, R, L, N, pool, rows, gather_out);",
                             "  if (gather_out) std::memset(gather_out, 0, (size_t)R * L * N * lay.row_bytes);"),
    "offload_skips_last_layer": ("for (int32_t l = 0; l < L; ++l)\n      std::memcpy(host",
                                 "for (int32_t l = 0; l + 1 < L; ++l)\n      std::memcpy(host"),
    "dup_count_wrong": ("stats[6] = n_nonpad - (int32_t)nonpad.size();", "stats[6] = 0;"),
    "grouped_copies_skip_last_layer": ("for (int32_t l = l0 + 1; l < l0 + G; ++l)",
                                       "for (int32_t l = l0 + 1; l < l0 + G - 1; ++l)"),
    "page_touch_ctx_off_by_one": ("if (t < 0 || t >= ctx_len[r]) continue;",
                                  "if (t < 0 || t > ctx_len[r]) continue;"),
    "page_touch_wrong_page": ("const int64_t pg = t / page;", "const int64_t pg = (t + 1) / page;"),
    "grouped_gather_wrong_group": ("const int64_t row = rows[((int64_t)r * NG + l / G) * N + i];",
                                   "const int64_t row = rows[((int64_t)r * NG + l % NG) * N + i];"),
}

FAST_PINS = ["tests/test_oracle.py::test_worked_example_steps",
             "tests/test_oracle.py::test_worked_example_plan_overflow_invalid",
             "tests/test_oracle.py::test_single_token_lists_are_textbook_lru",
             "tests/test_oracle.py::test_victims_are_the_unique_declarative_solution",
             "tests/test_oracle.py::test_matches_sequential_restatement",
             "tests/test_oracle.py::test_empty_buffer_fills_slots_in_token_order",
             "tests/test_oracle.py::test_offload_copies_every_layer_and_leaves_pool",
             "tests/test_oracle.py::test_tiny_workload_invariants",
             "tests/test_oracle.py::test_grouped_equals_per_layer_resolve",
             "tests/test_oracle.py::test_grouped_rows_hold_each_layers_content",
             "tests/test_oracle.py::test_page_touch_worked_example",
             "tests/test_oracle.py::test_page_touch_is_the_set_of_selected_pages"]


def test_unmutated_source_passes_the_pins():
    with tempfile.TemporaryDirectory() as d:
        lib = os.path.join(d, "liboracle_ok.so")
        subprocess.run(["g++", "-O1", "-std=c++17", "-shared", "-fPIC", "-o", lib, SRC], check=True)
        env = dict(os.environ, HS_ORACLE_LIB=lib)
        r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider"]
                           + FAST_PINS, cwd=ROOT, env=env, capture_output=True, text=True)
        assert r.returncode == 0, r.stdout[-2000:]


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_mutant(name):
    old, new = MUTANTS[name]
    src = open(SRC).read()
    assert src.count(old) == 1, f"mutation anchor for {name} not found exactly once"
    with tempfile.TemporaryDirectory() as d:
        path = os.path.join(d, "mutant.cpp")
        open(path, "w").write(src.replace(old, new))
        lib = os.path.join(d, "libmutant.so")
        subprocess.run(["g++", "-O1", "-std=c++17", "-shared", "-fPIC", "-w", "-o", lib, path],
                       check=True)
        env = dict(os.environ, HS_ORACLE_LIB=lib)
        r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider"]
                           + FAST_PINS, cwd=ROOT, env=env, capture_output=True, text=True,
                           timeout=600)
        assert r.returncode != 0, f"mutant {name} survived every pin"
