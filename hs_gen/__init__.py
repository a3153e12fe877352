"""Seeded synthetic inputs shared by the CPU oracle and the GPU path.

Holds random numbers, row content and workload construction only; nothing in
this package resolves, gathers or copies KV rows.
"""

from .content import PAGE, ROW_BYTES, content_np, content_torch, fill_rows
from .workloads import (CONFIGS, Spec, Step, Workload, build, build_dynamic, grouped_decode,
                        mixed_decode,
                        mixed_state, mtp_state, multi_layer, no_residency, tiny, ungrouped)

__all__ = ["PAGE", "ROW_BYTES", "content_np", "content_torch", "fill_rows", "CONFIGS", "Spec",
           "Step", "Workload", "build", "tiny", "mixed_decode", "multi_layer", "no_residency",
           "mixed_state", "mtp_state", "grouped_decode", "ungrouped", "build_dynamic"]
