"""Host checks of the build and of the binding's struct mirrors (no GPU).

- The ctypes mirrors of hs_layout and hs_batch have the sizes and field
  offsets a C compiler gives the header's structs, and the binding's limits
  are the header's.
- The build's scratch-memory guard reads hipcc's resource remarks: a kernel
  reporting scratch per lane is named, one without is not.
"""

from __future__ import annotations

import ctypes
import os
import subprocess
import tempfile

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

pytestmark = pytest.mark.filterwarnings("ignore")


def _c_layout():
    src = r"""
#include <stddef.h>
#include <stdio.h>
#include "hisparse.h"
int main(void) {
  printf("%zu %zu\n", sizeof(hs_layout), sizeof(hs_batch));
  printf("%zu %zu %zu %zu %zu\n", offsetof(hs_batch, slot_token), offsetof(hs_batch, slot_stamp),
         offsetof(hs_batch, fill_sync), offsetof(hs_batch, fill_sync_words),
         offsetof(hs_layout, host_layer_stride));
  printf("%d %d %d %d\n", HS_FILL_SYNC_WORDS, HS_MAX_ENTRIES, HS_MAX_HOT_CAPACITY, HS_MAX_ROW_BYTES);
  return 0;
}
"""
    with tempfile.TemporaryDirectory() as d:
        c = os.path.join(d, "layout.c")
        exe = os.path.join(d, "layout")
        with open(c, "w") as f:
            f.write(src)
        subprocess.run(["gcc", "-D__HIP_PLATFORM_AMD__", "-I", os.path.join(ROOT, "include"),
                        "-I", "/opt/rocm/include", c, "-o", exe], check=True,
                       capture_output=True)
        out = subprocess.run([exe], check=True, capture_output=True, text=True).stdout.split()
    return [int(x) for x in out]


def test_struct_mirrors_match_header():
    from serving_memory_tier_amd import _lib

    HsBatch, HsLayout = _lib.HsBatch, _lib.HsLayout
    lay, bat, o_tok, o_stp, o_sync, o_words, o_hls, words, n_max, c_max, row_max = _c_layout()
    assert ctypes.sizeof(HsLayout) == lay
    assert ctypes.sizeof(HsBatch) == bat
    assert HsBatch.slot_token.offset == o_tok
    assert HsBatch.slot_stamp.offset == o_stp
    assert HsBatch.fill_sync.offset == o_sync
    assert HsBatch.fill_sync_words.offset == o_words
    assert HsLayout.host_layer_stride.offset == o_hls
    assert _lib.HS_FILL_SYNC_WORDS == words
    assert (_lib.HS_MAX_ENTRIES, _lib.HS_MAX_HOT_CAPACITY, _lib.HS_MAX_ROW_BYTES) == (
        n_max, c_max, row_max)


def test_batch_of_leaves_fill_sync_null_by_default():
    from serving_memory_tier_amd.api import batch_of

    b = batch_of(2, 4, None, None, None, None, None, None, None, None)
    assert b.fill_sync is None and b.fill_sync_words == 0
    b2 = batch_of(2, 4, None, None, None, None, None, None, None, None, fill_sync=0x1000,
                  fill_sync_words=64)
    assert b2.fill_sync == 0x1000 and b2.fill_sync_words == 64


def test_scratch_guard_reads_resource_remarks():
    from serving_memory_tier_amd.build import _scratch_users

    msgs = [
        "a.hip:1:1: remark: Function Name: kern_a [-Rpass-analysis=kernel-resource-usage]",
        "a.hip:1:1: remark:     VGPRs: 78 [-Rpass-analysis=kernel-resource-usage]",
        "a.hip:1:1: remark:     ScratchSize [bytes/lane]: 0 [-Rpass-analysis=kernel-resource-usage]",
        "a.hip:9:1: remark: Function Name: kern_b [-Rpass-analysis=kernel-resource-usage]",
        "a.hip:9:1: remark:     ScratchSize [bytes/lane]: 80 [-Rpass-analysis=kernel-resource-usage]",
    ]
    assert _scratch_users(msgs) == ["kern_b: 80 bytes/lane"]
    assert _scratch_users(msgs[:3]) == []
