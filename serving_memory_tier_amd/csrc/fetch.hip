// The early fill as a kernel of its own (the staged entry point
// hs_resolve_fetch), and the launch shapes shared with the fused resolve
// kernel.  The device code is in fill.h; see there for the method and the
// bound.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <atomic>

#include "fill.h"
#include "hs_internal.h"

namespace hs {
namespace {

__global__ void __launch_bounds__(kFillThreads) fetch_kernel(FetchParams p) {
  extern __shared__ __align__(16) int32_t lds[];
  fill::fill_block(p, lds, (int32_t)blockIdx.x);
}

}  // namespace

// Entries per gather workgroup: about `target` workgroups in all
// (kFetchGatherTarget when target <= 0), kFetchGatherMin..kFetchGatherEntries
// entries each (a multiple of 4).
int32_t gather_entries(int32_t entries, int64_t n_rl, int64_t target) {
  const bool strict = target > 0;  // at most `target` workgroups where possible
  if (target <= 0) target = kFetchGatherTarget;
  int64_t per = (entries * n_rl + target - 1) / target;
  if (per < kFetchGatherMin) per = kFetchGatherMin;
  per = (per + 3) / 4 * 4;
  while (strict && per < kFetchGatherEntries && per < entries &&
         n_rl * ((entries + per - 1) / per) > target)
    per += 4;
  if (per > kFetchGatherEntries) per = kFetchGatherEntries;
  if (per > entries) per = entries;
  return (int32_t)((per + 3) / 4 * 4);
}

size_t fetch_lds_words(int32_t entries, int32_t ge, int32_t* miss_tab_n, int32_t* gather_tab_n) {
  const int32_t ln = ((entries + 3) / 4) * 4;
  // miss workgroups: keys, src and list of N entries, the table, 4 counters;
  // the table takes 2N + 64 words where that fits, at least 1.5N + 1
  const int32_t avail = (int32_t)(kMaxLdsBytes / 4) - 3 * ln - 4;
  int32_t mt = ((2 * entries) / 64 + 1) * 64;
  if (mt > avail) mt = (avail / 64) * 64;
  const int32_t lo_bound = entries + entries / 2 + 1;
  if (mt < lo_bound) mt = lo_bound;
  // gather workgroups: keys and src of their range, a table 4x its size, a flag
  const int32_t gt = ((4 * ge) / 64 + 1) * 64;
  if (miss_tab_n) *miss_tab_n = mt;
  if (gather_tab_n) *gather_tab_n = gt;
  const size_t miss_words = 3 * (size_t)ln + mt + 4;
  const size_t gather_words = 2 * (size_t)ge + gt + 4;
  return miss_words > gather_words ? miss_words : gather_words;
}

size_t fetch_lds_bytes(int32_t entries, int32_t hot_capacity) {
  (void)hot_capacity;
  // the largest gather range any launch uses
  const int32_t ge = entries < kFetchGatherEntries ? (entries + 3) / 4 * 4 : kFetchGatherEntries;
  return 4 * fetch_lds_words(entries, ge, nullptr, nullptr);
}

int64_t prepare_fetch(FetchParams& p, size_t* lds_bytes, int64_t gather_target) {
  const int64_t n_rl = (int64_t)p.num_reqs * p.num_layers;
  p.lds_n = ((p.entries + 3) / 4) * 4;
  p.gather_e = gather_entries(p.entries, n_rl, gather_target);
  size_t words = fetch_lds_words(p.entries, p.gather_e, &p.miss_tab_n, &p.gather_tab_n);
  // the miss workgroups' bitmap of the tokens the usable slots hold (one bit
  // per token of the block table's span), where the slots all come with the
  // workgroup's first loads and the bitmap fits beside the rest of its LDS
  p.slot_bits_words = 0;
  if (p.hot_capacity <= kFillThreads * fill::kScanUnroll) {
    const int64_t nb = (((int64_t)p.max_pages << p.page_shift) + 31) / 32;
    const int64_t need = 3 * (int64_t)p.lds_n + p.miss_tab_n + 4 + nb;
    if (nb > 0 && need <= (int64_t)(kMaxLdsBytes / 4)) {
      p.slot_bits_words = (int32_t)nb;
      if ((size_t)need > words) words = (size_t)need;
    }
  }
  *lds_bytes = 4 * words;
  const uint32_t pieces = (uint32_t)(p.row_bytes >> 4);
  // ceil(2^32 / pieces); 0 for one piece a row, where it would be 2^32
  p.piece_magic = pieces > 1 ? (uint32_t)(((1ull << 32) + pieces - 1) / pieces) : 0u;
  // miss workgroups: kFetchHostGroups in all (the host reads in flight that
  // saturate the link), split by token when there are few request-layers
  int64_t S = (kFetchHostGroups + n_rl - 1) / n_rl;
  S = S < 1 ? 1 : S > kFetchMaxSplits ? kFetchMaxSplits : S;
  p.miss_splits = (int32_t)S;
  const int64_t pairs = n_rl * S;
  p.miss_groups = (int32_t)(pairs < kFetchHostGroups ? pairs : kFetchHostGroups);
  // gather workgroups: gather_e entries each
  p.gather_splits = p.misses_only ? 0 : (p.entries + p.gather_e - 1) / p.gather_e;
  return p.miss_groups + n_rl * p.gather_splits;
}

hipError_t launch_fetch(FetchParams p, hipStream_t stream) {
  const int64_t n_rl = (int64_t)p.num_reqs * p.num_layers;
  if (n_rl == 0 || p.entries == 0) return hipSuccess;
  size_t lds = 0;
  int64_t grid = prepare_fetch(p, &lds, 0);
  if (grid > INT32_MAX || lds > kMaxLdsBytes) return hipErrorInvalidValue;
  static std::atomic<uint64_t> raised{0};
  hipError_t err = allow_full_lds(reinterpret_cast<const void*>(fetch_kernel), raised);
  if (err != hipSuccess) return err;
  // as many gather workgroups as fit beside the miss workgroups in one round
  // of the chip, so that no gather range waits for a free CU
  int64_t resident = 0;
  err = resident_groups(reinterpret_cast<const void*>(fetch_kernel), kFillThreads, lds, &resident);
  if (err != hipSuccess) return err;
  const int64_t target = resident - p.miss_groups;
  if (!p.misses_only && target >= kFetchGatherMinGroups) {
    grid = prepare_fetch(p, &lds, target);
    if (grid > INT32_MAX || lds > kMaxLdsBytes) return hipErrorInvalidValue;
  }
  return launch_kernel(fetch_kernel, dim3((uint32_t)grid), dim3(kFillThreads), lds, stream, p);
}

}  // namespace hs
