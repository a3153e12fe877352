// Page coldness for the residency policy: every valid top-K entry stamps its
// page in a per-request table ("vLLM GLM 5.3 ... Hybrid HiSparse offloading,
// Part 1", "Use sparsity when needed": under pressure a request gives up its
// coldest pages).  The lists already sit in device memory, so the policy
// reads one word per page instead of every entry.
//
// One workgroup covers kTouchPerBlock consecutive entries of one request's
// lists (grid: requests x chunks, at most 65535 chunks); each lane loads kTouchUnroll entries, coalesced, before it stores.
// Entries of one page store the same value, so concurrent stores to a word
// agree and the result does not depend on their order.

#include <hip/hip_runtime.h>

#include "hs_internal.h"

namespace hs {

namespace {

constexpr int kTouchThreads = 256;
constexpr int kTouchUnroll = 4;
static_assert(kTouchThreads * kTouchUnroll == kTouchPerBlock, "entries per workgroup");

__global__ void __launch_bounds__(kTouchThreads) page_touch_kernel(TouchParams p) {
  const int32_t r = (int32_t)blockIdx.x;
  const int64_t base = (int64_t)blockIdx.y * kTouchPerBlock + threadIdx.x;
  const int32_t* lists = p.topk + (int64_t)r * p.entries;
  const int32_t ctx = p.ctx_len[r];
  // tokens past the table's columns have no page to stamp
  const int64_t limit = (int64_t)p.max_pages << p.page_shift;
  const int32_t hi = (int32_t)((int64_t)ctx < limit ? (int64_t)ctx : limit);
  uint32_t* row = p.page_use + (int64_t)r * p.max_pages;
  int32_t t[kTouchUnroll];
#pragma unroll
  for (int j = 0; j < kTouchUnroll; ++j) {
    const int64_t e = base + (int64_t)j * kTouchThreads;
    t[j] = e < p.entries ? lists[e] : -1;
  }
#pragma unroll
  for (int j = 0; j < kTouchUnroll; ++j)
    if (t[j] >= 0 && t[j] < hi) row[t[j] >> p.page_shift] = p.stamp;
}

}  // namespace

hipError_t launch_page_touch(const TouchParams& p, hipStream_t stream) {
  if (p.num_reqs == 0 || p.entries == 0) return hipSuccess;
  const int64_t blocks = (p.entries + kTouchPerBlock - 1) / kTouchPerBlock;
  return launch_kernel(page_touch_kernel, dim3((uint32_t)p.num_reqs, (uint32_t)blocks),
                       dim3(kTouchThreads), 0, stream, p);
}

}  // namespace hs
