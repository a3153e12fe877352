// Streaming copy kernels for gfx950: the single-stride row gather and the
// post-forward prefix-page offload.
//
// Method: "vLLM GLM 5.3 ... Hybrid HiSparse offloading, Part 1", section
// "How it works": the resolver hands back a row id whether the row is
// resident or hot, and the rows are gathered at one stride; completed prefix
// pages are copied to host while still served from the GPU, all sparse layers
// in one launch after the forward, ordered on the model's stream.
//
// Both kernels are bound by memory bandwidth (HBM for the gather, the host
// link for the offload), not by arithmetic, so they are written as wide,
// coalesced 16-byte streams: consecutive lanes move consecutive 16-byte
// pieces, each lane keeps kCopyUnroll loads in flight before storing, and
// the grid is large enough to cover all 256 compute units several times.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "hs_internal.h"

namespace hs {
namespace {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

constexpr int kT = kCopyThreads;
constexpr int kU = kCopyUnroll;
constexpr int kPiecesPerBlock = kT * kU;

// One workgroup moves kPiecesPerBlock consecutive 16-byte pieces of one
// request-layer's output; blocks_per_rl workgroups cover a request-layer.
// PIECES = row_bytes / 16 when known at compile time (0 = runtime).
template <int PIECES>
__global__ void __launch_bounds__(kT) gather_kernel(GatherParams p, int32_t blocks_per_rl) {
  const int32_t rl = blockIdx.x / blocks_per_rl;
  const int32_t bx = blockIdx.x - rl * blocks_per_rl;
  const int32_t layer = rl % p.num_layers;
  const int32_t pieces = PIECES > 0 ? PIECES : (p.row_bytes >> 4);
  const uint32_t rl_pieces = (uint32_t)p.rows_per_rl * (uint32_t)pieces;
  const int32_t* rows = p.row_ids + (int64_t)rl * p.rows_per_rl;
  const uint8_t* pool_l = p.pool + (int64_t)layer * p.pool_stride;
  uint8_t* out = p.out + (int64_t)rl * p.rows_per_rl * p.row_bytes;
  const uint32_t base = (uint32_t)bx * kPiecesPerBlock + threadIdx.x;

  u32x4 v[kU];
#pragma unroll
  for (int u = 0; u < kU; ++u) {
    const uint32_t g = base + u * kT;
    v[u] = u32x4{0u, 0u, 0u, 0u};
    if (g < rl_pieces) {
      const uint32_t e = g / (uint32_t)pieces;
      const uint32_t pc = g - e * (uint32_t)pieces;
      const int32_t row = rows[e];
      if (row >= 0 && row < p.pool_rows)
        v[u] = *reinterpret_cast<const u32x4*>(pool_l + (int64_t)row * p.row_bytes + pc * 16u);
    }
  }
#pragma unroll
  for (int u = 0; u < kU; ++u) {
    const uint32_t g = base + u * kT;
    if (g < rl_pieces)
      __builtin_nontemporal_store(v[u], reinterpret_cast<u32x4*>(out + (uint64_t)g * 16u));
  }
}

// One workgroup copies one page of one layer: blockIdx.x = pair, blockIdx.y = layer.
__global__ void __launch_bounds__(kT) offload_kernel(OffloadParams p) {
  const int32_t i = blockIdx.x;
  const int32_t layer = blockIdx.y;
  const int64_t db = p.pairs[2 * i];
  const int64_t hb = p.pairs[2 * i + 1];
  if (db < 0 || db >= p.pool_blocks || hb < 0 || hb >= p.host_blocks) return;
  const uint8_t* src = p.pool + (int64_t)layer * p.pool_stride + db * p.page_bytes;
  uint8_t* dst = p.host + (int64_t)layer * p.host_stride + hb * p.page_bytes;
  const int32_t n = (int32_t)(p.page_bytes >> 4);
  for (int32_t b = threadIdx.x; b < n; b += kPiecesPerBlock) {
    u32x4 v[kU];
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const int32_t g = b + u * kT;
      if (g < n) v[u] = *reinterpret_cast<const u32x4*>(src + (int64_t)g * 16);
    }
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const int32_t g = b + u * kT;
      if (g < n) *reinterpret_cast<u32x4*>(dst + (int64_t)g * 16) = v[u];
    }
  }
}

}  // namespace

hipError_t launch_gather(const GatherParams& p, hipStream_t stream) {
  const int64_t n_rl = (int64_t)p.num_reqs * p.num_layers;
  if (n_rl == 0 || p.rows_per_rl == 0) return hipSuccess;
  const int64_t rl_pieces = (int64_t)p.rows_per_rl * (p.row_bytes >> 4);
  const int64_t blocks_per_rl = (rl_pieces + kPiecesPerBlock - 1) / kPiecesPerBlock;
  const int64_t grid = n_rl * blocks_per_rl;
  if (p.row_bytes == 656)
    hipLaunchKernelGGL(gather_kernel<41>, dim3((uint32_t)grid), dim3(kT), 0, stream, p,
                       (int32_t)blocks_per_rl);
  else
    hipLaunchKernelGGL(gather_kernel<0>, dim3((uint32_t)grid), dim3(kT), 0, stream, p,
                       (int32_t)blocks_per_rl);
  return hipGetLastError();
}

hipError_t launch_offload(const OffloadParams& p, hipStream_t stream) {
  if (p.n == 0 || p.num_layers == 0) return hipSuccess;
  hipLaunchKernelGGL(offload_kernel, dim3((uint32_t)p.n, (uint32_t)p.num_layers), dim3(kT), 0,
                     stream, p);
  return hipGetLastError();
}

}  // namespace hs
