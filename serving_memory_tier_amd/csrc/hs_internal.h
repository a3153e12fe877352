// Internal interface between the C-ABI layer (api.hip) and the kernels
// (resolve.hip, copy.hip).  Not installed; callers use include/hisparse.h.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace hs {

// Threads per resolver workgroup: 16 wave64s, one workgroup per request-layer.
constexpr int kResolveThreads = 1024;
// Threads per copy workgroup (gather / offload) and 16-byte pieces per thread
// per iteration.
constexpr int kCopyThreads = 256;
constexpr int kCopyUnroll = 4;

struct ResolveParams {
  // layout
  int32_t page_shift;
  int32_t row_bytes;
  int32_t num_layers;
  int32_t hot_capacity;      // C
  int64_t pool_rows, host_rows;
  int64_t pool_stride, host_stride;
  // batch
  int32_t num_reqs, max_pages;
  uint8_t* pool;
  const uint8_t* host;
  const int32_t* block_table;
  const int32_t* host_block_table;
  const int32_t* ctx_len;
  const int32_t* hot_blocks;
  int32_t* slot_token;
  uint32_t* slot_stamp;
  // call
  const int32_t* topk;
  int32_t entries;           // N = positions * top_k per request-layer
  uint32_t stamp;
  int32_t* row_ids;
  int32_t* stats;
};

// Enqueue the resolver (no gather).  Returns a hipError_t from the launch.
hipError_t launch_resolve(const ResolveParams& p, hipStream_t stream);

// Bytes of dynamic LDS the resolver needs for N entries and C slots.
size_t resolve_lds_bytes(int32_t entries, int32_t hot_capacity);

struct GatherParams {
  const uint8_t* pool;
  int64_t pool_rows;
  int64_t pool_stride;
  int32_t row_bytes;
  int32_t num_layers;
  const int32_t* row_ids;
  int32_t num_reqs;
  int32_t rows_per_rl;
  uint8_t* out;
};

hipError_t launch_gather(const GatherParams& p, hipStream_t stream);

struct OffloadParams {
  const uint8_t* pool;
  int64_t pool_stride;
  int64_t pool_blocks;
  uint8_t* host;
  int64_t host_stride;
  int64_t host_blocks;
  int64_t page_bytes;
  int32_t num_layers;
  const int32_t* pairs;
  int32_t n;
};

hipError_t launch_offload(const OffloadParams& p, hipStream_t stream);

}  // namespace hs
