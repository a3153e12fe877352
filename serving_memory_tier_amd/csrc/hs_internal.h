// Internal interface between the C-ABI layer (api.hip) and the kernels
// (resolve.hip, copy.hip).  Not installed; callers use include/hisparse.h.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace hs {

// Threads per resolver workgroup (one workgroup per request-layer).
#ifndef HS_RESOLVE_THREADS
#define HS_RESOLVE_THREADS 1024
#endif
constexpr int kResolveThreads = HS_RESOLVE_THREADS;
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

// LDS of one gfx950 compute unit, all of which one workgroup may use.
constexpr size_t kMaxLdsBytes = 160 * 1024;

// Bytes of dynamic LDS the resolver needs for N entries and C slots.
size_t resolve_lds_bytes(int32_t entries, int32_t hot_capacity);

// The row mover: the single-stride gather, and (fused) the host-link copies
// of the misses the resolver assigned.  Row ids in [0, pool_rows) are
// gathered from the pool; in fused mode a code -(8 + 2 q + c) names a miss
// assigned to hot slot q whose row is read from the host pool (and, when
// c = 1, also written into the slot), after which the code is replaced by
// the slot's row id; every other row id yields a zero row.
struct MoveParams {
  const uint8_t* pool;
  uint8_t* pool_w;              // hot-slot writes (fused mode)
  int64_t pool_rows;
  int64_t pool_stride;
  const uint8_t* host;          // fused mode
  int64_t host_rows;
  int64_t host_stride;
  int32_t row_bytes;
  int32_t num_layers;
  int32_t page_shift;
  int32_t max_pages;
  int32_t hot_capacity;
  const int32_t* topk;              // fused mode
  const int32_t* host_block_table;  // fused mode
  const int32_t* hot_blocks;        // fused mode
  int32_t* row_ids;
  int32_t num_reqs;
  int32_t rows_per_rl;
  uint8_t* out;                 // may be null in fused mode (copies only)
};

// Entries per wave in the row mover: a wave owns whole entries, so the codes
// it reads are rewritten only by itself.
constexpr int kMoveEntriesPerWave = 16;

hipError_t launch_move(const MoveParams& p, bool fused, hipStream_t stream);

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
