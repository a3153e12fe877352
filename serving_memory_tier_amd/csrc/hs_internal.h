// Internal interface between the C-ABI layer (api.hip) and the kernels
// (resolve.hip, copy.hip).  Not installed; callers use include/hisparse.h.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <atomic>

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
// Workgroups of the prefix-page offload, at most (each loops over its pages):
// 32 x 256 threads with 4 stores in flight each keep the link's device-to-host
// direction full and leave the rest of the chip to a resolve running beside
constexpr int64_t kOffloadGroups = 32;

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

struct FetchParams;

// Enqueue the resolver (no gather); with `fill`, the early fill's
// workgroups run in the same launch.  Returns the launch's hipError_t.
hipError_t launch_resolve(const ResolveParams& p, const FetchParams* fill, hipStream_t stream);

// LDS of one gfx950 compute unit, all of which one workgroup may use.
constexpr size_t kMaxLdsBytes = 160 * 1024;

// Raises a kernel's dynamic-LDS limit to the whole CU less its static LDS.
// The limit is a per-device attribute of the function, so it is set once on
// each device (bit d of `done` records device d).
inline hipError_t allow_full_lds(const void* fn, std::atomic<uint64_t>& done) {
  int dev = 0;
  hipError_t err = hipGetDevice(&dev);
  if (err != hipSuccess) return err;
  const uint64_t bit = 1ull << (dev & 63);
  if (done.load(std::memory_order_acquire) & bit) return hipSuccess;
  hipFuncAttributes attr{};
  err = hipFuncGetAttributes(&attr, fn);
  if (err != hipSuccess) return err;
  err = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize,
                            (int)(kMaxLdsBytes - attr.sharedSizeBytes));
  if (err != hipSuccess) return err;
  done.fetch_or(bit, std::memory_order_acq_rel);
  return hipSuccess;
}

// Workgroups of kernel `fn` (`threads` each, `lds` bytes of dynamic LDS) that
// the current device runs at once: compute units x workgroups per unit.  The
// unit count is read once per device.
inline hipError_t resident_groups(const void* fn, int threads, size_t lds, int64_t* groups) {
  static std::atomic<int32_t> cus[64] = {};
  int dev = 0;
  hipError_t err = hipGetDevice(&dev);
  if (err != hipSuccess) return err;
  int32_t n = cus[dev & 63].load(std::memory_order_acquire);
  if (n <= 0) {
    int v = 0;
    err = hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev);
    if (err != hipSuccess) return err;
    n = v;
    cus[dev & 63].store(n, std::memory_order_release);
  }
  int per = 0;
  err = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per, fn, threads, lds);
  if (err != hipSuccess) return err;
  *groups = (int64_t)n * per;
  return hipSuccess;
}

// Launches a kernel and returns that launch's own status (not whatever an
// earlier runtime call left behind for hipGetLastError).
template <typename... Args>
inline hipError_t launch_kernel(void (*fn)(Args...), dim3 grid, dim3 block, size_t lds,
                                hipStream_t stream, Args... args) {
  void* ptrs[] = {static_cast<void*>(&args)...};
  return hipLaunchKernel(reinterpret_cast<const void*>(fn), grid, block, ptrs, lds, stream);
}

// Bytes of dynamic LDS the resolver needs for N entries and C slots.
size_t resolve_lds_bytes(int32_t entries, int32_t hot_capacity);

// The row mover.  Row ids in [0, pool_rows) are gathered from the pool; a
// code -(8 + 2 q + c) names a miss assigned to hot slot q (c = 1 on the
// token's first entry, which fills the slot); -2 a miss left without a slot;
// any other negative id yields a zero row.  Modes:
//   kMoveGather  plain gather of row ids (no codes);
//   kMoveFused   misses read from the host pool into the output and, on the
//                first entry, into the slot; codes become the slot's row id
//                and the first entry records the slot's new token;
//   kMoveCommit  after the early fill (launch_fetch) wrote every output row:
//                first entries copy their row from the output into the slot
//                and record the slot's new token, codes become row ids, rows
//                of misses without a slot become zero rows.
enum MoveMode { kMoveGather = 0, kMoveFused = 1, kMoveCommit = 3 };

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
  int32_t* slot_token;              // fused / commit mode
  int32_t* row_ids;
  int32_t num_reqs;
  int32_t rows_per_rl;
  uint8_t* out;                 // may be null in fused mode (copies only)
  // layer groups sharing one top-K list and one hot-buffer state: num_layers
  // counts groups, each of `group` consecutive layers of the `layers` pool
  // planes; codes and row ids are per group, output rows per layer
  int32_t group = 1;
  int32_t layers = 0;           // 0: num_layers
};

// Entries per wave in the row mover: a wave owns whole entries, so the codes
// it reads are rewritten only by itself.
constexpr int kMoveEntriesPerWave = 16;

hipError_t launch_move(const MoveParams& p, MoveMode mode, hipStream_t stream);

// The early fill (fill.h; fetch.hip, and fused into the resolver's launch
// in resolve.hip): every entry's row of the gather output written from the
// state before the step -- resident and hot rows from the pool, misses from
// the host pool once per distinct token, zero rows otherwise -- while the
// resolver runs.
constexpr int kFillThreads = kResolveThreads;
// Host reads in flight per miss-workgroup thread, and miss workgroups per
// launch (at most): together they bound the host reads in flight.
#ifndef HS_HOST_UNROLL
#define HS_HOST_UNROLL 1
#endif
#ifndef HS_HOST_GROUPS
#define HS_HOST_GROUPS 32
#endif
constexpr int kHostUnroll = HS_HOST_UNROLL;
constexpr int kFetchHostGroups = HS_HOST_GROUPS;
constexpr int kFetchMaxSplits = 16;        // miss workgroups per request-layer, at most
constexpr int kFetchGatherTarget = 256;    // gather workgroups per launch to aim for
// (unless fewer fit beside the launch's other workgroups in one round of the
// chip; then that many, if at least this many)
constexpr int kFetchGatherMinGroups = 64;
constexpr int kFetchGatherMin = 64;        // entries per gather workgroup, at least
constexpr int kFetchGatherEntries = 512;   // entries per gather workgroup, at most

struct FetchParams {
  int32_t page_shift;
  int32_t row_bytes;
  int32_t num_layers;
  int32_t hot_capacity;
  int64_t pool_rows, host_rows;
  int64_t pool_stride, host_stride;
  int32_t num_reqs, max_pages;
  const uint8_t* pool;
  const uint8_t* host;
  const int32_t* block_table;
  const int32_t* host_block_table;
  const int32_t* ctx_len;
  const int32_t* hot_blocks;
  const int32_t* slot_token;
  const int32_t* topk;
  int32_t entries;
  uint8_t* out;
  // layer groups (as MoveParams): num_layers counts groups of `group` layers
  int32_t group;
  int32_t layers;
  // set by prepare_fetch
  int32_t miss_groups, miss_splits, gather_splits;
  int32_t lds_n, miss_tab_n, gather_e, gather_tab_n;
  uint32_t piece_magic;
  // 1: no gather workgroups; the misses' host rows go to their first entries
  // only (a staging buffer for callers that read rows in place)
  int32_t misses_only = 0;
  // > 0 (set by prepare_fetch where it fits): the miss workgroups mark the
  // tokens the usable slots hold in a bitmap of this many words
  int32_t slot_bits_words = 0;
  // the batch's fill_sync words (zero between launches), or null: with more
  // items than miss workgroups, each takes its next item from a counter
  int32_t* sync = nullptr;
};

// fill_sync words: workgroups done, items taken (on separate 128-byte lines)
constexpr int kSyncDone = 0;
constexpr int kSyncItems = 32;

// Bytes of dynamic LDS a fill workgroup needs for N entries.
size_t fetch_lds_bytes(int32_t entries, int32_t hot_capacity);
// Completes p's launch shape; returns the number of fill workgroups and sets
// *lds_bytes.
// gather_target: gather workgroups to aim for (<= 0: kFetchGatherTarget).
int64_t prepare_fetch(FetchParams& p, size_t* lds_bytes, int64_t gather_target);
// The fill as a kernel of its own.
hipError_t launch_fetch(FetchParams p, hipStream_t stream);

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

// Page coldness stamps from the top-K lists: for every request r and entry
// t = topk[r * entries + e] with 0 <= t < min(ctx_len[r], max_pages <<
// page_shift), page_use[r * max_pages + (t >> page_shift)] = stamp.
struct TouchParams {
  const int32_t* topk;
  const int32_t* ctx_len;
  uint32_t* page_use;
  int64_t entries;      // entries per request
  int32_t num_reqs;
  int32_t max_pages;
  int32_t page_shift;
  uint32_t stamp;
};

constexpr int64_t kTouchPerBlock = 1024;
constexpr int64_t kTouchMaxEntries = kTouchPerBlock * 65535;

hipError_t launch_page_touch(const TouchParams& p, hipStream_t stream);

// Sparse MLA decode over rows read in place by row id (attend.hip): 656-byte
// FP8 MLA rows, 576-wide bf16 queries, 512-wide float32 outputs.
constexpr int kAttendThreads = 512;
#ifndef HS_ATTEND_TARGET
#define HS_ATTEND_TARGET 256
#endif
constexpr int kAttendHeadsPerGroup = 64;  // heads per workgroup
constexpr int kAttendMaxSplits = 64;       // key splits per (token, head group), at most
constexpr int kAttendMaxSplitKeys = 2048;  // keys per split, at most (their row ids sit in LDS)
constexpr int64_t kAttendTargetGroups = HS_ATTEND_TARGET;  // workgroups per launch to aim for

struct AttendParams {
  const uint8_t* kv;        // one layer of the pool
  int64_t pool_rows;
  const int32_t* row_ids;   // [tokens][top_k]
  int32_t top_k;
  int32_t num_tokens;
  const uint16_t* q;        // [tokens][heads][576] bf16
  int32_t num_heads;
  float sm_scale;
  float* out;               // [tokens][heads][512]
  float* lse;               // [tokens][heads]
  uint16_t* part_o;         // workspace: [tokens][splits][heads][512] IEEE half bits, each
                            // split's output already divided by its sum
  float* part_ml;           // workspace: [tokens][splits][heads][2] (running max, sum)
  int32_t splits;
  int32_t keys_per_split;   // a multiple of 32
  int32_t head_groups;      // ceil(num_heads / kAttendHeadsPerGroup)
};

// Bytes of the per-device workspace of hs_sparse_mla_decode_noalloc.
constexpr size_t kAttendScratchBytes = size_t(64) << 20;
// That workspace's device address on the current device (looked up once per
// device; no allocation).
hipError_t attend_scratch(void** ptr);

size_t attend_lds_bytes();
// Sets splits and keys_per_split for about target_groups workgroups.
void plan_attend(AttendParams& p, int64_t target_groups);
hipError_t launch_attend(const AttendParams& p, hipStream_t stream);

}  // namespace hs
