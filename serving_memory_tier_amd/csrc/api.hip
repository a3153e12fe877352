// C ABI of the Hybrid HiSparse hot path (declared in include/hisparse.h):
// argument validation, launch shapes and HIP error mapping.  Every entry
// point validates everything the host can see before enqueuing anything,
// then enqueues its kernels on the caller's stream and returns without
// waiting ("How it works": nothing on the decode path waits on the CPU).

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <cstdio>

#include "hisparse.h"
#include "hs_internal.h"

namespace {

bool is_pow2(int64_t x) { return x > 0 && (x & (x - 1)) == 0; }

int log2i(int64_t x) {
  int s = 0;
  while ((int64_t(1) << s) < x) ++s;
  return s;
}

// The kernels move 16-byte pieces: pools, outputs and layer strides are
// 16-byte aligned.
bool aligned16(const void* ptr) { return ((uintptr_t)ptr & 15) == 0; }

// Checks shared by every call that reads the pool layout.
hs_status check_layout(const hs_layout* lay) {
  if (!lay) return HS_ERR_INVALID_ARGUMENT;
  if (!is_pow2(lay->page_size) || lay->page_size > 4096) return HS_ERR_INVALID_ARGUMENT;
  if (lay->row_bytes <= 0 || lay->row_bytes % 16 != 0 || lay->row_bytes > (1 << 20))
    return HS_ERR_INVALID_ARGUMENT;
  if (lay->num_layers < 1 || lay->num_layers > 65535) return HS_ERR_INVALID_ARGUMENT;
  if (lay->pool_rows <= 0 || lay->pool_rows % lay->page_size != 0 || lay->pool_rows > INT32_MAX)
    return HS_ERR_INVALID_ARGUMENT;
  if (lay->host_rows < 0 || lay->host_rows % lay->page_size != 0 || lay->host_rows > INT32_MAX)
    return HS_ERR_INVALID_ARGUMENT;
  if (lay->num_layers > 1) {
    if (lay->pool_layer_stride < lay->pool_rows * lay->row_bytes) return HS_ERR_INVALID_ARGUMENT;
    if (lay->host_layer_stride < lay->host_rows * lay->row_bytes) return HS_ERR_INVALID_ARGUMENT;
    if (lay->pool_layer_stride % 16 != 0 || lay->host_layer_stride % 16 != 0)
      return HS_ERR_INVALID_ARGUMENT;
  }
  return HS_OK;
}

hs_status check_hot(const hs_layout* lay) {
  if (lay->hot_capacity < lay->page_size || lay->hot_capacity % lay->page_size != 0)
    return HS_ERR_INVALID_ARGUMENT;
  if (lay->hot_capacity > HS_MAX_HOT_CAPACITY) return HS_ERR_UNSUPPORTED;
  return HS_OK;
}

// The last HIP failure on this thread, for hs_last_error.
thread_local char g_last_error[160] = "";

void note(const char* what, hipError_t e) {
  snprintf(g_last_error, sizeof g_last_error, "%s: %s (%d)", what, hipGetErrorName(e), (int)e);
}

hs_status from_hip(hipError_t e, const char* what) {
  if (e == hipSuccess) return HS_OK;
  note(what, e);
  return HS_ERR_LAUNCH;
}

// A HIP runtime call other than a launch.
bool hip_ok(hipError_t e, const char* what) {
  if (e == hipSuccess) return true;
  note(what, e);
  return false;
}

hs_status check_gather(const hs_layout* lay, int64_t n_rl, int64_t rows_per_rl) {
  (void)lay;
  const int64_t chunks = (rows_per_rl + hs::kMoveEntriesPerWave - 1) / hs::kMoveEntriesPerWave;
  if (n_rl * chunks >= (int64_t(1) << 31)) return HS_ERR_UNSUPPORTED;
  return HS_OK;
}

hs_status check_offload(int32_t n) {
  if (n < 0) return HS_ERR_INVALID_ARGUMENT;
  return HS_OK;
}

hs::OffloadParams offload_params(const hs_layout* lay, const uint8_t* pool, uint8_t* host,
                                 const int32_t* pairs, int32_t n) {
  hs::OffloadParams o;
  o.pool = pool;
  o.pool_stride = lay->pool_layer_stride;
  o.pool_blocks = lay->pool_rows / lay->page_size;
  o.host = host;
  o.host_stride = lay->host_layer_stride;
  o.host_blocks = lay->host_rows / lay->page_size;
  o.page_bytes = (int64_t)lay->page_size * lay->row_bytes;
  o.num_layers = lay->num_layers;
  o.pairs = pairs;
  o.n = n;
  return o;
}

hs::MoveParams move_params(const hs_layout* lay, const uint8_t* pool, int32_t* rows,
                           int32_t num_reqs, int32_t rows_per_rl, uint8_t* out) {
  hs::MoveParams g{};
  g.pool = pool;
  g.pool_rows = lay->pool_rows;
  g.pool_stride = lay->pool_layer_stride;
  g.row_bytes = lay->row_bytes;
  g.num_layers = lay->num_layers;
  g.page_shift = log2i(lay->page_size);
  g.hot_capacity = lay->hot_capacity;
  g.row_ids = rows;
  g.num_reqs = num_reqs;
  g.rows_per_rl = rows_per_rl;
  g.out = out;
  return g;
}

// Checks shared by hs_resolve, hs_plan_replay and their two halves.
hs_status check_resolve(const hs_layout* lay, const hs_batch* b, const int32_t* topk,
                        int32_t num_pos, int32_t top_k, const int32_t* row_ids) {
  hs_status s = check_layout(lay);
  if (s != HS_OK) return s;
  if ((s = check_hot(lay)) != HS_OK) return s;
  if (!b || !topk || !row_ids) return HS_ERR_INVALID_ARGUMENT;
  if (b->num_reqs < 0 || b->max_pages < 1) return HS_ERR_INVALID_ARGUMENT;
  if (lay->row_bytes > HS_MAX_ROW_BYTES) return HS_ERR_UNSUPPORTED;
  if (b->fill_sync ? b->fill_sync_words < HS_FILL_SYNC_WORDS : b->fill_sync_words != 0)
    return HS_ERR_INVALID_ARGUMENT;
  if (num_pos < 1 || top_k < 1) return HS_ERR_INVALID_ARGUMENT;
  if ((int64_t)num_pos * top_k > HS_MAX_ENTRIES) return HS_ERR_UNSUPPORTED;
  const int64_t n_rl = (int64_t)b->num_reqs * lay->num_layers;
  if (n_rl > INT32_MAX) return HS_ERR_UNSUPPORTED;
  if ((s = check_gather(lay, n_rl, (int64_t)num_pos * top_k)) != HS_OK) return s;
  if (hs::resolve_lds_bytes(num_pos * top_k, lay->hot_capacity) > hs::kMaxLdsBytes)
    return HS_ERR_UNSUPPORTED;
  if (b->num_reqs > 0) {
    if (!b->kv_pool || !b->block_table || !b->host_block_table || !b->ctx_len ||
        !b->hot_blocks || !b->slot_token || !b->slot_stamp)
      return HS_ERR_INVALID_ARGUMENT;
    if (!b->host_pool && lay->host_rows > 0) return HS_ERR_INVALID_ARGUMENT;
    if (!aligned16(b->kv_pool) || !aligned16(b->host_pool)) return HS_ERR_INVALID_ARGUMENT;
  }
  return HS_OK;
}

hs::FetchParams fetch_params(const hs_layout* lay, const hs_batch* b, const int32_t* topk,
                             int32_t N, uint8_t* gather_out);

hs_status launch_decide(const hs_layout* lay, const hs_batch* b, const int32_t* topk,
                        int32_t N, uint32_t stamp, int32_t* row_ids, int32_t* stats,
                        hipStream_t stream, uint8_t* fill_out = nullptr, int32_t group = 1,
                        bool misses_only = false) {
  if ((int64_t)b->num_reqs * lay->num_layers == 0) return HS_OK;
  // with layer groups the resolver runs once per (request, group): the state,
  // lists and row ids are per group
  hs_layout glay = *lay;
  glay.num_layers = lay->num_layers / group;
  hs::ResolveParams p;
  p.page_shift = log2i(lay->page_size);
  p.row_bytes = lay->row_bytes;
  p.num_layers = glay.num_layers;
  p.hot_capacity = lay->hot_capacity;
  p.pool_rows = lay->pool_rows;
  p.host_rows = lay->host_rows;
  p.pool_stride = lay->pool_layer_stride;
  p.host_stride = lay->host_layer_stride;
  p.num_reqs = b->num_reqs;
  p.max_pages = b->max_pages;
  p.pool = b->kv_pool;
  p.host = b->host_pool;
  p.block_table = b->block_table;
  p.host_block_table = b->host_block_table;
  p.ctx_len = b->ctx_len;
  p.hot_blocks = b->hot_blocks;
  p.slot_token = b->slot_token;
  p.slot_stamp = b->slot_stamp;
  p.topk = topk;
  p.entries = N;
  p.stamp = stamp;
  p.row_ids = row_ids;
  p.stats = stats;
  if (fill_out) {
    hs::FetchParams f = fetch_params(&glay, b, topk, N, fill_out);
    f.group = group;
    f.layers = lay->num_layers;
    f.misses_only = misses_only ? 1 : 0;
    return from_hip(hs::launch_resolve(p, &f, stream), "resolver launch");
  }
  return from_hip(hs::launch_resolve(p, nullptr, stream), "resolver launch");
}

hs_status launch_move_mode(const hs_layout* lay, const hs_batch* b, const int32_t* topk,
                           int32_t N, int32_t* row_ids, uint8_t* gather_out, hs::MoveMode mode,
                           hipStream_t stream, int32_t group = 1) {
  if ((int64_t)b->num_reqs * lay->num_layers == 0) return HS_OK;
  hs::MoveParams g = move_params(lay, b->kv_pool, row_ids, b->num_reqs, N, gather_out);
  g.num_layers = lay->num_layers / group;  // codes and row ids per (request, group)
  g.group = group;
  g.layers = lay->num_layers;
  g.pool_w = b->kv_pool;
  g.host = b->host_pool;
  g.host_rows = lay->host_rows;
  g.host_stride = lay->host_layer_stride;
  g.max_pages = b->max_pages;
  g.topk = topk;
  g.host_block_table = b->host_block_table;
  g.hot_blocks = b->hot_blocks;
  g.slot_token = b->slot_token;
  return from_hip(hs::launch_move(g, mode, stream), "row mover launch");
}

hs::FetchParams fetch_params(const hs_layout* lay, const hs_batch* b, const int32_t* topk,
                             int32_t N, uint8_t* gather_out) {
  hs::FetchParams f{};
  f.page_shift = log2i(lay->page_size);
  f.row_bytes = lay->row_bytes;
  f.num_layers = lay->num_layers;
  f.hot_capacity = lay->hot_capacity;
  f.pool_rows = lay->pool_rows;
  f.host_rows = lay->host_rows;
  f.pool_stride = lay->pool_layer_stride;
  f.host_stride = lay->host_layer_stride;
  f.num_reqs = b->num_reqs;
  f.max_pages = b->max_pages;
  f.pool = b->kv_pool;
  f.host = b->host_pool;
  f.block_table = b->block_table;
  f.host_block_table = b->host_block_table;
  f.ctx_len = b->ctx_len;
  f.hot_blocks = b->hot_blocks;
  f.slot_token = b->slot_token;
  f.sync = b->fill_sync;
  f.topk = topk;
  f.entries = N;
  f.out = gather_out;
  f.group = 1;
  f.layers = lay->num_layers;
  return f;
}

hs_status launch_fetch(const hs_layout* lay, const hs_batch* b, const int32_t* topk, int32_t N,
                       uint8_t* gather_out, hipStream_t stream) {
  if ((int64_t)b->num_reqs * lay->num_layers == 0) return HS_OK;
  return from_hip(hs::launch_fetch(fetch_params(lay, b, topk, N, gather_out), stream),
                  "prefetch launch");
}

bool fetch_fits(const hs_layout* lay, int32_t N) {
  return hs::fetch_lds_bytes(N, lay->hot_capacity) <= hs::kMaxLdsBytes;
}

// Shared body of hs_resolve and hs_plan_replay, on the caller's stream.
//
// With a gather output: one launch holds the resolver's workgroups and the
// early fill's (every output row, the misses' host-link reads included,
// written from the pre-call state); then the commit fills the assigned hot
// slots from the output.  Without one: the resolver, then the misses'
// copies into their slots.  The offload of completed prefix pages comes
// last.
hs_status resolve_common(const hs_layout* lay, const hs_batch* b, const int32_t* topk,
                         int32_t num_pos, int32_t top_k, uint32_t stamp, int32_t* row_ids,
                         uint8_t* gather_out, int32_t* stats, const int32_t* offload_pairs,
                         int32_t n_offload, hipStream_t stream, int32_t group = 1,
                         uint8_t* staging = nullptr) {
  hs_status s = check_resolve(lay, b, topk, num_pos, top_k, row_ids);
  if (s != HS_OK) return s;
  if (group < 1 || lay->num_layers % group != 0) return HS_ERR_INVALID_ARGUMENT;
  if (!stats || stamp == 0) return HS_ERR_INVALID_ARGUMENT;
  if (!aligned16(gather_out) || !aligned16(staging)) return HS_ERR_INVALID_ARGUMENT;
  if ((s = check_offload(n_offload)) != HS_OK) return s;
  if (n_offload > 0 && (!offload_pairs || !b->kv_pool || !b->host_pool))
    return HS_ERR_INVALID_ARGUMENT;
  const int32_t N = num_pos * top_k;
  if (staging && fetch_fits(lay, N)) {
    // rows read in place later: only the misses' host rows are staged, at
    // their first entries, while the resolver decides; commit moves them
    s = launch_decide(lay, b, topk, N, stamp, row_ids, stats, stream, staging, group, true);
    if (s != HS_OK) return s;
    s = launch_move_mode(lay, b, topk, N, row_ids, staging, hs::kMoveCommit, stream, group);
    if (s != HS_OK) return s;
  } else if (gather_out && fetch_fits(lay, N)) {
    s = launch_decide(lay, b, topk, N, stamp, row_ids, stats, stream, gather_out, group);
    if (s != HS_OK) return s;
    s = launch_move_mode(lay, b, topk, N, row_ids, gather_out, hs::kMoveCommit, stream, group);
    if (s != HS_OK) return s;
  } else {
    s = launch_decide(lay, b, topk, N, stamp, row_ids, stats, stream, nullptr, group);
    if (s != HS_OK) return s;
    s = launch_move_mode(lay, b, topk, N, row_ids, gather_out, hs::kMoveFused, stream, group);
    if (s != HS_OK) return s;
  }
  if (n_offload > 0) {
    hs::OffloadParams o = offload_params(lay, b->kv_pool, const_cast<uint8_t*>(b->host_pool),
                                         offload_pairs, n_offload);
    if ((s = from_hip(hs::launch_offload(o, stream), "offload launch")) != HS_OK) return s;
  }
  return HS_OK;
}

}  // namespace

extern "C" {

hs_status hs_resolve(const hs_layout* layout, const hs_batch* batch, const int32_t* topk,
                     int32_t top_k, uint32_t stamp, int32_t* row_ids, uint8_t* gather_out,
                     int32_t* stats, hipStream_t stream) {
  return resolve_common(layout, batch, topk, 1, top_k, stamp, row_ids, gather_out, stats,
                        nullptr, 0, stream);
}

hs_status hs_plan_replay(const hs_layout* layout, const hs_batch* batch, const int32_t* topk,
                         int32_t num_pos, int32_t top_k, uint32_t stamp, int32_t* row_ids,
                         uint8_t* gather_out, int32_t* stats, const int32_t* offload_pairs,
                         int32_t n_offload, hipStream_t stream) {
  return resolve_common(layout, batch, topk, num_pos, top_k, stamp, row_ids, gather_out, stats,
                        offload_pairs, n_offload, stream);
}

hs_status hs_resolve_in_place(const hs_layout* layout, const hs_batch* batch, const int32_t* topk,
                              int32_t num_pos, int32_t top_k, uint32_t stamp, int32_t* row_ids,
                              uint8_t* staging, int32_t* stats, const int32_t* offload_pairs,
                              int32_t n_offload, hipStream_t stream) {
  if (!staging) return HS_ERR_INVALID_ARGUMENT;
  return resolve_common(layout, batch, topk, num_pos, top_k, stamp, row_ids, nullptr, stats,
                        offload_pairs, n_offload, stream, 1, staging);
}

hs_status hs_resolve_grouped(const hs_layout* layout, const hs_batch* batch, int32_t group_layers,
                             const int32_t* topk, int32_t num_pos, int32_t top_k, uint32_t stamp,
                             int32_t* row_ids, uint8_t* gather_out, int32_t* stats,
                             const int32_t* offload_pairs, int32_t n_offload,
                             hipStream_t stream) {
  return resolve_common(layout, batch, topk, num_pos, top_k, stamp, row_ids, gather_out, stats,
                        offload_pairs, n_offload, stream, group_layers);
}

hs_status hs_resolve_decide(const hs_layout* layout, const hs_batch* batch, const int32_t* topk,
                            int32_t num_pos, int32_t top_k, uint32_t stamp, int32_t* row_ids,
                            uint8_t* gather_out, int32_t* stats, hipStream_t stream) {
  hs_status s = check_resolve(layout, batch, topk, num_pos, top_k, row_ids);
  if (s != HS_OK) return s;
  if (!stats || stamp == 0) return HS_ERR_INVALID_ARGUMENT;
  if (!aligned16(gather_out)) return HS_ERR_INVALID_ARGUMENT;
  const int32_t N = num_pos * top_k;
  if (gather_out && !fetch_fits(layout, N)) return HS_ERR_UNSUPPORTED;
  return launch_decide(layout, batch, topk, N, stamp, row_ids, stats, stream, gather_out);
}

hs_status hs_resolve_fetch(const hs_layout* layout, const hs_batch* batch, const int32_t* topk,
                           int32_t num_pos, int32_t top_k, uint8_t* gather_out,
                           hipStream_t stream) {
  hs_status s = check_resolve(layout, batch, topk, num_pos, top_k, topk);
  if (s != HS_OK) return s;
  if (!gather_out || !aligned16(gather_out)) return HS_ERR_INVALID_ARGUMENT;
  if (!fetch_fits(layout, num_pos * top_k)) return HS_ERR_UNSUPPORTED;
  return launch_fetch(layout, batch, topk, num_pos * top_k, gather_out, stream);
}

hs_status hs_resolve_move(const hs_layout* layout, const hs_batch* batch, const int32_t* topk,
                          int32_t num_pos, int32_t top_k, int32_t* row_ids, uint8_t* gather_out,
                          hipStream_t stream) {
  hs_status s = check_resolve(layout, batch, topk, num_pos, top_k, row_ids);
  if (s != HS_OK) return s;
  if (!aligned16(gather_out)) return HS_ERR_INVALID_ARGUMENT;
  return launch_move_mode(layout, batch, topk, num_pos * top_k, row_ids, gather_out,
                          hs::kMoveFused, stream);
}

hs_status hs_resolve_commit(const hs_layout* layout, const hs_batch* batch, const int32_t* topk,
                            int32_t num_pos, int32_t top_k, int32_t* row_ids,
                            uint8_t* gather_out, hipStream_t stream) {
  hs_status s = check_resolve(layout, batch, topk, num_pos, top_k, row_ids);
  if (s != HS_OK) return s;
  if (!gather_out || !aligned16(gather_out)) return HS_ERR_INVALID_ARGUMENT;
  return launch_move_mode(layout, batch, topk, num_pos * top_k, row_ids, gather_out,
                          hs::kMoveCommit, stream);
}

hs_status hs_gather(const hs_layout* layout, const uint8_t* kv_pool, const int32_t* row_ids,
                    int32_t num_reqs, int32_t rows_per_req_layer, uint8_t* out,
                    hipStream_t stream) {
  hs_status s = check_layout(layout);
  if (s != HS_OK) return s;
  if (num_reqs < 0 || rows_per_req_layer < 0) return HS_ERR_INVALID_ARGUMENT;
  const int64_t n_rl = (int64_t)num_reqs * layout->num_layers;
  if (n_rl == 0 || rows_per_req_layer == 0) return HS_OK;
  if (!kv_pool || !row_ids || !out) return HS_ERR_INVALID_ARGUMENT;
  if (!aligned16(kv_pool) || !aligned16(out)) return HS_ERR_INVALID_ARGUMENT;
  if ((s = check_gather(layout, n_rl, rows_per_req_layer)) != HS_OK) return s;
  return from_hip(hs::launch_move(
      move_params(layout, kv_pool, const_cast<int32_t*>(row_ids), num_reqs, rows_per_req_layer,
                  out),
      hs::kMoveGather, stream), "gather launch");
}

hs_status hs_offload_prefix_pages(const hs_layout* layout, const uint8_t* kv_pool,
                                  uint8_t* host_pool, const int32_t* pairs, int32_t n,
                                  hipStream_t stream) {
  hs_status s = check_layout(layout);
  if (s != HS_OK) return s;
  if ((s = check_offload(n)) != HS_OK) return s;
  if (n == 0) return HS_OK;
  if (!kv_pool || !host_pool || !pairs) return HS_ERR_INVALID_ARGUMENT;
  if (!aligned16(kv_pool) || !aligned16(host_pool)) return HS_ERR_INVALID_ARGUMENT;
  return from_hip(hs::launch_offload(offload_params(layout, kv_pool, host_pool, pairs, n), stream),
                  "offload launch");
}

hs_status hs_page_touch(const hs_layout* layout, const hs_batch* batch, const int32_t* topk,
                        int32_t entries_per_req, uint32_t stamp, uint32_t* page_use,
                        hipStream_t stream) {
  hs_status s = check_layout(layout);
  if (s != HS_OK) return s;
  if (!batch || batch->num_reqs < 0 || batch->max_pages < 1 || entries_per_req < 0)
    return HS_ERR_INVALID_ARGUMENT;
  if (entries_per_req > hs::kTouchMaxEntries) return HS_ERR_UNSUPPORTED;
  if (batch->num_reqs == 0 || entries_per_req == 0) return HS_OK;
  if (!topk || !page_use || !batch->ctx_len) return HS_ERR_INVALID_ARGUMENT;
  hs::TouchParams p;
  p.topk = topk;
  p.ctx_len = batch->ctx_len;
  p.page_use = page_use;
  p.entries = entries_per_req;
  p.num_reqs = batch->num_reqs;
  p.max_pages = batch->max_pages;
  p.page_shift = log2i(layout->page_size);
  p.stamp = stamp;
  return from_hip(hs::launch_page_touch(p, stream), "page touch launch");
}

namespace {

// The attention plan for a call, and the workspace it needs (0: one split).
hs::AttendParams attend_plan(int32_t num_tokens, int32_t num_heads, int32_t top_k,
                             size_t* workspace) {
  hs::AttendParams p{};
  p.num_tokens = num_tokens;
  p.num_heads = num_heads;
  p.top_k = top_k;
  hs::plan_attend(p, hs::kAttendTargetGroups);
  // per (token, split, head): 512 half-precision outputs and two floats
  *workspace = p.splits > 1 ? (size_t)num_tokens * p.splits * num_heads * (512 * 2 + 2 * 4) : 0;
  return p;
}


}  // namespace

size_t hs_sparse_mla_workspace_bytes(int32_t num_tokens, int32_t num_heads, int32_t top_k) {
  if (num_tokens <= 0 || num_heads <= 0 || top_k < 0) return 0;
  size_t ws = 0;
  attend_plan(num_tokens, num_heads, top_k, &ws);
  return ws;
}

namespace {

// Shared body of hs_sparse_mla_decode and its allocation-free form; with
// `noalloc` the workspace is the library's per-device array instead of the
// caller's.
hs_status sparse_mla_decode(const hs_layout* layout, const uint8_t* kv_layer,
                            const int32_t* row_ids, int32_t num_tokens, int32_t top_k,
                            const uint16_t* q, int32_t num_heads, float sm_scale, float* out,
                            float* lse, void* workspace, size_t workspace_bytes, bool noalloc,
                            hipStream_t stream) {
  hs_status s = check_layout(layout);
  if (s != HS_OK) return s;
  if (layout->row_bytes != 656) return HS_ERR_UNSUPPORTED;
  if (num_tokens < 0 || top_k < 0 || num_heads <= 0 || num_heads % 16 != 0)
    return HS_ERR_INVALID_ARGUMENT;
  if (num_tokens > 65535 || num_heads > 16 * 65535) return HS_ERR_UNSUPPORTED;
  if ((int64_t)top_k > (int64_t)hs::kAttendMaxSplits * hs::kAttendMaxSplitKeys)
    return HS_ERR_UNSUPPORTED;
  if (num_tokens == 0) return HS_OK;
  if (!q || !out || !lse || (top_k > 0 && (!kv_layer || !row_ids))) return HS_ERR_INVALID_ARGUMENT;
  if (!aligned16(q) || !aligned16(out) || (kv_layer && !aligned16(kv_layer)))
    return HS_ERR_INVALID_ARGUMENT;
  size_t need = 0;
  hs::AttendParams p = attend_plan(num_tokens, num_heads, top_k, &need);
  if (noalloc) {
    if (need > hs::kAttendScratchBytes) return HS_ERR_UNSUPPORTED;
    workspace = nullptr;
    if (need > 0 && !hip_ok(hs::attend_scratch(&workspace), "workspace symbol lookup"))
      return HS_ERR_HIP;
    workspace_bytes = hs::kAttendScratchBytes;
  }
  if (need > 0 && (!workspace || workspace_bytes < need || !aligned16(workspace)))
    return HS_ERR_INVALID_ARGUMENT;
  p.kv = kv_layer;
  p.pool_rows = layout->pool_rows;
  p.row_ids = row_ids;
  p.q = q;
  p.sm_scale = sm_scale;
  p.out = out;
  p.lse = lse;
  p.part_o = need > 0 ? static_cast<uint16_t*>(workspace) : nullptr;
  p.part_ml = need > 0 ? reinterpret_cast<float*>(p.part_o + (size_t)num_tokens * p.splits *
                                                                 num_heads * 512)
                       : nullptr;
  return from_hip(hs::launch_attend(p, stream), "sparse MLA launch");
}

}  // namespace

hs_status hs_sparse_mla_decode(const hs_layout* layout, const uint8_t* kv_layer,
                               const int32_t* row_ids, int32_t num_tokens, int32_t top_k,
                               const uint16_t* q, int32_t num_heads, float sm_scale, float* out,
                               float* lse, void* workspace, size_t workspace_bytes,
                               hipStream_t stream) {
  return sparse_mla_decode(layout, kv_layer, row_ids, num_tokens, top_k, q, num_heads, sm_scale,
                           out, lse, workspace, workspace_bytes, false, stream);
}

hs_status hs_sparse_mla_decode_noalloc(const hs_layout* layout, const uint8_t* kv_layer,
                                       const int32_t* row_ids, int32_t num_tokens,
                                       int32_t top_k, const uint16_t* q, int32_t num_heads,
                                       float sm_scale, float* out, float* lse,
                                       hipStream_t stream) {
  return sparse_mla_decode(layout, kv_layer, row_ids, num_tokens, top_k, q, num_heads, sm_scale,
                           out, lse, nullptr, 0, true, stream);
}

size_t hs_sparse_mla_noalloc_max_workspace(void) { return hs::kAttendScratchBytes; }

const char* hs_last_error(void) { return g_last_error; }

const char* hs_status_string(hs_status status) {
  switch (status) {
    case HS_OK: return "ok";
    case HS_ERR_INVALID_ARGUMENT: return "invalid argument";
    case HS_ERR_UNSUPPORTED: return "unsupported size (beyond the kernel limits)";
    case HS_ERR_LAUNCH: return "kernel launch failed";
    case HS_ERR_HIP: return "HIP runtime call failed";
    default: return "unknown status";
  }
}

hs_status hs_host_alloc(size_t bytes, void** host_ptr) {
  if (!host_ptr) return HS_ERR_INVALID_ARGUMENT;
  *host_ptr = nullptr;
  if (bytes == 0) return HS_ERR_INVALID_ARGUMENT;
  void* p = nullptr;
  if (hipHostMalloc(&p, bytes, hipHostMallocMapped | hipHostMallocPortable) != hipSuccess)
    return HS_ERR_HIP;
  *host_ptr = p;
  return HS_OK;
}

hs_status hs_host_free(void* host_ptr) {
  if (!host_ptr) return HS_OK;
  return hipHostFree(host_ptr) == hipSuccess ? HS_OK : HS_ERR_HIP;
}

hs_status hs_host_device_pointer(void* host_ptr, void** device_ptr) {
  if (!host_ptr || !device_ptr) return HS_ERR_INVALID_ARGUMENT;
  *device_ptr = nullptr;
  void* d = nullptr;
  if (hipHostGetDevicePointer(&d, host_ptr, 0) != hipSuccess) return HS_ERR_HIP;
  *device_ptr = d;
  return HS_OK;
}

}  // extern "C"
