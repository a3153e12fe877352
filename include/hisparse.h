/*
 * hisparse.h -- C ABI of the MI355X (gfx950) Hybrid HiSparse hot path:
 * the fused sparse-MLA top-K resolver, the single-stride row gather, the
 * post-forward prefix-page offload and the replayable per-step plan.
 *
 * Source of the method: "vLLM GLM 5.3 ... Hybrid HiSparse offloading, Part 1"
 * (blog post, three renderings).  Sections cited:
 *   "How it works"            -- residency states, null placeholders, the
 *                                fused resolver, row ids, proactive copy,
 *                                one post-forward launch over all layers;
 *   "How it works" figure     -- a miss copies one row, a hit copies none;
 *   "Integration with the rest of vLLM" -- replayable resolve plans for
 *                                speculative decoding; 2 x top-K hot rows.
 *
 * General rules for every call below
 *   - Asynchronous: work is enqueued on the caller's HIP stream; nothing waits
 *     for the host ("nothing on the decode path waits on a CPU decision",
 *     "How it works").  No call allocates memory.
 *   - The caller owns every buffer.  Device pointers must come from hipMalloc
 *     (or a PyTorch CUDA tensor); the host pool must be pinned, device-mapped
 *     memory (hs_host_alloc) and is passed as its device-visible address.
 *   - The return value reports only what the host can check before any
 *     launch (null pointers, sizes, limits); on error nothing is enqueued.
 *     Data-dependent outcomes are reported per entry (sentinel row ids) and
 *     per request-layer (the stats record), never through the return value.
 *   - Calls on disjoint state may run concurrently; calls that share state
 *     (slot_token / slot_stamp / pool rows / fill_sync) must be ordered by
 *     the caller.
 *
 * Data layout (all little-endian, all row ids int32):
 *   kv_pool    uint8 [L][pool_rows][row_bytes], layer l at l * pool_layer_stride
 *              bytes.  Row id = block * page_size + offset, the same id in every
 *              layer.  Resident pages and hot pages live in this one pool.
 *   host_pool  uint8 [L][host_rows][row_bytes], layer stride host_layer_stride.
 *   block_table, host_block_table   int32 [R][max_pages]; entry < 0 = null
 *              placeholder / no host copy.
 *   ctx_len    int32 [R]: tokens 0..ctx-1 are valid.
 *   hot_blocks int32 [R][C / page_size]: the pool blocks leased as the
 *              request's hot buffer; slot q lives at row
 *              hot_blocks[q / page_size] * page_size + q % page_size.
 *   slot_token int32  [R][L][C]: token held by each slot, < 0 = empty.
 *   slot_stamp uint32 [R][L][C]: LRU stamp of each slot, 0 = never used.
 *   topk       int32 [R][L][P][K] (P = 1 for hs_resolve); -1 = padding.
 *   row_ids    int32, same shape as topk:  >= 0 pool row;  -1 padding;
 *              -2 overflow (no usable hot slot left for the miss: never when
 *              P = 1 and C >= K with every hot block usable);
 *              -3 invalid (outside [0, ctx), or neither resident nor on host).
 *   stats      int32 [R][L][8] = {resident, hit, miss, overflow, invalid,
 *              pad, dup, 0}; the first five count distinct tokens, pad and
 *              dup count entries; they always sum to P * K.
 *   gather_out uint8 [R][L][P][K][row_bytes].
 *   kv_pool, host_pool, gather_out and the staging buffer start on 16-byte
 *   boundaries, and with L > 1 both layer strides are multiples of 16 (the
 *   kernels move 16-byte pieces); otherwise HS_ERR_INVALID_ARGUMENT.
 */
#ifndef HISPARSE_H
#define HISPARSE_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef int32_t hs_status;
#define HS_OK 0
#define HS_ERR_INVALID_ARGUMENT 1 /* a null pointer, a size out of range */
#define HS_ERR_UNSUPPORTED 2      /* valid, but beyond this build's kernel limits */
#define HS_ERR_LAUNCH 3           /* the HIP runtime refused a launch */
#define HS_ERR_HIP 4              /* another HIP runtime call failed */

/* Limits of the resolver kernel (one workgroup per request-layer, state in LDS). */
#define HS_MAX_ENTRIES 8192       /* P * K per request-layer */
#define HS_MAX_HOT_CAPACITY 12288 /* C: up to (speculative tokens + 2) x 2048 for 4 tokens */
#define HS_MAX_ROW_BYTES 4096     /* row_bytes for the resolving calls (656 here) */

typedef struct {
  int32_t page_size;          /* tokens per page: a power of two, 1..4096 (64 here) */
  int32_t row_bytes;          /* bytes per KV row: a positive multiple of 16 (656 here);
                                 the resolving calls take at most HS_MAX_ROW_BYTES */
  int32_t num_layers;         /* L >= 1 */
  int32_t hot_capacity;       /* C: hot slots per request-layer, a multiple of page_size */
  int64_t pool_rows;          /* rows per layer in kv_pool: multiple of page_size, < 2^31 */
  int64_t host_rows;          /* rows per layer in host_pool: multiple of page_size, < 2^31 */
  int64_t pool_layer_stride;  /* bytes between layers of kv_pool, >= pool_rows * row_bytes */
  int64_t host_layer_stride;  /* bytes between layers of host_pool, >= host_rows * row_bytes */
} hs_layout;

typedef struct {
  int32_t num_reqs;                 /* R >= 0 */
  int32_t max_pages;                /* columns of both block tables, >= 1 */
  uint8_t* kv_pool;                 /* device; hot-slot rows are written */
  const uint8_t* host_pool;         /* pinned host pool, device-visible address */
  const int32_t* block_table;       /* device [R][max_pages] */
  const int32_t* host_block_table;  /* device [R][max_pages] */
  const int32_t* ctx_len;           /* device [R] */
  const int32_t* hot_blocks;        /* device [R][C / page_size] */
  int32_t* slot_token;              /* device [R][L][C], read and updated */
  uint32_t* slot_stamp;             /* device [R][L][C], read and updated */
  int32_t* fill_sync;               /* device [fill_sync_words], or NULL (see below) */
  int32_t fill_sync_words;          /* int32 words at fill_sync: >= HS_FILL_SYNC_WORDS, 0 with NULL */
} hs_batch;

/*
 * fill_sync -- optional work counters of the early fill's miss workgroups.
 * With more (request-layer, split) items than miss workgroups, a non-NULL
 * fill_sync lets each workgroup take its next item from a counter as it
 * finishes the last one (the host link serves the chip's XCDs at different
 * rates, so a fixed share per workgroup ends with the slowest); NULL keeps
 * the fixed share.  The words must be zero before the first call that uses
 * them; every call leaves them zero again (the last miss workgroup to finish
 * clears them), so one zeroed allocation serves a batch's calls for good.
 * fill_sync_words gives the allocation's size, which the call checks (fewer
 * than HS_FILL_SYNC_WORDS, or words without a pointer: invalid argument).
 * They are state like slot_token: calls that share a fill_sync must be
 * ordered by the caller.  Results do not depend on fill_sync.
 */
#define HS_FILL_SYNC_WORDS 64

/*
 * hs_resolve -- the fused top-K resolver ("How it works": mixed residency;
 * the figure's solid and dotted arrows).  For every request r and layer l,
 * resolves the K entries topk[r][l][*] to pool rows:
 *   - a token whose page has a real block-table entry is read in place:
 *     row = block * page_size + token % page_size; the hot buffer is not
 *     consulted;
 *   - the distinct remaining tokens are looked up in the request-layer's hot
 *     buffer; a hit refreshes the slot's stamp to `stamp`, copies nothing;
 *   - the distinct misses (tokens with a host copy, not in the buffer), in
 *     ascending token order, take the non-hit slots in ascending
 *     (stamp, slot) order -- least recently used first, empty slots first --
 *     and each copies exactly one row from host_pool into its slot, which then
 *     holds the token with stamp `stamp`;
 *   - all decisions read the state as it was before the call.
 * Slots whose hot block lies outside the pool are never used; block-table,
 * host-table and pair entries outside their pools are treated as absent.
 * Precondition: a leased hot block belongs to one request only and is not
 * also a resident block in any block table (otherwise the rows a copy writes
 * and the rows a gather reads may overlap within one call).
 * Arguments: top_k = K (1..HS_MAX_ENTRIES); stamp > 0, normally the step
 * counter (calling again with the same inputs and the same stamp leaves the
 * state unchanged); gather_out may be NULL, otherwise it receives the rows
 * gathered after every copy of this call (as hs_gather would).
 * Execution: all on `stream`.  With a gather_out, one launch carries the
 * resolver's workgroups and those of an early fill that writes every output
 * row from the pre-call state (the misses' host rows included) while the
 * resolver works; a short commit kernel then fills the assigned hot slots
 * from the output.
 * Errors: HS_ERR_INVALID_ARGUMENT (null pointer, stamp 0, bad layout),
 * HS_ERR_UNSUPPORTED (K or C over the limits), HS_ERR_LAUNCH.
 */
hs_status hs_resolve(const hs_layout* layout, const hs_batch* batch, const int32_t* topk,
                     int32_t top_k, uint32_t stamp, int32_t* row_ids, uint8_t* gather_out,
                     int32_t* stats, hipStream_t stream);

/*
 * hs_gather -- the single-stride gather ("How it works": the resolver hands
 * back a row id whether the row is resident or hot, and the rows are gathered
 * at one stride).  out[r][l][i] = kv_pool[l][row_ids[r][l][i]] (row_bytes
 * bytes); a row id < 0 or >= pool_rows yields a zero row.
 * Arguments: kv_pool device; row_ids device int32 [num_reqs][L][rows_per_req_layer];
 * out device uint8 [num_reqs][L][rows_per_req_layer][row_bytes].
 * Errors: HS_ERR_INVALID_ARGUMENT, HS_ERR_LAUNCH.
 */
hs_status hs_gather(const hs_layout* layout, const uint8_t* kv_pool, const int32_t* row_ids,
                    int32_t num_reqs, int32_t rows_per_req_layer, uint8_t* out,
                    hipStream_t stream);

/*
 * hs_offload_prefix_pages -- the post-forward batched prefix copy ("How it
 * works": completed cacheable prefix pages are copied to host while still
 * served from the GPU, in one launch over all sparse layers, ordered on the
 * model's stream).  For each pair i and every layer l, copies the
 * page_size rows of device block pairs[i][0] to host block pairs[i][1].
 * Pairs naming a block outside either pool are skipped.  Host blocks must be
 * distinct within one call.  Stream-later work may reuse the device block at
 * once; host readers must wait for the stream (an event or a sync).
 * Arguments: pairs device int32 [n][2] = {device block, host block}; n >= 0.
 * Errors: HS_ERR_INVALID_ARGUMENT, HS_ERR_LAUNCH.
 */
hs_status hs_offload_prefix_pages(const hs_layout* layout, const uint8_t* kv_pool,
                                  uint8_t* host_pool, const int32_t* pairs, int32_t n,
                                  hipStream_t stream);

/*
 * hs_plan_replay -- a per-step replayable resolve plan for speculative decoding
 * ("Integration with the rest of vLLM": one plan per step sharing the
 * request's hot state).  The P query positions of each request-layer are
 * resolved as one list of P * K entries with one stamp commit (a token shared
 * by several positions is resolved once and every position gets its row);
 * then the optional gather, then the optional prefix offload of
 * offload_pairs[n_offload][2] -- all on `stream`, in that order.
 * num_pos = 1 with no offload is exactly hs_resolve.  Misses beyond the
 * free slots overflow (row -2) and leave the state untouched for them.
 * Errors: as hs_resolve; P * K over HS_MAX_ENTRIES is HS_ERR_UNSUPPORTED.
 */
hs_status hs_plan_replay(const hs_layout* layout, const hs_batch* batch, const int32_t* topk,
                         int32_t num_pos, int32_t top_k, uint32_t stamp, int32_t* row_ids,
                         uint8_t* gather_out, int32_t* stats, const int32_t* offload_pairs,
                         int32_t n_offload, hipStream_t stream);

/*
 * hs_resolve_grouped -- the resolve for layers that share a top-K list
 * ("Use sparsity when needed": GLM 5.3's IndexShare places one indexer layer
 * per 4 sparse-MLA layers, so those layers attend to the same tokens).  The
 * layout's L layers form L / G groups of G consecutive layers; each group of
 * a request has one top-K list and one hot-buffer state.  The decisions are
 * made once per group, exactly as hs_plan_replay makes them for one layer;
 * every copy into a slot is made in each of the group's layers (each layer's
 * own host row into its own slot row), and every layer of a group receives
 * the group's rows.  G = 1 is hs_plan_replay.
 * Arguments: group_layers = G >= 1, dividing layout->num_layers; the batch's
 * slot_token and slot_stamp are [R][L/G][C]; topk and row_ids are
 * [R][L/G][P*K]; stats [R][L/G][8]; gather_out (may be NULL)
 * [R][L][P*K][row_bytes], gather_out[r][l][i] from layer l's pool plane at
 * row_ids[r][l/G][i]; the offload pairs copy every layer, as in
 * hs_plan_replay.
 * Errors: as hs_plan_replay; G not dividing L is HS_ERR_INVALID_ARGUMENT.
 */
hs_status hs_resolve_grouped(const hs_layout* layout, const hs_batch* batch, int32_t group_layers,
                             const int32_t* topk, int32_t num_pos, int32_t top_k, uint32_t stamp,
                             int32_t* row_ids, uint8_t* gather_out, int32_t* stats,
                             const int32_t* offload_pairs, int32_t n_offload, hipStream_t stream);

/*
 * The stages of hs_resolve / hs_plan_replay, for callers that time or
 * schedule them on their own streams.
 *
 * Serial form (what the calls do without a gather output):
 *   hs_resolve_decide(layout, batch, topk, P, K, stamp, row_ids, NULL, stats, s);
 *   hs_resolve_move(layout, batch, topk, P, K, row_ids, gather_out, s);
 * Overlapped form (what the calls do with one):
 *   hs_resolve_decide(layout, batch, topk, P, K, stamp, row_ids, gather_out, stats, s);
 *   hs_resolve_commit(layout, batch, topk, P, K, row_ids, gather_out, s);
 * or, scheduled by the caller on two streams:
 *   s2: hs_resolve_decide(..., NULL, stats, s2);
 *   s:  hs_resolve_fetch(layout, batch, topk, P, K, gather_out, s);
 *       <wait for decide>  hs_resolve_commit(layout, batch, topk, P, K, row_ids,
 *                                            gather_out, s);
 * fetch and decide must start after every earlier change to the batch's
 * state, tables and pools, and both finish before commit; they may overlap.
 *
 * decide runs one workgroup per request-layer: it classifies, finds hits and
 * victims and writes the stamps; row_ids then hold final rows except for the
 * misses: -(8 + 2 * slot + c) for a miss assigned to a slot (c = 1 on the
 * token's first entry, which fills the slot) and -2 for a miss left without
 * one.  The victims' new tokens are recorded by the entry that fills the
 * slot, in move (serial) or commit (overlapped), so slot_token still holds
 * the pre-call tokens until then.  With a gather_out, the same launch also
 * carries fetch's workgroups.
 * move runs on the whole chip: it copies each missed row from the host pool
 * into its slot, gathers every row into gather_out (NULL: copies only) and
 * replaces the codes by the slots' row ids.
 * fetch writes every entry's row of gather_out from the pre-call state, as
 * decide classifies it: resident and hot rows from kv_pool, a miss's row from
 * the host pool (read once per distinct token), zero rows otherwise -- a
 * miss left without a slot included, until commit.  It writes nothing else.
 * commit copies each assigned miss's row from gather_out into its slot,
 * records the slot's token, replaces the codes by row ids, and zeroes the
 * rows of misses left without a slot.
 * Until the last stage has run, the hot slots of the misses do not hold
 * their rows.  Errors: as hs_resolve; fetch and commit need a gather_out
 * (HS_ERR_INVALID_ARGUMENT).
 */
hs_status hs_resolve_decide(const hs_layout* layout, const hs_batch* batch, const int32_t* topk,
                            int32_t num_pos, int32_t top_k, uint32_t stamp, int32_t* row_ids,
                            uint8_t* gather_out, int32_t* stats, hipStream_t stream);
hs_status hs_resolve_fetch(const hs_layout* layout, const hs_batch* batch, const int32_t* topk,
                           int32_t num_pos, int32_t top_k, uint8_t* gather_out,
                           hipStream_t stream);
hs_status hs_resolve_move(const hs_layout* layout, const hs_batch* batch, const int32_t* topk,
                          int32_t num_pos, int32_t top_k, int32_t* row_ids, uint8_t* gather_out,
                          hipStream_t stream);
hs_status hs_resolve_commit(const hs_layout* layout, const hs_batch* batch, const int32_t* topk,
                            int32_t num_pos, int32_t top_k, int32_t* row_ids,
                            uint8_t* gather_out, hipStream_t stream);

/*
 * hs_page_touch -- page coldness for the host-side residency policy ("Use
 * sparsity when needed": under pressure a request gives up its coldest
 * pages first).  For every request r < batch->num_reqs and every entry
 * t = topk[r * entries_per_req + e], e < entries_per_req, with
 * 0 <= t < ctx_len[r] and t / page_size < max_pages:
 *   page_use[r * max_pages + t / page_size] = stamp.
 * Every other word of page_use (device [R][max_pages], caller-owned) keeps
 * its value.  topk is device memory, any [R][...] list layout flattened per
 * request (e.g. [R][L][P][K] with entries_per_req = L * P * K, or one group
 * list per layer group); padding (-1) and out-of-range entries stamp
 * nothing.  Uses batch->num_reqs, max_pages and ctx_len only.  Enqueue it
 * after a step's resolve on the same stream and copy page_use to host when
 * the policy runs (hs_policy_step_pages reads it), so the policy never reads
 * the lists themselves.  Any stamp value is stored as given.
 * Errors: HS_ERR_INVALID_ARGUMENT (null pointer with work to do, negative
 * sizes, bad layout), HS_ERR_UNSUPPORTED (entries_per_req over 67,107,840),
 * HS_ERR_LAUNCH.
 */
hs_status hs_page_touch(const hs_layout* layout, const hs_batch* batch, const int32_t* topk,
                        int32_t entries_per_req, uint32_t stamp, uint32_t* page_use,
                        hipStream_t stream);

/*
 * hs_resolve_in_place -- hs_plan_replay for consumers that read the rows in
 * place by row id (hs_sparse_mla_decode): the same row ids, stats, hot-buffer
 * state, pool and offload as hs_plan_replay with gather_out = NULL, but the
 * misses' host reads run while the resolver decides, as in the overlapped
 * form, staged through `staging` instead of a gathered output: no resident
 * or hot row is copied anywhere.
 * staging: device [R][L][P][K][row_bytes], caller-owned scratch; only the
 * rows of missed tokens' first entries (and of misses left without a slot)
 * are written, its contents afterwards are unspecified.
 * Errors: as hs_plan_replay; a NULL staging is HS_ERR_INVALID_ARGUMENT.
 */
hs_status hs_resolve_in_place(const hs_layout* layout, const hs_batch* batch, const int32_t* topk,
                              int32_t num_pos, int32_t top_k, uint32_t stamp, int32_t* row_ids,
                              uint8_t* staging, int32_t* stats, const int32_t* offload_pairs,
                              int32_t n_offload, hipStream_t stream);

/*
 * hs_sparse_mla_decode -- gather-free consumption of the resolved rows: sparse
 * MLA decode attention that reads every selected row in place, by the row
 * id the resolver returned ("Use sparsity when needed": hot pages live in the
 * same KV-cache tensor as resident pages, so the sparse MLA kernel sees them
 * as ordinary pages; "How it works": one row id whether resident or hot).
 * No gathered copy of the rows is made.
 * Row format (layout->row_bytes must be 656, else HS_ERR_UNSUPPORTED): 512
 * latent values in OCP FP8 E4M3, then 4 little-endian float32 scales (scale
 * t for latent values [128 t, 128 t + 128)), then 64 rope values in
 * bfloat16.  A row's key is its scaled latent values followed by its rope
 * values (576); its value is the scaled latent values (512).
 * For token i < num_tokens and head h < num_heads:
 *   s_j = sm_scale * <q[i][h], key(row_ids[i][j])> over j < top_k whose row id
 *         lies in [0, layout->pool_rows) (others select nothing);
 *   out[i][h] = sum_j softmax(s)_j value(row_ids[i][j]);
 *   lse[i][h] = log(sum_j exp(s_j)) (natural log); out 0 and lse -inf when
 *   no row is selected.
 * Arguments: kv_layer = one layer of the pool (device, 16-byte aligned; add
 * the layer stride to kv_pool); row_ids device [num_tokens][top_k] (e.g. a
 * plan's [R][P][K] row ids for one layer, tokens = R * P); q device bf16
 * [num_tokens][num_heads][576]; out device float [num_tokens][num_heads][512];
 * lse device float [num_tokens][num_heads]; num_heads a multiple of 16;
 * workspace: device memory of at least hs_sparse_mla_workspace_bytes(...)
 * bytes, 16-byte aligned (may be NULL when that is 0), overwritten.
 * Precision: keys and values are used exactly (E4M3 values are bfloat16
 * values; the scales are applied in float32), products accumulate in
 * float32, the probabilities times the value scales are rounded to bfloat16
 * for the value products; where the rows are split across workgroups, each
 * split's normalised output is kept in half precision (a relative 2^-11)
 * until the splits are merged in float32.
 * Execution: all on `stream`; calls sharing a workspace must not overlap.
 * Errors: HS_ERR_INVALID_ARGUMENT (null or misaligned pointers with work to
 * do, a short workspace, num_heads not a positive multiple of 16, negative
 * sizes, bad layout), HS_ERR_UNSUPPORTED (row_bytes != 656, more than 65535
 * tokens, top_k over 131,072), HS_ERR_LAUNCH.
 */
hs_status hs_sparse_mla_decode(const hs_layout* layout, const uint8_t* kv_layer,
                               const int32_t* row_ids, int32_t num_tokens, int32_t top_k,
                               const uint16_t* q, int32_t num_heads, float sm_scale, float* out,
                               float* lse, void* workspace, size_t workspace_bytes,
                               hipStream_t stream);

/* Bytes of workspace hs_sparse_mla_decode needs for these sizes (0 when it
 * needs none, or for non-positive sizes). */
size_t hs_sparse_mla_workspace_bytes(int32_t num_tokens, int32_t num_heads, int32_t top_k);

/*
 * hs_sparse_mla_decode_noalloc -- hs_sparse_mla_decode for callers that
 * cannot allocate device memory at all (code under HIP graph capture, tight
 * serving loops, harnesses that forbid hipMalloc): the same computation and
 * results, with the key splits' partial outputs in a workspace the library
 * holds in device memory instead of a caller buffer.  It calls no
 * allocating routine of any kind.
 * Workspace: one array of hs_sparse_mla_noalloc_max_workspace() bytes
 * (64 MiB) per device, a static part of the library's code object that each
 * GPU the library runs on holds until the process ends; its device address
 * is looked up once per device, on the first call that needs it.  Calls whose
 * hs_sparse_mla_workspace_bytes(num_tokens, num_heads, top_k) exceeds it
 * return HS_ERR_UNSUPPORTED before enqueuing anything (the decode shape, 32
 * tokens x 128 heads x 2048 rows, needs about 17 MB).
 * Concurrency: every call on one device shares that device's array and
 * overwrites it; calls that overlap in time on one device (other streams,
 * other threads) race and must be ordered by the caller.  Nothing in the
 * array needs to start at zero: each call writes every part it reads.
 * Arguments, precision and other errors: as hs_sparse_mla_decode; a failed
 * address lookup is HS_ERR_HIP.
 */
hs_status hs_sparse_mla_decode_noalloc(const hs_layout* layout, const uint8_t* kv_layer,
                                       const int32_t* row_ids, int32_t num_tokens,
                                       int32_t top_k, const uint16_t* q, int32_t num_heads,
                                       float sm_scale, float* out, float* lse,
                                       hipStream_t stream);

/* The size of hs_sparse_mla_decode_noalloc's per-device workspace, bytes. */
size_t hs_sparse_mla_noalloc_max_workspace(void);

/* A static English description of a status code. */
const char* hs_status_string(hs_status status);

/* The HIP runtime failure behind the last HS_ERR_LAUNCH or HS_ERR_HIP
 * returned on the calling thread: "<what>: <hipError name> (<code>)", or ""
 * if there was none.  The text is owned by the library and stays valid
 * until the thread's next failing call. */
const char* hs_last_error(void);

/* Pinned host memory for the host pool, mapped into the device address space.
 * *host_ptr is the host address; hs_host_device_pointer gives the address
 * kernels use (equal on ROCm, but callers should not rely on that).
 * Errors: HS_ERR_INVALID_ARGUMENT (null out-pointer), HS_ERR_HIP. */
hs_status hs_host_alloc(size_t bytes, void** host_ptr);
hs_status hs_host_free(void* host_ptr);
hs_status hs_host_device_pointer(void* host_ptr, void** device_ptr);

#ifdef __cplusplus
}
#endif

#endif /* HISPARSE_H */
