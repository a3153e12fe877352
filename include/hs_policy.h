/*
 * hs_policy.h -- the host-side residency policy of Hybrid HiSparse: which
 * pages of each request stay in the GPU block pool, which become null
 * placeholders whose rows live only in the pinned host pool, which completed
 * pages are copied to host, and which pool blocks are leased to requests as
 * hot-buffer capacity.  It runs on the CPU between decode steps and never on
 * the decode path; its per-step edits are what the GPU path's block tables,
 * host tables and hot-block leases receive.
 *
 * Source: "vLLM GLM 5.3 ... Hybrid HiSparse offloading, Part 1":
 *   - "Use sparsity when needed" / "Offload only where needed": KV stays on
 *     the GPU while the pool has room; under pressure requests free their
 *     coldest pages in place, page by page, and the freed blocks become new
 *     tail pages and hot pages -- of any request;
 *   - "How it works": the tail of a request never leaves the GPU; hot pages
 *     are ordinary pool blocks, leased when a request first needs them and
 *     returned when it no longer does; completed cacheable prefix pages are
 *     copied to host ahead of pressure while still served from the GPU, so
 *     a page can later give up its block without another copy.
 *
 * Readings (the pages leave these open):
 *   - a page's coldness is the last step in which a top-K list of the
 *     request selected one of its tokens (0 = never); eviction takes the
 *     coldest eligible page first, ties broken by request, then page index;
 *   - a page is eligible for eviction when it is complete, outside the tail
 *     (the last tail_pages pages of the context, the page being written
 *     included) and its host copy was queued in an earlier step;
 *   - a request needs a hot lease exactly while one of its pages is a null
 *     placeholder; the lease is hot_blocks_per_request blocks, all or none;
 *   - the blocks a step frees are available to the same step's demand;
 *   - demand that the pool cannot meet even after every eligible eviction
 *     is an error (HS_POLICY_ERR_POOL_EXHAUSTED); after it, or after
 *     HS_POLICY_ERR_HOST_EXHAUSTED, the policy's state is unspecified and it
 *     must be destroyed.
 *
 * Host memory only; no HIP calls.  Not thread-safe: one caller per policy.
 */
#ifndef HS_POLICY_H_
#define HS_POLICY_H_

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef int32_t hs_policy_status;
#define HS_POLICY_OK 0
#define HS_POLICY_ERR_INVALID_ARGUMENT 1
#define HS_POLICY_ERR_POOL_EXHAUSTED 2   /* pages and leases need more blocks than the pool has */
#define HS_POLICY_ERR_HOST_EXHAUSTED 3   /* completed pages need more host blocks than exist */

typedef struct {
  int32_t page_size;               /* tokens per page, a power of two */
  int32_t num_blocks;              /* device blocks in the pool */
  int32_t num_host_blocks;         /* blocks in the pinned host pool */
  int32_t max_requests;            /* request slots 0..max_requests-1 */
  int32_t max_pages;               /* columns of the block tables */
  int32_t hot_blocks_per_request;  /* C / page_size */
  int32_t tail_pages;              /* resident tail, >= 1 */
} hs_policy_config;

typedef struct hs_policy hs_policy;

/* One step's edits, in caller-owned arrays sized by the caps; counts out.
 * Apply before the step: bt_set / hbt_set entries (request, page, value);
 * hot_set entries (request, index, block) for hs_batch.hot_blocks; the
 * requests in reset[] must have their hot-buffer state cleared (every slot
 * token -1, stamp 0, all layers) because their lease changed.  Apply after
 * the step: offload pairs (device block, host block), with
 * hs_offload_prefix_pages; those host copies become valid host-table entries
 * in the next step's hbt_set. */
typedef struct {
  int32_t* bt_set;   int32_t n_bt;   int32_t cap_bt;     /* [cap][3] */
  int32_t* hbt_set;  int32_t n_hbt;  int32_t cap_hbt;    /* [cap][3] */
  int32_t* hot_set;  int32_t n_hot;  int32_t cap_hot;    /* [cap][3] */
  int32_t* reset;    int32_t n_reset; int32_t cap_reset; /* [cap] */
  int32_t* offload;  int32_t n_offload; int32_t cap_offload; /* [cap][2] */
  int32_t evicted;   /* pages nulled this step */
  int32_t leased;    /* leases granted this step */
  int32_t returned;  /* leases returned this step */
} hs_policy_edits;

hs_policy_status hs_policy_create(const hs_policy_config* cfg, hs_policy** out);
void hs_policy_destroy(hs_policy* p);

/* Admits request `req` with `ctx_len` tokens.  Its pages [0, ctx/page) are
 * complete; host_block_of_page (may be NULL) gives an existing host copy per
 * complete page (-1 = none), e.g. a reused prefix.  Complete pages that have
 * a host copy start as null placeholders unless `resident_prefix`; all others
 * take pool blocks (resident).  The edits of admission are returned like a
 * step's (the block-table row, the host-table row, a lease if needed). */
hs_policy_status hs_policy_admit(hs_policy* p, int32_t req, int32_t ctx_len,
                                 const int32_t* host_block_of_page, int32_t resident_prefix,
                                 hs_policy_edits* edits);

/* Releases every block and host block of `req`; edits as for a step. */
hs_policy_status hs_policy_finish(hs_policy* p, int32_t req, hs_policy_edits* edits);

/* Prepares one decode step for the admitted requests in req[0..n): their
 * new context lengths ctx_len[i] (>= the previous), and the top-K tokens the
 * last executed step selected per request, topk[i][0..k) (-1 padding
 * ignored; may be NULL with k = 0), which make their pages warm at `stamp`.
 * Order: host copies queued last step become host-table entries; tokens
 * are appended (new pages take blocks); pressure evicts the coldest
 * eligible pages; leases are granted and returned; completed pages without
 * a host copy are queued for copy after the step. */
hs_policy_status hs_policy_step(hs_policy* p, int32_t stamp, const int32_t* req,
                                const int32_t* ctx_len, int32_t n, const int32_t* topk,
                                int32_t k, hs_policy_edits* edits);

/* hs_policy_step with page coldness given per page instead of as lists:
 * page_use[i * page_stride + page] is the last stamp at which a top-K list of
 * req[i] selected a token of that page (0 = never), as hs_page_touch writes
 * it on the GPU; a page's coldness becomes the later of its own and this
 * one.  Pages at or beyond page_stride keep their coldness.  Stamps here
 * and in hs_policy_step share one scale: use one form throughout.
 * page_use may be NULL when page_stride is 0. */
hs_policy_status hs_policy_step_pages(hs_policy* p, const int32_t* req, const int32_t* ctx_len,
                                      int32_t n, const uint32_t* page_use, int32_t page_stride,
                                      hs_policy_edits* edits);

/* Read-only views for tests: the policy's block table row, host table row
 * and lease of `req` (arrays of max_pages, max_pages, hot_blocks_per_request
 * entries), and the pool's free block count. */
hs_policy_status hs_policy_tables(const hs_policy* p, int32_t req, int32_t* bt, int32_t* hbt,
                                  int32_t* hot);
int32_t hs_policy_free_blocks(const hs_policy* p);

#ifdef __cplusplus
}
#endif

#endif  /* HS_POLICY_H_ */
