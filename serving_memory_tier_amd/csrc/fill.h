// Device code of the early fill (gfx950), shared by the fused resolve kernel
// (resolve.hip: the fill's workgroups run in the same launch as the
// resolver's) and the stand-alone fill kernel (fetch.hip).
//
// Method: "vLLM GLM 5.3 ... Hybrid HiSparse offloading, Part 1", section
// "How it works": a resident token's row is read in place through the block
// table, a hot token's from its slot, and a miss's row comes over the host
// link from pinned host memory; the rows of a request are gathered at one
// stride.  None of these rows depends on the LRU order: resident blocks and
// the slots of hits are never written by the step (victims are non-hit
// slots), and a miss's row is the host row whichever slot it gets.  So the
// whole gather -- host-link reads included -- can start at once and run
// while the resolver works; afterwards a short commit kernel copies each
// assigned miss's row from the output into its slot, records the slot's
// token, turns the codes into row ids and zeroes the rows of misses left
// without a slot.
//
// Two kinds of fill workgroup classify entries the same way (the block
// tables, then whether a usable hot slot holds the token):
//   * gather workgroups (several per request-layer, a range of entries each)
//     write every row but the misses': resident and hot rows from the pool,
//     zero rows for padded and invalid entries and tokens without a host copy
//     (an LDS map of the range's non-resident tokens, probed by every slot,
//     gives each hit its slot);
//   * miss workgroups (a fixed few for the whole launch) classify every entry
//     of a request-layer, deduplicate the misses and read each distinct
//     missed token's row once from the host into one of its entries, then
//     copy it to the token's other entries (the hits come from a bitmap of
//     the slots' tokens where it fits, else from the slots probing an LDS map
//     of the host-backed entries).  With several per request-layer,
//     workgroup s owns the tokens t with t mod S == s; with the batch's
//     fill_sync counters, a workgroup done with its (request-layer, split)
//     item takes the next one not yet taken.
// Keeping the host reads to a few workgroups bounds how many are in flight:
// the link saturates with a few tens of thousands of 16-byte reads
// outstanding, and more only hold back the HBM reads of the rest of the
// chip, which share the memory system's queues with them.
//
// Bound: the host link (PCIe 5.0 x16) while misses are in flight; HBM
// otherwise.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "hs_internal.h"

// Timing hooks (per-workgroup timestamps), empty unless a profiling build
// defines them; negative indices mark steps inside the miss workgroups.
#ifndef HS_FILL_MARK
#define HS_FILL_MARK(i)
#endif

namespace hs {
namespace fill {
namespace {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

constexpr int kT = kFillThreads;
constexpr int kU = kCopyUnroll;

// n / pieces for the piece counters of one row size: (n * magic) >> 32 with
// magic = ceil(2^32 / pieces) is exact for n < 2^32 / pieces (magic * pieces
// exceeds 2^32 by less than pieces), above any piece count here: entries
// <= 8192 and pieces <= 256 (rows of at most 4096 bytes) give n < 2^21,
// against a bound of 2^24.  One piece a row (16-byte rows) would need magic
// 2^32, which a 32-bit word does not hold: magic 0 stands for it.
__device__ __forceinline__ int32_t pdiv(int32_t n, uint32_t magic) {
  return magic == 0 ? n : (int32_t)(((uint64_t)(uint32_t)n * magic) >> 32);
}

// The token map: an open-addressing table (linear probing) over the tokens
// of the non-resident entries.  A word holds (first entry << 16) | slot: the
// smallest entry index holding the token -- its key is keys[entry] -- and the
// smallest usable hot slot holding it, kNoSlot if none.  Entries are
// inserted first (atomicMin over whole words of the same token keeps the
// smallest entry, since the slot half is still kNoSlot); after a barrier the
// hot buffer's slots probe the table and lower the slot half with atomicMin
// (the entry half of a claimed word never changes).  The table holds at most
// two thirds as many keys as words (a half or less but at the largest
// sizes), and the slots' probes mostly end at an empty word at once.
constexpr uint32_t kEmptyWord = 0xFFFFFFFFu;
constexpr uint32_t kNoSlot = 0xFFFFu;

__device__ __forceinline__ int32_t home(uint32_t key, int32_t n) {
  return (int32_t)(((uint64_t)(key * 0x9E3779B1u) * (uint32_t)n) >> 32);
}

__device__ __forceinline__ int32_t next(int32_t h, int32_t n) { return h + 1 == n ? 0 : h + 1; }

__device__ void map_insert(uint32_t* tab, int32_t n, const int32_t* keys, int32_t t, int32_t e) {
  const uint32_t w = ((uint32_t)e << 16) | kNoSlot;
  int32_t h = home((uint32_t)t, n);
  while (true) {
    const uint32_t old = atomicCAS(&tab[h], kEmptyWord, w);
    if (old == kEmptyWord) return;
    if (keys[old >> 16] == t) {
      atomicMin(&tab[h], w);
      return;
    }
    h = next(h, n);
  }
}

// Claims token t's word for entry e: -1 when e claimed it, otherwise the
// entry that did (the word is not lowered afterwards).
__device__ int32_t map_claim(uint32_t* tab, int32_t n, const int32_t* keys, int32_t t, int32_t e) {
  const uint32_t w = ((uint32_t)e << 16) | kNoSlot;
  int32_t h = home((uint32_t)t, n);
  while (true) {
    const uint32_t old = atomicCAS(&tab[h], kEmptyWord, w);
    if (old == kEmptyWord) return -1;
    if (keys[old >> 16] == t) return (int32_t)(old >> 16);
    h = next(h, n);
  }
}

// The table index holding token t, or -1.
__device__ int32_t map_find(const uint32_t* tab, int32_t n, const int32_t* keys, int32_t t) {
  int32_t h = home((uint32_t)t, n);
  while (true) {
    const uint32_t w = tab[h];
    if (w == kEmptyWord) return -1;
    if (keys[w >> 16] == t) return h;
    h = next(h, n);
  }
}

// The hot buffer's usable slots lower the slot half of their token's word.
// The first kT * kScanUnroll slots come prefetched from the workgroup's
// start (`pre`); for the others a slot's hot block is read only when its
// token is in the table.  Only slots whose token t has t mod S == s look
// (the table holds only such tokens).  Ends with a barrier.
constexpr int kScanUnroll = 4;

// The first kT * kScanUnroll slots' tokens, already masked to -1 where the
// slot's hot block is not a usable pool block.
__device__ __forceinline__ void prefetch_slots(const FetchParams& p, int32_t rl,
                                               int32_t (&pre)[kScanUnroll]) {
  const int32_t C = p.hot_capacity;
  const int ps = p.page_shift;
  const int64_t pool_blocks = p.pool_rows >> ps;
  const int32_t r = rl / p.num_layers;
  const int32_t* stok = p.slot_token + (int64_t)rl * C;
  const int32_t* hot = p.hot_blocks + (int64_t)r * (C >> ps);
  int32_t hb[kScanUnroll];
#pragma unroll
  for (int u = 0; u < kScanUnroll; ++u) {
    const int32_t q = u * kT + (int32_t)threadIdx.x;
    pre[u] = q < C ? stok[q] : -1;
    hb[u] = q < C ? hot[q >> ps] : -1;
  }
#pragma unroll
  for (int u = 0; u < kScanUnroll; ++u)
    if (hb[u] < 0 || hb[u] >= pool_blocks) pre[u] = -1;
}

__device__ void scan_slots(const FetchParams& p, int32_t rl, uint32_t* tab, int32_t n,
                           const int32_t* keys, const int32_t (&pre)[kScanUnroll], int32_t s = 0,
                           int32_t S = 1) {
  const int tid = threadIdx.x;
  const int32_t C = p.hot_capacity;
  const int ps = p.page_shift;
  const int64_t pool_blocks = p.pool_rows >> ps;
  const int32_t r = rl / p.num_layers;
  const int32_t* stok = p.slot_token + (int64_t)rl * C;
  const int32_t* hot = p.hot_blocks + (int64_t)r * (C >> ps);
  for (int32_t q0 = 0; q0 < C; q0 += kT * kScanUnroll) {
    int32_t tq[kScanUnroll], h[kScanUnroll];
    const bool first = q0 == 0;  // the prefetched slots, already masked
#pragma unroll
    for (int u = 0; u < kScanUnroll; ++u) {
      const int32_t q = q0 + u * kT + tid;
      tq[u] = first ? pre[u] : q < C ? stok[q] : -1;
    }
#pragma unroll
    for (int u = 0; u < kScanUnroll; ++u)
      h[u] = tq[u] >= 0 && (S == 1 || tq[u] % S == s) ? map_find(tab, n, keys, tq[u]) : -1;
#pragma unroll
    for (int u = 0; u < kScanUnroll; ++u) {
      if (h[u] < 0) continue;
      const int32_t q = q0 + u * kT + tid;
      if (!first) {
        const int32_t hb = hot[q >> ps];
        if (hb < 0 || hb >= pool_blocks) continue;
      }
      atomicMin(&tab[h[u]], (tab[h[u]] & 0xFFFF0000u) | (uint32_t)q);
    }
  }
  __syncthreads();
}

// Appends `take` lanes' items to an LDS list, one LDS atomic per wave.
__device__ __forceinline__ int32_t wave_append(int32_t* counter, bool take) {
  const uint64_t m = __ballot(take);
  if (m == 0) return -1;
  const int lane = threadIdx.x & 63;
  const int leader = __ffsll((unsigned long long)m) - 1;
  int32_t base = 0;
  if (lane == leader) base = atomicAdd(counter, __popcll(m));
  base = __shfl(base, leader);
  const int32_t rank = __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32),
                                                 __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
  return take ? base + rank : -1;
}

// Row sources in LDS: >= 0 a pool row, kZeroRow a zero row, kSkip a row
// another workgroup writes, kNoHost (before the slot scan) a non-resident
// entry without a host copy, otherwise a non-resident entry with one whose
// host row r is stored as r | 0x80000000 (host rows are < 2^31 - 1, so it
// never reads as one of the markers).
constexpr int32_t kZeroRow = -1;
constexpr int32_t kSkip = -2;
constexpr int32_t kNoHost = -3;
constexpr uint32_t kHostTag = 0x80000000u;

__device__ __forceinline__ bool is_host_row(int32_t v) { return v < kNoHost; }
__device__ __forceinline__ bool non_resident(int32_t v) { return v == kNoHost || is_host_row(v); }

// A request-layer's (or a layer group's) pointers and sizes.  With layer
// groups, rl counts (request, group) pairs; pool_l, host_l and out address
// the group's first layer, the next layers follow at the strides.
struct Rl {
  int32_t N, ps, pm, pieces, ctx, group;
  uint32_t magic;
  int64_t pool_blocks, host_blocks;
  int64_t pool_stride, host_stride, out_stride;
  const int32_t *topk, *bt, *hbt, *hot;
  const uint8_t *pool_l, *host_l;
  uint8_t* out;
};

__device__ __forceinline__ Rl rl_view(const FetchParams& p, int32_t rl) {
  Rl v;
  const int32_t r = rl / p.num_layers;
  const int32_t l0 = (rl - r * p.num_layers) * p.group;
  v.N = p.entries;
  v.ps = p.page_shift;
  v.pm = (1 << v.ps) - 1;
  v.pieces = p.row_bytes >> 4;
  v.group = p.group;
  v.magic = p.piece_magic;
  v.pool_blocks = p.pool_rows >> v.ps;
  v.host_blocks = p.host_rows >> v.ps;
  v.pool_stride = p.pool_stride;
  v.host_stride = p.host_stride;
  v.out_stride = (int64_t)v.N * p.row_bytes;
  v.topk = p.topk + (int64_t)rl * v.N;
  v.bt = p.block_table + (int64_t)r * p.max_pages;
  v.hbt = p.host_block_table + (int64_t)r * p.max_pages;
  v.hot = p.hot_blocks + (int64_t)r * (p.hot_capacity >> v.ps);
  v.pool_l = p.pool + (int64_t)l0 * p.pool_stride;
  v.host_l = p.host + (int64_t)l0 * p.host_stride;
  v.out = p.out + ((int64_t)r * p.layers + l0) * v.out_stride;
  v.ctx = p.ctx_len[r];
  return v;
}

// Entries e0 + u * kT + tid (< lim): the tokens, -1 for padded and invalid
// entries.
__device__ __forceinline__ void load_tokens(const FetchParams& p, const Rl& v, int32_t e0,
                                            int32_t lim, int32_t (&t)[kU]) {
  const int tid = threadIdx.x;
#pragma unroll
  for (int u = 0; u < kU; ++u) {
    const int32_t e = e0 + u * kT + tid;
    t[u] = e < lim ? v.topk[e] : -1;
    if (t[u] >= v.ctx || (t[u] >> v.ps) >= p.max_pages) t[u] = -1;
  }
}

// The row source of each token before the hot-buffer lookup: a resident row,
// kZeroRow, kNoHost or a tagged host row.  The block-table and host-table
// loads are issued together.
__device__ __forceinline__ void classify_tokens(const Rl& v, const int32_t* bt,
                                                const int32_t* hbt, const int32_t (&t)[kU],
                                                int32_t (&src)[kU]) {
  int32_t b[kU], hb[kU];
#pragma unroll
  for (int u = 0; u < kU; ++u) {
    b[u] = t[u] >= 0 ? bt[t[u] >> v.ps] : 0;
    hb[u] = t[u] >= 0 ? hbt[t[u] >> v.ps] : -1;
  }
#pragma unroll
  for (int u = 0; u < kU; ++u) {
    src[u] = kZeroRow;
    if (t[u] < 0) continue;
    if (b[u] >= 0) {
      if (b[u] < v.pool_blocks) src[u] = (b[u] << v.ps) | (t[u] & v.pm);
    } else if (hb[u] >= 0 && hb[u] < v.host_blocks) {
      src[u] = (int32_t)(kHostTag | (uint32_t)((hb[u] << v.ps) | (t[u] & v.pm)));
    } else {
      src[u] = kNoHost;
    }
  }
}

// Classifies entries [lo, hi) into keys[e - lo] (the token) and src[e - lo];
// returns whether this thread saw an entry for which `want` holds.  The
// first kT * kU entries' tokens come loaded (t0, from load_tokens at lo).
// Ends with a barrier.
template <typename Want>
__device__ __forceinline__ bool classify_range(const FetchParams& p, const Rl& v, int32_t lo,
                                               int32_t hi, int32_t* keys, int32_t* src,
                                               const int32_t (&t0)[kU], Want want) {
  const int tid = threadIdx.x;
  bool any = false;
  for (int32_t e0 = lo; e0 < hi; e0 += kT * kU) {
    int32_t t[kU], sv[kU];
    if (e0 == lo) {
#pragma unroll
      for (int u = 0; u < kU; ++u) t[u] = t0[u];
    } else {
      load_tokens(p, v, e0, hi, t);
    }
    classify_tokens(v, v.bt, v.hbt, t, sv);
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const int32_t el = e0 + u * kT + tid - lo;
      if (el < hi - lo) {
        keys[el] = t[u];
        src[el] = sv[u];
        any |= want(sv[u]);
      }
    }
  }
  __syncthreads();
  return any;
}

// Gather workgroup: entries [lo, hi) of one request-layer, every row but the
// misses': resident and hot rows from the pool, zero rows otherwise.
__device__ void fill_gather(const FetchParams& p, int32_t* lds, int32_t rl, int32_t lo,
                            int32_t hi) {
  const int tid = threadIdx.x;
  const Rl v = rl_view(p, rl);
  const int32_t E = hi - lo;
  // LDS: keys[E] | src[E] | tab[n] | flag
  int32_t* keys = lds;
  int32_t* src = keys + p.gather_e;
  uint32_t* tab = reinterpret_cast<uint32_t*>(src + p.gather_e);
  const int32_t n = p.gather_tab_n;
  int32_t* flag = reinterpret_cast<int32_t*>(tab + n);
  // the first entries' tokens are loaded before the slots, so that their
  // block-table loads need not wait for the slots' loads
  int32_t t0[kU];
  load_tokens(p, v, lo, hi, t0);
  int32_t pre[kScanUnroll];
  prefetch_slots(p, rl, pre);
  for (int32_t h = tid; h < n; h += kT) tab[h] = kEmptyWord;
  if (tid == 0) *flag = 0;
  const bool any = classify_range(p, v, lo, hi, keys, src, t0,
                                  [](int32_t s) { return non_resident(s); });
  if (any) *flag = 1;
  for (int32_t el = tid; el < E; el += kT)
    if (non_resident(src[el])) map_insert(tab, n, keys, keys[el], el);
  __syncthreads();
  if (*flag) {
    scan_slots(p, rl, tab, n, keys, pre);
    for (int32_t el = tid; el < E; el += kT) {
      const int32_t sv = src[el];
      if (!non_resident(sv)) continue;
      const uint32_t q = tab[map_find(tab, n, keys, keys[el])] & 0xFFFFu;
      src[el] = q != kNoSlot ? (v.hot[q >> v.ps] << v.ps) | ((int32_t)q & v.pm)  // hot
                             : sv == kNoHost ? kZeroRow : kSkip;                  // miss
    }
    __syncthreads();
  }
  HS_FILL_MARK(2);
  const int32_t total = E * v.pieces;
  for (int32_t j = 0; j < v.group; ++j) {  // each layer of the group
    const uint8_t* pool_l = v.pool_l + j * v.pool_stride;
    uint8_t* out = v.out + j * v.out_stride;
    for (int32_t g0 = 0; g0 < total; g0 += kT * kU) {
      u32x4 val[kU];
      uint8_t* dst[kU];
#pragma unroll
      for (int u = 0; u < kU; ++u) {
        const int32_t g = g0 + u * kT + tid;
        dst[u] = nullptr;
        val[u] = u32x4{0u, 0u, 0u, 0u};
        if (g < total) {
          const int32_t el = pdiv(g, v.magic);
          const int32_t pc = g - el * v.pieces;
          const int32_t code = src[el];
          if (code != kSkip) dst[u] = out + (int64_t)(lo + el) * p.row_bytes + pc * 16;
          if (code >= 0)
            val[u] = *reinterpret_cast<const u32x4*>(pool_l + (int64_t)code * p.row_bytes +
                                                     pc * 16);
        }
      }
#pragma unroll
      for (int u = 0; u < kU; ++u)
        if (dst[u]) __builtin_nontemporal_store(val[u], reinterpret_cast<u32x4*>(dst[u]));
    }
  }
}

// Pieces [g_lo, g_hi) of the host rows of the first entries list[], U reads
// in flight a thread; g_lo is a multiple of kT.
template <int U>
__device__ __forceinline__ void host_rows(const FetchParams& p, const Rl& v, const int32_t* list,
                                          const int32_t* src, const uint8_t* host_l,
                                          uint8_t* out, int32_t g_lo, int32_t g_hi) {
  const int tid = threadIdx.x;
  for (int32_t g0 = g_lo; g0 < g_hi; g0 += kT * U) {
    u32x4 val[U];
    uint8_t* dst[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int32_t g = g0 + u * kT + tid;
      dst[u] = nullptr;
      if (g < g_hi) {
        const int32_t j = pdiv(g, v.magic);
        const int32_t pc = g - j * v.pieces;
        const int32_t e = list[j];
        const int64_t hrow = (int64_t)((uint32_t)src[e] & ~kHostTag);
        val[u] = *reinterpret_cast<const u32x4*>(host_l + hrow * p.row_bytes + pc * 16);
        dst[u] = out + (int64_t)e * p.row_bytes + pc * 16;
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u)
      if (dst[u]) __builtin_nontemporal_store(val[u], reinterpret_cast<u32x4*>(dst[u]));
  }
}

// Miss workgroup s of S for one request-layer: the rows of the miss tokens t
// with t mod S == s, each read once from the host into its first entry and
// then copied to its later entries.
__device__ void fill_misses(const FetchParams& p, int32_t* lds, int32_t rl, int32_t s,
                            int32_t S) {
  const int tid = threadIdx.x;
  const Rl v = rl_view(p, rl);
  const int32_t N = v.N;
  // LDS: keys[N] | src[N] | list[N] | tab[n] | counters[4] (| slot bitmap)
  int32_t* keys = lds;
  int32_t* src = keys + p.lds_n;
  int32_t* list = src + p.lds_n;
  uint32_t* tab = reinterpret_cast<uint32_t*>(list + p.lds_n);
  const int32_t n = p.miss_tab_n;
  int32_t* cnt = reinterpret_cast<int32_t*>(tab + n);
  // the first entries' tokens before the slots (as in fill_gather)
  int32_t t0[kU];
  load_tokens(p, v, 0, N, t0);
  int32_t pre[kScanUnroll];
  prefetch_slots(p, rl, pre);
  for (int32_t h = tid; h < n; h += kT) tab[h] = kEmptyWord;
  if (tid < 4) cnt[tid] = 0;
  // with a slot bitmap (after the counters): bit t set when a usable slot
  // holds token t; only the misses then enter the table, and no slot probes it
  const int32_t nb = p.slot_bits_words;
  uint32_t* bits = reinterpret_cast<uint32_t*>(cnt + 4);
  for (int32_t h = tid; h < nb; h += kT) bits[h] = 0u;
  const bool any = classify_range(p, v, 0, N, keys, src, t0,
                                  [](int32_t s) { return is_host_row(s); });
  if (any) cnt[2] = 1;  // racing writes of the same value
  HS_FILL_MARK(1);
  bool listed = false;  // the work lists below are already built
  if (nb > 0) {
    // every usable slot came with the first loads (pre); the bitmap was
    // cleared before classify_range's barrier
    const int32_t lim = nb * 32;
#pragma unroll
    for (int u = 0; u < kScanUnroll; ++u) {
      const int32_t t = pre[u];
      if (t >= 0 && t < lim && (S == 1 || t % S == s)) atomicOr(&bits[t >> 5], 1u << (t & 31));
    }
    __syncthreads();
    // a host row whose token a slot holds is a hit, which the gather
    // workgroups write; the others of this workgroup's tokens are misses
    if (!p.misses_only) {
      // the entry that claims a miss token's word reads its row; the token's
      // other entries copy that row (every entry ends with the same bytes,
      // whichever entry reads)
      for (int32_t e0 = 0; e0 < N; e0 += kT) {
        const int32_t e = e0 + tid;
        const int32_t sv = e < N ? src[e] : kZeroRow;
        const int32_t t = e < N ? keys[e] : -1;
        bool first = false, dup = false;
        int32_t f = -1;
        if (is_host_row(sv) && (S == 1 || t % S == s)) {
          if ((bits[t >> 5] >> (t & 31)) & 1u) {
            src[e] = kSkip;
          } else {
            f = map_claim(tab, n, keys, t, e);
            first = f < 0;
            dup = !first;
          }
        }
        const int32_t i = wave_append(&cnt[0], first);
        if (first) list[i] = e;
        const int32_t j = wave_append(&cnt[1], dup);
        if (dup) {
          list[p.lds_n - 1 - j] = e;
          src[e] = f;  // a later entry copies the reading entry's output row
        }
      }
      __syncthreads();
      listed = true;
      HS_FILL_MARK(-1);
      if (cnt[0] == 0) return;  // no miss among this workgroup's tokens
    } else {
      // the staging rows are the first entries' only: the smallest entry of
      // each miss token reads its row (the table keeps the smallest)
      for (int32_t e = tid; e < N; e += kT) {
        if (!is_host_row(src[e])) continue;
        const int32_t t = keys[e];
        if (S != 1 && t % S != s) continue;
        if ((bits[t >> 5] >> (t & 31)) & 1u) {
          src[e] = kSkip;
        } else {
          map_insert(tab, n, keys, t, e);
          cnt[3] = 1;  // racing writes of the same value
        }
      }
      __syncthreads();
      HS_FILL_MARK(-1);
      if (cnt[3] == 0) return;  // no miss among this workgroup's tokens
    }
  } else {
    // only this workgroup's tokens (t mod S == s) enter the table and are
    // looked up by the slots
    for (int32_t e = tid; e < N; e += kT)
      if (is_host_row(src[e]) && (S == 1 || keys[e] % S == s)) map_insert(tab, n, keys, keys[e], e);
    __syncthreads();
    HS_FILL_MARK(-1);
    if (cnt[2] == 0) return;  // nothing to read from the host
    scan_slots(p, rl, tab, n, keys, pre, s, S);
  }
  HS_FILL_MARK(2);

  // ---- this workgroup's work lists: first entries of its miss tokens from
  // the front of list[], their later entries from the back ----------------
  if (!listed) {
    for (int32_t e0 = 0; e0 < N; e0 += kT) {
      const int32_t e = e0 + tid;
      const int32_t sv = e < N ? src[e] : kZeroRow;
      const int32_t t = e < N ? keys[e] : -1;
      bool first = false, dup = false;
      int32_t f = -1;
      if (is_host_row(sv) && (t % S) == s) {
        const uint32_t w = tab[map_find(tab, n, keys, t)];
        if ((w & 0xFFFFu) == kNoSlot) {  // not in the hot buffer: a miss
          f = (int32_t)(w >> 16);
          first = f == e;
          dup = !first;
        }
      }
      const int32_t i = wave_append(&cnt[0], first);
      if (first) list[i] = e;
      const int32_t j = wave_append(&cnt[1], dup);
      if (dup) {
        list[p.lds_n - 1 - j] = e;
        src[e] = f;  // a later entry copies the first entry's output row
      }
    }
    __syncthreads();
  }
  const int32_t n_first = cnt[0];
  const int32_t n_dup = cnt[1];
  HS_FILL_MARK(3);

  // ---- host rows of the first entries, in each layer of the group,
  // kHostUnroll reads in flight a thread (more in flight at the end of the
  // step, when the gathers are done, gains nothing: the link is the bound)
  const int32_t total = n_first * v.pieces;
  for (int32_t l = 0; l < v.group; ++l)
    host_rows<kHostUnroll>(p, v, list, src, v.host_l + l * v.host_stride, v.out + l * v.out_stride,
                           0, total);
  HS_FILL_MARK(-2);
  if (n_dup == 0 || p.misses_only) return;
  __syncthreads();  // this workgroup's row writes are visible to it

  // ---- later entries of the owned miss tokens copy the first entry's row
  const int32_t total2 = n_dup * v.pieces;
  const int32_t* dl = list + p.lds_n - n_dup;
  for (int32_t l = 0; l < v.group; ++l) {
    uint8_t* out = v.out + l * v.out_stride;
    for (int32_t g0 = 0; g0 < total2; g0 += kT * kU) {
      u32x4 val[kU];
      uint8_t* dst[kU];
#pragma unroll
      for (int u = 0; u < kU; ++u) {
        const int32_t g = g0 + u * kT + tid;
        dst[u] = nullptr;
        if (g < total2) {
          const int32_t j = pdiv(g, v.magic);
          const int32_t pc = g - j * v.pieces;
          const int32_t e = dl[j];
          val[u] = *reinterpret_cast<const u32x4*>(out + (int64_t)src[e] * p.row_bytes + pc * 16);
          dst[u] = out + (int64_t)e * p.row_bytes + pc * 16;
        }
      }
#pragma unroll
      for (int u = 0; u < kU; ++u)
        if (dst[u]) __builtin_nontemporal_store(val[u], reinterpret_cast<u32x4*>(dst[u]));
    }
  }
}

// Fill block b of the launch's fill blocks: [0, miss_groups) are miss
// workgroups, the rest gather workgroups, gather_splits per request-layer.
// Miss workgroup g takes the (request-layer, split) item g first, then, with
// fill_sync and more items than miss workgroups, the next item not yet taken
// (a counter in fill_sync; the host link serves the XCDs at different rates,
// so fixed shares end with the slowest), otherwise items g + miss_groups, ...
__device__ void fill_block(const FetchParams& p, int32_t* lds, int32_t b) {
  HS_FILL_MARK(0);
  const int32_t n_rl = p.num_reqs * p.num_layers;
  if (b < p.miss_groups) {
    const int tid = threadIdx.x;
    const int32_t S = p.miss_splits;
    const int32_t items = n_rl * S;
    const bool dyn = p.sync != nullptr && items > p.miss_groups;
    // the fourth counter word of fill_misses carries the next item between
    // its calls (it clears the word only after the barrier that starts a
    // call)
    int32_t* next = lds + 3 * p.lds_n + p.miss_tab_n + 3;
    int32_t it = b;
    for (int32_t round = 0; it < items && round < items; ++round) {
      if (round > 0) __syncthreads();  // the previous item's LDS reads are done
      fill_misses(p, lds, it / S, it % S, S);
      if (dyn) {
        __syncthreads();
        if (tid == 0) *next = atomicAdd(&p.sync[kSyncItems], 1) + p.miss_groups;
        __syncthreads();
        it = *next;
      } else {
        it += p.miss_groups;
      }
    }
    if (dyn && tid == 0) {
      // every take of this workgroup precedes its count; the last workgroup
      // counted clears both words for the next launch
      __threadfence();
      if (atomicAdd(&p.sync[kSyncDone], 1) == p.miss_groups - 1) {
        __hip_atomic_store(&p.sync[kSyncItems], 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __hip_atomic_store(&p.sync[kSyncDone], 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
    }
    HS_FILL_MARK(5);
    return;
  }
  const int32_t i = b - p.miss_groups;
  const int32_t rl = i / p.gather_splits;
  const int32_t s = i - rl * p.gather_splits;
  const int32_t lo = min(p.entries, s * p.gather_e);
  const int32_t hi = min(p.entries, lo + p.gather_e);
  fill_gather(p, lds, rl, lo, hi);
  HS_FILL_MARK(5);
}

}  // namespace
}  // namespace fill
}  // namespace hs
