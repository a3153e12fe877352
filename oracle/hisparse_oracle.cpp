// Plain CPU oracle for the Hybrid HiSparse top-K resolver, the single-stride
// row gather and the post-forward prefix-page offload.
//
// TEST INFRASTRUCTURE ONLY.  This file is the slow, obviously correct
// statement of what the GPU library computes.  Only the test suite, the smoke
// check and the benchmark's CPU-baseline leg may load it; the product path
// never does.  It shares no code, header or table with the HIP library.
//
// Source: "vLLM GLM 5.3 ... Hybrid HiSparse offloading, Part 1" (three
// renderings of one blog post).  Sections cited below:
//   [HOW]   "How it works" -- mixed residency: block tables hold real blocks
//           and null placeholders, the tail never leaves; one fused kernel
//           resolves the top-K: resident tokens are read in place, hot tokens
//           are read and their LRU entry refreshed, a miss copies one row from
//           pinned host memory into the LRU slot; nothing waits on the CPU.
//   [FIG2]  caption of the "How it works" figure: a miss copies one row into
//           a hot page, a hit reuses it without a copy.
//   [HMA]   "How it works", last paragraphs: hot pages are ordinary KV blocks
//           of the same pool; the resolver hands back an HMA row id whether
//           the row is resident or hot, and rows are gathered at one stride;
//           completed prefix pages are copied to host while still served from
//           the GPU, in one launch over all sparse layers after the forward.
//   [INTEG] "Integration with the rest of vLLM": speculative decoding uses a
//           per-step replayable resolve plan sharing the request's hot state;
//           the hot buffer defaults to 2 x top-K rows per request.
//   [SHARE] "Use sparsity when needed": GLM 5.3's IndexShare places one
//           indexer layer per 4 sparse-MLA layers, so a group of layers
//           attends to one top-K list.
//   [COLD]  "Use sparsity when needed": under pressure a request frees its
//           coldest pages in place; a page's coldness here is the last stamp
//           at which a top-K list selected one of its tokens.
//
// Where the pages leave a choice open the plainest reading is taken:
//   * null placeholder / no host copy / empty slot = a negative entry;
//   * row id = block * page_size + offset, the same id in every layer;
//   * hot slot q lives at row hot_blocks[q / page] * page + q % page;
//   * an LRU entry is a uint32 stamp (the caller's step counter, 0 = never);
//   * victims are the non-hit slots in ascending (stamp, slot) order and are
//     given to the misses in ascending token order;
//   * duplicate tokens in one list are resolved once and share one row;
//   * -1 entries are padding (row -1); a token outside [0, ctx) or without a
//     resident page or host copy is invalid (row -3); a miss with no slot
//     left is an overflow (row -2, only possible when several query
//     positions share one plan);
//   * all reads see the state as it was before the call, then everything is
//     committed at once; request-layers are independent.
//   * entries that point outside the arrays the caller described (a block
//     past the pool, a host block past the host pool, a hot block past the
//     pool) are treated as absent, never dereferenced.

#include <algorithm>
#include <cstdint>
#include <cstring>
#include <unordered_map>
#include <vector>

namespace {

enum Kind { PAD = 0, INVALID = 1, RESIDENT = 2, NONRES = 3 };

const int32_t ROW_PAD = -1;
const int32_t ROW_OVERFLOW = -2;
const int32_t ROW_INVALID = -3;

struct Layout {
  int32_t page;
  int32_t row_bytes;
  int64_t pool_rows, host_rows;               // rows per layer
  int64_t pool_layer_stride, host_layer_stride;  // bytes between layers
};

inline bool row_in(int64_t row, int64_t rows) { return row >= 0 && row < rows; }

// Resolve the N entries of one request-layer ([HOW], [FIG2], [HMA], [INTEG]).
// `copies`, when given, receives the (host row, pool row) of every row copy
// made into pool_l.
void resolve_one(const Layout& lay, int32_t N, int32_t C, int32_t max_pages, int32_t ctx,
                 const int32_t* bt, const int32_t* hbt, const int32_t* hot_blocks,
                 int32_t* tok, uint32_t* stp, uint32_t stamp, const int32_t* topk,
                 int32_t* rows, int32_t* stats, uint8_t* pool_l, const uint8_t* host_l,
                 std::vector<std::pair<int64_t, int64_t>>* copies = nullptr) {
  const int32_t page = lay.page;
  const int64_t pool_blocks = lay.pool_rows / page;
  const int64_t host_blocks = lay.host_rows / page;

  // Step 1: classify every entry.  Resident tokens are translated in place
  // through the block table and never consult the hot buffer ([HOW]).
  std::vector<int> kind(N);
  for (int32_t i = 0; i < N; ++i) {
    const int32_t t = topk[i];
    rows[i] = 0;
    if (t == -1) { kind[i] = PAD; rows[i] = ROW_PAD; continue; }
    if (t < 0 || t >= ctx || t / page >= max_pages) { kind[i] = INVALID; rows[i] = ROW_INVALID; continue; }
    const int32_t b = bt[t / page];
    if (b >= 0) {
      if (b >= pool_blocks) { kind[i] = INVALID; rows[i] = ROW_INVALID; continue; }
      kind[i] = RESIDENT;
      rows[i] = b * page + t % page;
    } else {
      kind[i] = NONRES;
    }
  }

  // Step 2: the ascending set of distinct non-resident tokens.
  std::vector<int32_t> U;
  for (int32_t i = 0; i < N; ++i)
    if (kind[i] == NONRES) U.push_back(topk[i]);
  std::sort(U.begin(), U.end());
  U.erase(std::unique(U.begin(), U.end()), U.end());

  // A slot is usable only if its leased block lies inside the pool.
  auto slot_ok = [&](int32_t q) {
    const int32_t hb = hot_blocks[q / page];
    return hb >= 0 && hb < pool_blocks;
  };
  auto hot_row = [&](int32_t q) { return hot_blocks[q / page] * page + q % page; };

  // Step 3: hot map lookup (the token -> slot map is the slot_token array,
  // pre-call).  A hit beats a missing host copy: the row is already on GPU.
  std::unordered_map<int32_t, int32_t> where;  // token -> smallest slot holding it
  for (int32_t q = C - 1; q >= 0; --q)
    if (tok[q] >= 0 && slot_ok(q)) where[tok[q]] = q;
  enum UKind { U_HIT, U_MISS, U_INVALID };
  std::vector<int> ukind(U.size());
  std::vector<int32_t> uslot(U.size(), -1);
  std::vector<char> is_hit_slot(C, 0);
  std::vector<int32_t> misses;  // ascending, since U is ascending
  std::vector<int32_t> miss_uidx;
  for (size_t k = 0; k < U.size(); ++k) {
    auto it = where.find(U[k]);
    if (it != where.end()) {
      ukind[k] = U_HIT;
      uslot[k] = it->second;
      is_hit_slot[it->second] = 1;
    } else {
      const int32_t hb = hbt[U[k] / page];
      if (hb < 0 || hb >= host_blocks) {
        ukind[k] = U_INVALID;
      } else {
        ukind[k] = U_MISS;
        misses.push_back(U[k]);
        miss_uidx.push_back((int32_t)k);
      }
    }
  }

  // Step 4: victims = usable non-hit slots in ascending (stamp, slot) order,
  // i.e. least recently used first; empty slots (stamp 0) come first.
  std::vector<int32_t> V;
  for (int32_t q = 0; q < C; ++q)
    if (!is_hit_slot[q] && slot_ok(q)) V.push_back(q);
  std::sort(V.begin(), V.end(), [&](int32_t a, int32_t b) {
    if (stp[a] != stp[b]) return stp[a] < stp[b];
    return a < b;
  });

  // Step 5: the j-th smallest miss takes the j-th victim; the rest overflow.
  const size_t M = misses.size();
  const size_t A = std::min(M, V.size());

  // Step 6: commit.  Hits refresh their stamp; each assigned miss copies one
  // row from the host pool into its victim slot and takes the slot over.
  for (size_t k = 0; k < U.size(); ++k)
    if (ukind[k] == U_HIT) stp[uslot[k]] = stamp;
  for (size_t j = 0; j < A; ++j) {
    const int32_t q = V[j];
    const int32_t u = misses[j];
    const int64_t src_row = (int64_t)hbt[u / page] * page + u % page;
    const int64_t dst_row = hot_row(q);
    std::memcpy(pool_l + dst_row * lay.row_bytes, host_l + src_row * lay.row_bytes,
                (size_t)lay.row_bytes);
    if (copies) copies->emplace_back(src_row, dst_row);
    tok[q] = u;
    stp[q] = stamp;
    uslot[miss_uidx[j]] = q;
  }

  // Step 7: row ids for the non-resident entries.
  for (int32_t i = 0; i < N; ++i) {
    if (kind[i] != NONRES) continue;
    const size_t k = std::lower_bound(U.begin(), U.end(), topk[i]) - U.begin();
    if (ukind[k] == U_INVALID) rows[i] = ROW_INVALID;
    else if (uslot[k] >= 0) rows[i] = hot_row(uslot[k]);
    else rows[i] = ROW_OVERFLOW;
  }

  // Step 9: statistics over distinct tokens (pad and dup count entries).
  std::vector<int32_t> nonpad;
  for (int32_t i = 0; i < N; ++i)
    if (kind[i] != PAD) nonpad.push_back(topk[i]);
  const int32_t n_nonpad = (int32_t)nonpad.size();
  std::sort(nonpad.begin(), nonpad.end());
  nonpad.erase(std::unique(nonpad.begin(), nonpad.end()), nonpad.end());
  // The class of an entry depends only on its token, so distinct resident
  // (or invalid) tokens are the distinct values among those entries.
  std::vector<int32_t> res_tok, inv_tok;
  for (int32_t i = 0; i < N; ++i) {
    if (kind[i] == RESIDENT) res_tok.push_back(topk[i]);
    if (kind[i] == INVALID) inv_tok.push_back(topk[i]);
  }
  auto n_distinct = [](std::vector<int32_t>& v) {
    std::sort(v.begin(), v.end());
    return (int32_t)(std::unique(v.begin(), v.end()) - v.begin());
  };
  const int32_t resident = n_distinct(res_tok), invalid = n_distinct(inv_tok);
  int32_t hit = 0, uinv = 0;
  for (size_t k = 0; k < U.size(); ++k) {
    if (ukind[k] == U_HIT) ++hit;
    if (ukind[k] == U_INVALID) ++uinv;
  }
  int32_t pad = N - n_nonpad;
  stats[0] = resident;
  stats[1] = hit;
  stats[2] = (int32_t)A;
  stats[3] = (int32_t)(M - A);
  stats[4] = invalid + uinv;
  stats[5] = pad;
  stats[6] = n_nonpad - (int32_t)nonpad.size();
  stats[7] = 0;
}

void gather_rows(const Layout& lay, int32_t R, int32_t L, int32_t N, const uint8_t* pool,
                 const int32_t* rows, uint8_t* out) {
  for (int32_t r = 0; r < R; ++r)
    for (int32_t l = 0; l < L; ++l)
      for (int32_t i = 0; i < N; ++i) {
        const int64_t e = ((int64_t)r * L + l) * N + i;
        const int64_t row = rows[e];
        uint8_t* dst = out + e * lay.row_bytes;
        if (row_in(row, lay.pool_rows))
          std::memcpy(dst, pool + l * lay.pool_layer_stride + row * lay.row_bytes,
                      (size_t)lay.row_bytes);
        else
          std::memset(dst, 0, (size_t)lay.row_bytes);
      }
}

}  // namespace

extern "C" {

// Gather ([HMA]: rows handed back by the resolver are gathered at one stride):
// out[r][l][i] = pool[l][rows[r][l][i]], a zero row for ids outside the pool.
int oracle_gather(int32_t page, int32_t row_bytes, int64_t pool_rows, int64_t pool_layer_stride,
                  int32_t R, int32_t L, int32_t N, const uint8_t* pool, const int32_t* rows,
                  uint8_t* out) {
  Layout lay{page, row_bytes, pool_rows, 0, pool_layer_stride, 0};
  gather_rows(lay, R, L, N, pool, rows, out);
  return 0;
}

// Prefix-page offload ([HMA], proactive copy in one launch over every sparse
// layer): for each (device block, host block) pair and every layer, the
// page's rows are copied device -> host.  Pairs naming a block outside either
// pool are skipped.
int oracle_offload(int32_t page, int32_t row_bytes, int32_t L, int64_t pool_rows,
                   int64_t pool_layer_stride, int64_t host_rows, int64_t host_layer_stride,
                   const uint8_t* pool, uint8_t* host, const int32_t* pairs, int32_t n) {
  const int64_t page_bytes = (int64_t)page * row_bytes;
  for (int32_t i = 0; i < n; ++i) {
    const int64_t db = pairs[2 * i], hb = pairs[2 * i + 1];
    if (db < 0 || db >= pool_rows / page || hb < 0 || hb >= host_rows / page) continue;
    for (int32_t l = 0; l < L; ++l)
      std::memcpy(host + l * host_layer_stride + hb * page_bytes,
                  pool + l * pool_layer_stride + db * page_bytes, (size_t)page_bytes);
  }
  return 0;
}

// Page coldness ([COLD]): for every request r and every list entry t of
// topk[r][0..E) that is a token of the context (0 <= t < ctx_len[r]) on a
// page the table has (t / page < max_pages), the page's word in
// page_use[r][max_pages] becomes `stamp`; every other word keeps its value.
int oracle_page_touch(int32_t page, int32_t R, int32_t max_pages, int32_t E,
                      const int32_t* ctx_len, const int32_t* topk, uint32_t stamp,
                      uint32_t* page_use) {
  for (int32_t r = 0; r < R; ++r) {
    for (int32_t e = 0; e < E; ++e) {
      const int64_t t = topk[(int64_t)r * E + e];
      if (t < 0 || t >= ctx_len[r]) continue;
      const int64_t pg = t / page;
      if (pg >= max_pages) continue;
      page_use[(int64_t)r * max_pages + pg] = stamp;
    }
  }
  return 0;
}

// Resolve (and optionally gather) one batch: R requests x L layers, each with
// N = positions x top_k entries; a replayable plan over several query
// positions ([INTEG]) is the same resolve over the concatenated lists with one
// stamp commit.  Arrays:
//   block_table, host_block_table [R][max_pages]; ctx_len [R];
//   hot_blocks [R][C / page]; slot_token, slot_stamp [R][L][C] (in/out);
//   topk, rows [R][L][N]; stats [R][L][8]; gather_out [R][L][N][row_bytes] or null.
int oracle_resolve(int32_t page, int32_t row_bytes, int32_t L, int32_t C, int64_t pool_rows,
                   int64_t pool_layer_stride, int64_t host_rows, int64_t host_layer_stride,
                   int32_t R, int32_t max_pages, uint8_t* pool, const uint8_t* host,
                   const int32_t* block_table, const int32_t* host_block_table,
                   const int32_t* ctx_len, const int32_t* hot_blocks, int32_t* slot_token,
                   uint32_t* slot_stamp, const int32_t* topk, int32_t N, uint32_t stamp,
                   int32_t* rows, int32_t* stats, uint8_t* gather_out) {
  Layout lay{page, row_bytes, pool_rows, host_rows, pool_layer_stride, host_layer_stride};
  for (int32_t r = 0; r < R; ++r)
    for (int32_t l = 0; l < L; ++l) {
      const int64_t rl = (int64_t)r * L + l;
      resolve_one(lay, N, C, max_pages, ctx_len[r], block_table + (int64_t)r * max_pages,
                  host_block_table + (int64_t)r * max_pages, hot_blocks + (int64_t)r * (C / page),
                  slot_token + rl * C, slot_stamp + rl * C, stamp, topk + rl * N, rows + rl * N,
                  stats + rl * 8, pool + l * pool_layer_stride, host + l * host_layer_stride);
    }
  // Step 8: the gather reads the pool after every copy of the call.
  if (gather_out) gather_rows(lay, R, L, N, pool, rows, gather_out);
  return 0;
}

// Grouped resolve ([SHARE]): the L layers form L / G groups of G layers that
// share one top-K list and one hot-buffer state (slot tokens and stamps per
// group).  A group's decisions are those of a resolve on its lists and state;
// every copy it makes is made in each of its G layers (the layer's own host
// row into the layer's own slot row), and every layer of the group gets the
// group's row ids.  Arrays as oracle_resolve, but: slot_token, slot_stamp
// [R][L/G][C]; topk, rows [R][L/G][N]; stats [R][L/G][8]; gather_out
// [R][L][N][row_bytes] or null (out[r][l][i] = pool[l][rows[r][l/G][i]]).
int oracle_resolve_grouped(int32_t page, int32_t row_bytes, int32_t L, int32_t G, int32_t C,
                           int64_t pool_rows, int64_t pool_layer_stride, int64_t host_rows,
                           int64_t host_layer_stride, int32_t R, int32_t max_pages, uint8_t* pool,
                           const uint8_t* host, const int32_t* block_table,
                           const int32_t* host_block_table, const int32_t* ctx_len,
                           const int32_t* hot_blocks, int32_t* slot_token, uint32_t* slot_stamp,
                           const int32_t* topk, int32_t N, uint32_t stamp, int32_t* rows,
                           int32_t* stats, uint8_t* gather_out) {
  if (G < 1 || L % G != 0) return 1;
  Layout lay{page, row_bytes, pool_rows, host_rows, pool_layer_stride, host_layer_stride};
  const int32_t NG = L / G;
  for (int32_t r = 0; r < R; ++r)
    for (int32_t g = 0; g < NG; ++g) {
      const int64_t rg = (int64_t)r * NG + g;
      const int32_t l0 = g * G;
      std::vector<std::pair<int64_t, int64_t>> copies;
      resolve_one(lay, N, C, max_pages, ctx_len[r], block_table + (int64_t)r * max_pages,
                  host_block_table + (int64_t)r * max_pages, hot_blocks + (int64_t)r * (C / page),
                  slot_token + rg * C, slot_stamp + rg * C, stamp, topk + rg * N, rows + rg * N,
                  stats + rg * 8, pool + l0 * pool_layer_stride, host + l0 * host_layer_stride,
                  &copies);
      for (int32_t l = l0 + 1; l < l0 + G; ++l)
        for (const auto& c : copies)
          std::memcpy(pool + l * pool_layer_stride + c.second * row_bytes,
                      host + l * host_layer_stride + c.first * row_bytes, (size_t)row_bytes);
    }
  if (gather_out) {
    for (int32_t r = 0; r < R; ++r)
      for (int32_t l = 0; l < L; ++l)
        for (int32_t i = 0; i < N; ++i) {
          const int64_t row = rows[((int64_t)r * NG + l / G) * N + i];
          uint8_t* dst = gather_out + (((int64_t)r * L + l) * N + i) * row_bytes;
          if (row_in(row, pool_rows))
            std::memcpy(dst, pool + l * pool_layer_stride + row * row_bytes, (size_t)row_bytes);
          else
            std::memset(dst, 0, (size_t)row_bytes);
        }
  }
  return 0;
}

}  // extern "C"
