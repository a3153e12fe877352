// A native driver for the host-side C++ built with AddressSanitizer and
// UndefinedBehaviorSanitizer: the CPU oracle (oracle/hisparse_oracle.cpp) and
// the residency policy (serving_memory_tier_amd/csrc/policy.cpp).  The test
// suite compiles it together with those two sources and runs it; any
// out-of-bounds access, use after free, leak or undefined operation aborts
// the run.  It also checks the hand-worked resolve example (4-token pages, 8
// slots) so that a sanitized build computes what the plain one does.
//
// Build (what tests/test_sanitize.py runs):
//   g++ -std=c++17 -O1 -g -fsanitize=address,undefined -fno-sanitize-recover=all
//       -I include tests/native/sanitize_driver.cpp oracle/hisparse_oracle.cpp
//       serving_memory_tier_amd/csrc/policy.cpp -o sanitize_driver

#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <random>
#include <vector>

#include "hs_policy.h"

extern "C" {
int oracle_gather(int32_t page, int32_t row_bytes, int64_t pool_rows, int64_t pool_layer_stride,
                  int32_t R, int32_t L, int32_t N, const uint8_t* pool, const int32_t* rows,
                  uint8_t* out);
int oracle_offload(int32_t page, int32_t row_bytes, int32_t L, int64_t pool_rows,
                   int64_t pool_layer_stride, int64_t host_rows, int64_t host_layer_stride,
                   const uint8_t* pool, uint8_t* host, const int32_t* pairs, int32_t n);
int oracle_page_touch(int32_t page, int32_t R, int32_t max_pages, int32_t E,
                      const int32_t* ctx_len, const int32_t* topk, uint32_t stamp,
                      uint32_t* page_use);
int oracle_resolve(int32_t page, int32_t row_bytes, int32_t L, int32_t C, int64_t pool_rows,
                   int64_t pool_layer_stride, int64_t host_rows, int64_t host_layer_stride,
                   int32_t R, int32_t max_pages, uint8_t* pool, const uint8_t* host,
                   const int32_t* block_table, const int32_t* host_block_table,
                   const int32_t* ctx_len, const int32_t* hot_blocks, int32_t* slot_token,
                   uint32_t* slot_stamp, const int32_t* topk, int32_t N, uint32_t stamp,
                   int32_t* rows, int32_t* stats, uint8_t* gather_out);
int oracle_resolve_grouped(int32_t page, int32_t row_bytes, int32_t L, int32_t G, int32_t C,
                           int64_t pool_rows, int64_t pool_layer_stride, int64_t host_rows,
                           int64_t host_layer_stride, int32_t R, int32_t max_pages, uint8_t* pool,
                           const uint8_t* host, const int32_t* block_table,
                           const int32_t* host_block_table, const int32_t* ctx_len,
                           const int32_t* hot_blocks, int32_t* slot_token, uint32_t* slot_stamp,
                           const int32_t* topk, int32_t N, uint32_t stamp, int32_t* rows,
                           int32_t* stats, uint8_t* gather_out);
}

namespace {

int g_failures = 0;

void check(bool ok, const char* what) {
  if (!ok) {
    std::fprintf(stderr, "CHECK FAILED: %s\n", what);
    ++g_failures;
  }
}

constexpr int32_t kRow = 656;

// The hand-worked instance: 4-token pages, context 24, 8 slots in hot blocks
// 9 and 6, pages 4 and 5 resident in blocks 7 and 2, every page on host.
void worked_example() {
  const int32_t page = 4, C = 8, ctx = 24, max_pages = 6;
  const int64_t pool_rows = 10 * page, host_rows = 6 * page;
  std::vector<uint8_t> pool(pool_rows * kRow), host(host_rows * kRow);
  for (int64_t r = 0; r < pool_rows; ++r) std::memcpy(&pool[r * kRow], &r, 4);
  for (int64_t r = 0; r < host_rows; ++r) std::memcpy(&host[r * kRow], &r, 4);
  std::vector<int32_t> bt = {-1, -1, -1, -1, 7, 2}, hbt = {3, 0, 5, 1, 4, 2};
  std::vector<int32_t> hot = {9, 6}, tok(C, -1);
  std::vector<uint32_t> stp(C, 0);
  const int32_t lists[4][6] = {{21, 5, 13, 2, 17, 9},
                               {9, 1, 22, 13, 6, 14},
                               {17, 2, 10, 6, 20, 3},
                               {17, 2, 10, 6, 20, 3}};
  const int32_t want[4][6] = {{9, 37, 39, 36, 29, 38},
                              {38, 24, 10, 39, 25, 26},
                              {38, 36, 37, 25, 8, 27},
                              {38, 36, 37, 25, 8, 27}};
  std::vector<int32_t> rows(6), stats(8);
  std::vector<uint8_t> out(6 * kRow);
  for (int s = 0; s < 4; ++s) {
    if (s == 2) bt[4] = -1;  // page 4 becomes a null placeholder
    oracle_resolve(page, kRow, 1, C, pool_rows, pool_rows * kRow, host_rows, host_rows * kRow, 1,
                   max_pages, pool.data(), host.data(), bt.data(), hbt.data(), &ctx, hot.data(),
                   tok.data(), stp.data(), lists[s], 6, (uint32_t)(s + 1), rows.data(),
                   stats.data(), out.data());
    for (int i = 0; i < 6; ++i) check(rows[i] == want[s][i], "worked example row id");
    // every gathered row is the pool row its id names, after the step's copies
    for (int i = 0; i < 6; ++i)
      check(std::memcmp(&out[i * kRow], &pool[(size_t)rows[i] * kRow], kRow) == 0,
            "worked example gathered row");
  }
  check(stats[0] == 1 && stats[1] == 5 && stats[2] == 0, "worked example replay stats");
}

// Random tiny batches with tables that also point outside the pools, every
// entry kind, several steps: resolve, grouped resolve, gather, offload, page
// touch.
void random_cases(uint64_t seed) {
  std::mt19937_64 rs(seed);
  auto uni = [&](int64_t lo, int64_t hi) {  // [lo, hi]
    return lo + (int64_t)(rs() % (uint64_t)(hi - lo + 1));
  };
  for (int trial = 0; trial < 40; ++trial) {
    const int32_t page = 1 << uni(0, 4);
    const int32_t R = (int32_t)uni(1, 3), G = (int32_t)uni(1, 2), L = G * (int32_t)uni(1, 2);
    const int32_t C = page * (int32_t)uni(1, 4), max_pages = (int32_t)uni(1, 12);
    const int32_t n_blocks = R * (C / page) + (int32_t)uni(1, 10);
    const int32_t n_host = (int32_t)uni(1, 12);
    const int64_t pool_rows = (int64_t)n_blocks * page, host_rows = (int64_t)n_host * page;
    const int32_t N = (int32_t)uni(1, 3 * C);
    std::vector<uint8_t> pool(L * pool_rows * kRow), host(L * host_rows * kRow);
    for (auto& b : pool) b = (uint8_t)rs();
    for (auto& b : host) b = (uint8_t)rs();
    std::vector<int32_t> bt(R * max_pages), hbt(R * max_pages), ctx(R), hot(R * (C / page));
    for (auto& v : bt) v = (int32_t)uni(-2, n_blocks + 1) < n_blocks / 2 ? -1 : (int32_t)uni(-1, n_blocks + 1);
    for (auto& v : hbt) v = (int32_t)uni(-1, n_host);
    for (auto& v : ctx) v = (int32_t)uni(0, max_pages * page + 3);
    for (size_t i = 0; i < hot.size(); ++i) hot[i] = uni(0, 9) == 0 ? n_blocks + 2 : (int32_t)i;
    const int32_t NG = L / G;
    std::vector<int32_t> tok(R * NG * C, -1), topk(R * NG * N), rows(R * NG * N),
        stats(R * NG * 8);
    std::vector<uint32_t> stp(R * NG * C, 0);
    std::vector<uint8_t> out((size_t)R * L * N * kRow);
    for (int step = 0; step < 4; ++step) {
      for (auto& t : topk) {
        const int k = (int)uni(0, 9);
        t = k == 0 ? -1 : k == 1 ? (int32_t)uni(-5, max_pages * page + 5)
                                 : (int32_t)uni(0, max_pages * page - 1);
      }
      const uint32_t stamp = step == 3 ? 0xFFFFFFFFu : (uint32_t)(3 * step + 1);
      if (G == 1) {
        oracle_resolve(page, kRow, L, C, pool_rows, pool_rows * kRow, host_rows,
                       host_rows * kRow, R, max_pages, pool.data(), host.data(), bt.data(),
                       hbt.data(), ctx.data(), hot.data(), tok.data(), stp.data(), topk.data(), N,
                       stamp, rows.data(), stats.data(), step % 2 ? nullptr : out.data());
      } else {
        oracle_resolve_grouped(page, kRow, L, G, C, pool_rows, pool_rows * kRow, host_rows,
                               host_rows * kRow, R, max_pages, pool.data(), host.data(),
                               bt.data(), hbt.data(), ctx.data(), hot.data(), tok.data(),
                               stp.data(), topk.data(), N, stamp, rows.data(), stats.data(),
                               step % 2 ? nullptr : out.data());
      }
      for (int32_t rl = 0; rl < R * NG; ++rl) {
        int32_t sum = 0;
        for (int k = 0; k < 8; ++k) sum += stats[rl * 8 + k];
        check(sum == N, "stats sum to the entries");
      }
      if (G == 1) {
        oracle_gather(page, kRow, pool_rows, pool_rows * kRow, R, L, N, pool.data(), rows.data(),
                      out.data());
      }
      std::vector<int32_t> pairs;
      for (int i = 0; i < 3; ++i) {
        pairs.push_back((int32_t)uni(-1, n_blocks));
        pairs.push_back(i < n_host ? i : -1);
      }
      oracle_offload(page, kRow, L, pool_rows, pool_rows * kRow, host_rows, host_rows * kRow,
                     pool.data(), host.data(), pairs.data(), 3);
      std::vector<uint32_t> use(R * max_pages, 0);
      oracle_page_touch(page, R, max_pages, NG * N, ctx.data(), topk.data(), stamp, use.data());
    }
  }
}

// The residency policy over a run under pressure: admissions with and
// without a reused prefix, steps from random lists and from per-page stamps,
// finishes, and admissions into the freed slots.
void policy_runs(uint64_t seed) {
  std::mt19937_64 rs(seed);
  auto uni = [&](int64_t lo, int64_t hi) { return lo + (int64_t)(rs() % (uint64_t)(hi - lo + 1)); };
  const int32_t page = 16, R = 6, max_pages = 64, hot_per = 4, tail = 2;
  hs_policy_config cfg{page, 160, 400, R, max_pages, hot_per, tail};
  hs_policy* p = nullptr;
  check(hs_policy_create(&cfg, &p) == HS_POLICY_OK, "policy create");
  const int cap = 4096;
  std::vector<int32_t> bt(cap * 3), hbt(cap * 3), hot(cap * 3), reset(cap), off(cap * 2);
  hs_policy_edits e{};
  auto reset_edits = [&] {
    e = hs_policy_edits{};
    e.bt_set = bt.data(); e.cap_bt = cap;
    e.hbt_set = hbt.data(); e.cap_hbt = cap;
    e.hot_set = hot.data(); e.cap_hot = cap;
    e.reset = reset.data(); e.cap_reset = cap;
    e.offload = off.data(); e.cap_offload = cap;
  };
  std::vector<int32_t> ctx(R), reqs(R);
  std::vector<int32_t> prefix(max_pages);
  for (int32_t r = 0; r < R; ++r) {
    ctx[r] = (int32_t)uni(page * 4, page * 20);
    reqs[r] = r;
    for (int32_t pg = 0; pg < max_pages; ++pg) prefix[pg] = pg < ctx[r] / page ? r * 64 + pg : -1;
    reset_edits();
    check(hs_policy_admit(p, r, ctx[r], r % 2 ? prefix.data() : nullptr, r % 3 == 0, &e) ==
              HS_POLICY_OK, "policy admit");
  }
  const int32_t k = 24;
  std::vector<int32_t> topk(R * k);
  std::vector<uint32_t> use(R * max_pages, 0);
  for (int32_t s = 1; s <= 30; ++s) {
    for (int32_t r = 0; r < R; ++r) {
      ctx[r] = std::min(ctx[r] + (int32_t)uni(0, 9), max_pages * page - 1);
      for (int32_t i = 0; i < k; ++i) topk[r * k + i] = uni(0, 7) ? (int32_t)uni(0, ctx[r] - 1) : -1;
    }
    reset_edits();
    hs_policy_status st;
    if (s % 2) {
      st = hs_policy_step(p, s, reqs.data(), ctx.data(), R, topk.data(), k, &e);
    } else {
      oracle_page_touch(page, R, max_pages, k, ctx.data(), topk.data(), (uint32_t)s, use.data());
      st = hs_policy_step_pages(p, reqs.data(), ctx.data(), R, use.data(), max_pages, &e);
    }
    if (st != HS_POLICY_OK) break;  // an exhausted pool is a defined error, not a fault
    std::vector<int32_t> tb(max_pages), th(max_pages), tl(hot_per);
    for (int32_t r = 0; r < R; ++r)
      check(hs_policy_tables(p, r, tb.data(), th.data(), tl.data()) == HS_POLICY_OK,
            "policy tables");
    check(hs_policy_free_blocks(p) >= 0, "free blocks");
  }
  for (int32_t r = 0; r < R; ++r) {
    reset_edits();
    hs_policy_finish(p, r, &e);
  }
  hs_policy_destroy(p);
}

}  // namespace

int main() {
  worked_example();
  for (uint64_t seed = 1; seed <= 6; ++seed) random_cases(seed);
  for (uint64_t seed = 1; seed <= 4; ++seed) policy_runs(seed);
  if (g_failures) {
    std::fprintf(stderr, "%d check(s) failed\n", g_failures);
    return 1;
  }
  std::printf("sanitized oracle and policy: clean\n");
  return 0;
}
