// The host-side residency policy of Hybrid HiSparse (declared in
// include/hs_policy.h): GPU-first residency with pressure-driven, in-place
// eviction of each request's coldest pages, a never-evicted tail, proactive
// host copies of completed pages, and hot-buffer leases from the same block
// pool.  Host code only; it decides between decode steps and hands the GPU
// path its table and lease edits.
//
// Source: "vLLM GLM 5.3 ... Hybrid HiSparse offloading, Part 1", sections
// "Use sparsity when needed", "How it works" and "Offload only where
// needed" (the readings the pages leave open are listed in the header).

#include "hs_policy.h"

#include <algorithm>
#include <cstring>
#include <tuple>
#include <vector>

namespace {

struct Req {
  bool active = false;
  int32_t ctx = 0;
  std::vector<int32_t> bt;         // device block per page, -1 = null placeholder
  std::vector<int32_t> hbt;        // valid host copy per page, -1 = none
  std::vector<int32_t> queued_at;  // step a host copy was queued at, -1 = none
  std::vector<int32_t> host_of;    // host block of a queued or valid copy, -1 = none
  std::vector<char> own_host;      // the host block is the policy's (freed at finish)
  std::vector<uint32_t> last_use;  // coldness: last stamp a top-K list touched the page
  std::vector<int32_t> hot;        // leased blocks, empty = no lease
  int32_t copied_upto = 0;         // pages below have a host copy, valid or queued
};

struct Out {
  hs_policy_edits* e;
  bool ok = true;
  void set3(int32_t* a, int32_t& n, int32_t cap, int32_t x, int32_t y, int32_t z) {
    if (!e) return;
    if (n >= cap) {
      ok = false;
      return;
    }
    a[3 * n] = x;
    a[3 * n + 1] = y;
    a[3 * n + 2] = z;
    ++n;
  }
  void bt(int32_t r, int32_t p, int32_t v) { if (e) set3(e->bt_set, e->n_bt, e->cap_bt, r, p, v); }
  void hbt(int32_t r, int32_t p, int32_t v) { if (e) set3(e->hbt_set, e->n_hbt, e->cap_hbt, r, p, v); }
  void hot(int32_t r, int32_t j, int32_t v) { if (e) set3(e->hot_set, e->n_hot, e->cap_hot, r, j, v); }
  void reset(int32_t r) {
    if (!e) return;
    if (e->n_reset >= e->cap_reset) {
      ok = false;
      return;
    }
    e->reset[e->n_reset++] = r;
  }
  void offload(int32_t db, int32_t hb) {
    if (!e) return;
    if (e->n_offload >= e->cap_offload) {
      ok = false;
      return;
    }
    e->offload[2 * e->n_offload] = db;
    e->offload[2 * e->n_offload + 1] = hb;
    ++e->n_offload;
  }
};

void clear_counts(hs_policy_edits* e) {
  if (!e) return;
  e->n_bt = e->n_hbt = e->n_hot = e->n_reset = e->n_offload = 0;
  e->evicted = e->leased = e->returned = 0;
}

}  // namespace

struct hs_policy {
  hs_policy_config cfg;
  int32_t page_shift = 0;            // log2(page_size)
  std::vector<int32_t> free_blocks;  // popped from the back: lowest block first
  std::vector<int32_t> free_host;
  std::vector<Req> reqs;
  std::vector<std::tuple<int32_t, int32_t, int32_t>> pending;  // host copies valid next step
  int32_t step = 0;

  int32_t pages_of(int32_t ctx) const { return (ctx + cfg.page_size - 1) / cfg.page_size; }

  bool has_placeholder(const Req& q) const {
    const int32_t np = pages_of(q.ctx);
    for (int32_t p = 0; p < np; ++p)
      if (q.bt[p] < 0) return true;
    return false;
  }

  void free_block(int32_t b) { free_blocks.push_back(b); }
  int32_t take_block() {
    const int32_t b = free_blocks.back();
    free_blocks.pop_back();
    return b;
  }

  // Makes `need` blocks free, evicting the coldest eligible pages; a request
  // that gets its first placeholder (and holds no lease) adds a lease to the
  // demand.  `lease_want` marks requests already counted as needing one.
  hs_policy_status make_room(int32_t need, std::vector<char>& lease_want, Out& out) {
    if ((int32_t)free_blocks.size() >= need) return HS_POLICY_OK;
    struct Cand {
      uint32_t use;
      int32_t r, p;
    };
    std::vector<Cand> cands;
    for (int32_t r = 0; r < cfg.max_requests; ++r) {
      const Req& q = reqs[r];
      if (!q.active) continue;
      const int32_t complete = q.ctx / cfg.page_size;
      const int32_t tail_lo = pages_of(q.ctx) - cfg.tail_pages;
      for (int32_t p = 0; p < complete && p < tail_lo; ++p) {
        if (q.bt[p] < 0) continue;
        const bool copied = q.hbt[p] >= 0 || (q.queued_at[p] >= 0 && q.queued_at[p] < step);
        if (copied) cands.push_back({q.last_use[p], r, p});
      }
    }
    const auto colder = [](const Cand& a, const Cand& b) {
      if (a.use != b.use) return a.use < b.use;
      if (a.r != b.r) return a.r < b.r;
      return a.p < b.p;
    };
    // only the coldest few are needed: order them a batch at a time
    size_t i = 0, ordered = 0;
    while ((int32_t)free_blocks.size() < need) {
      if (i == cands.size()) return HS_POLICY_ERR_POOL_EXHAUSTED;
      if (i == ordered) {
        const size_t want = std::max<size_t>(64, 2 * (size_t)(need - (int32_t)free_blocks.size()));
        const size_t upto = std::min(cands.size(), ordered + want);
        std::partial_sort(cands.begin() + ordered, cands.begin() + upto, cands.end(), colder);
        ordered = upto;
      }
      const Cand c = cands[i++];
      Req& q = reqs[c.r];
      free_block(q.bt[c.p]);
      q.bt[c.p] = -1;
      out.bt(c.r, c.p, -1);
      if (out.e) ++out.e->evicted;
      if (q.hot.empty() && !lease_want[c.r]) {
        lease_want[c.r] = 1;
        need += cfg.hot_blocks_per_request;
      }
    }
    return HS_POLICY_OK;
  }

  // Grants the wanted leases (blocks must be free) and records the resets.
  void grant(std::vector<char>& lease_want, Out& out) {
    for (int32_t r = 0; r < cfg.max_requests; ++r) {
      if (!lease_want[r]) continue;
      Req& q = reqs[r];
      q.hot.resize(cfg.hot_blocks_per_request);
      for (int32_t j = 0; j < cfg.hot_blocks_per_request; ++j) {
        q.hot[j] = take_block();
        out.hot(r, j, q.hot[j]);
      }
      out.reset(r);
      if (out.e) ++out.e->leased;
      lease_want[r] = 0;
    }
  }

  // Completed pages without a host copy get one queued after the step.
  hs_policy_status queue_copies(int32_t r, Out& out) {
    Req& q = reqs[r];
    const int32_t complete = q.ctx / cfg.page_size;
    for (int32_t p = q.copied_upto; p < complete; q.copied_upto = ++p) {
      if (q.host_of[p] >= 0 || q.bt[p] < 0) continue;
      if (free_host.empty()) return HS_POLICY_ERR_HOST_EXHAUSTED;
      const int32_t hb = free_host.back();
      free_host.pop_back();
      q.host_of[p] = hb;
      q.own_host[p] = 1;
      q.queued_at[p] = step;
      out.offload(q.bt[p], hb);
      pending.emplace_back(r, p, hb);
    }
    return HS_POLICY_OK;
  }
};

namespace {

hs_policy_status check_step(const hs_policy* p, const int32_t* req, const int32_t* ctx_len,
                            int32_t n) {
  if (!p || n < 0 || (n > 0 && (!req || !ctx_len))) return HS_POLICY_ERR_INVALID_ARGUMENT;
  for (int32_t i = 0; i < n; ++i) {
    if (req[i] < 0 || req[i] >= p->cfg.max_requests || !p->reqs[req[i]].active)
      return HS_POLICY_ERR_INVALID_ARGUMENT;
    const Req& q = p->reqs[req[i]];
    if (ctx_len[i] < q.ctx || p->pages_of(ctx_len[i]) > p->cfg.max_pages)
      return HS_POLICY_ERR_INVALID_ARGUMENT;
  }
  return HS_POLICY_OK;
}

// Host copies queued after the previous step are now valid.
void publish_copies(hs_policy* p, Out& out) {
  ++p->step;
  for (const auto& t : p->pending) {
    Req& q = p->reqs[std::get<0>(t)];
    q.hbt[std::get<1>(t)] = std::get<2>(t);
    out.hbt(std::get<0>(t), std::get<1>(t), std::get<2>(t));
  }
  p->pending.clear();
}

// The rest of a step, once coldness is up to date: appended tokens take
// blocks, pressure evicts, leases are granted, completed pages are queued.
hs_policy_status finish_step(hs_policy* p, const int32_t* req, const int32_t* ctx_len,
                             int32_t n, Out& out) {
  hs_policy_status s;
  // appended tokens: new pages take blocks
  std::vector<std::pair<int32_t, int32_t>> new_pages;
  for (int32_t i = 0; i < n; ++i) {
    Req& q = p->reqs[req[i]];
    const int32_t old_np = p->pages_of(q.ctx), new_np = p->pages_of(ctx_len[i]);
    for (int32_t pg = old_np; pg < new_np; ++pg) new_pages.emplace_back(req[i], pg);
    q.ctx = ctx_len[i];
  }
  std::vector<char> lease_want(p->cfg.max_requests, 0);
  s = p->make_room((int32_t)new_pages.size(), lease_want, out);
  if (s != HS_POLICY_OK) return s;
  for (const auto& np : new_pages) {
    Req& q = p->reqs[np.first];
    q.bt[np.second] = p->take_block();
    out.bt(np.first, np.second, q.bt[np.second]);
  }
  p->grant(lease_want, out);
  // completed pages: proactive host copies, queued after the step
  for (int32_t i = 0; i < n; ++i)
    if ((s = p->queue_copies(req[i], out)) != HS_POLICY_OK) return s;
  return out.ok ? HS_POLICY_OK : HS_POLICY_ERR_INVALID_ARGUMENT;
}

}  // namespace

extern "C" {

hs_policy_status hs_policy_create(const hs_policy_config* cfg, hs_policy** out) {
  if (!cfg || !out) return HS_POLICY_ERR_INVALID_ARGUMENT;
  *out = nullptr;
  if (cfg->page_size < 1 || (cfg->page_size & (cfg->page_size - 1)) != 0 ||
      cfg->num_blocks < 0 || cfg->num_host_blocks < 0 || cfg->max_requests < 1 || cfg->max_pages < 1 || cfg->hot_blocks_per_request < 1 ||
      cfg->tail_pages < 1)
    return HS_POLICY_ERR_INVALID_ARGUMENT;
  hs_policy* p = new hs_policy();
  p->cfg = *cfg;
  while ((1 << p->page_shift) < cfg->page_size) ++p->page_shift;
  for (int32_t b = cfg->num_blocks - 1; b >= 0; --b) p->free_blocks.push_back(b);
  for (int32_t b = cfg->num_host_blocks - 1; b >= 0; --b) p->free_host.push_back(b);
  p->reqs.resize(cfg->max_requests);
  *out = p;
  return HS_POLICY_OK;
}

void hs_policy_destroy(hs_policy* p) { delete p; }

hs_policy_status hs_policy_admit(hs_policy* p, int32_t req, int32_t ctx_len,
                                 const int32_t* host_block_of_page, int32_t resident_prefix,
                                 hs_policy_edits* edits) {
  clear_counts(edits);
  if (!p || req < 0 || req >= p->cfg.max_requests || ctx_len < 1) return HS_POLICY_ERR_INVALID_ARGUMENT;
  if (p->reqs[req].active || p->pages_of(ctx_len) > p->cfg.max_pages)
    return HS_POLICY_ERR_INVALID_ARGUMENT;
  Out out{edits};
  Req& q = p->reqs[req];
  const int32_t mp = p->cfg.max_pages;
  q = Req();
  q.active = true;
  q.ctx = ctx_len;
  q.bt.assign(mp, -1);
  q.hbt.assign(mp, -1);
  q.queued_at.assign(mp, -1);
  q.host_of.assign(mp, -1);
  q.own_host.assign(mp, 0);
  q.last_use.assign(mp, 0);
  const int32_t np = p->pages_of(ctx_len), complete = ctx_len / p->cfg.page_size;
  const int32_t tail_lo = np - p->cfg.tail_pages;
  int32_t need = 0;
  std::vector<int32_t> want_pages;
  for (int32_t pg = 0; pg < np; ++pg) {
    const int32_t hb = (host_block_of_page && pg < complete) ? host_block_of_page[pg] : -1;
    if (hb >= 0) {
      q.hbt[pg] = hb;
      q.host_of[pg] = hb;
      out.hbt(req, pg, hb);
    }
    if (hb >= 0 && !resident_prefix && pg < tail_lo) {
      out.bt(req, pg, -1);  // a host-only page: a null placeholder
    } else {
      want_pages.push_back(pg);
      ++need;
    }
  }
  std::vector<char> lease_want(p->cfg.max_requests, 0);
  if ((int32_t)want_pages.size() < np) {
    lease_want[req] = 1;
    need += p->cfg.hot_blocks_per_request;
  }
  hs_policy_status s = p->make_room(need, lease_want, out);
  if (s != HS_POLICY_OK) {
    q = Req();
    return s;
  }
  for (int32_t pg : want_pages) {
    q.bt[pg] = p->take_block();
    out.bt(req, pg, q.bt[pg]);
  }
  p->grant(lease_want, out);
  return out.ok ? HS_POLICY_OK : HS_POLICY_ERR_INVALID_ARGUMENT;
}

hs_policy_status hs_policy_finish(hs_policy* p, int32_t req, hs_policy_edits* edits) {
  clear_counts(edits);
  if (!p || req < 0 || req >= p->cfg.max_requests || !p->reqs[req].active)
    return HS_POLICY_ERR_INVALID_ARGUMENT;
  Out out{edits};
  Req& q = p->reqs[req];
  const int32_t np = p->pages_of(q.ctx);
  for (int32_t pg = 0; pg < np; ++pg) {
    if (q.bt[pg] >= 0) {
      p->free_block(q.bt[pg]);
      out.bt(req, pg, -1);
    }
    if (q.own_host[pg]) p->free_host.push_back(q.host_of[pg]);
    if (q.hbt[pg] >= 0) out.hbt(req, pg, -1);
  }
  if (!q.hot.empty()) {
    for (int32_t j = 0; j < (int32_t)q.hot.size(); ++j) {
      p->free_block(q.hot[j]);
      out.hot(req, j, -1);
    }
    out.reset(req);
    if (edits) ++edits->returned;
  }
  // drop its pending host-table entries (the copies still run, in stream order)
  auto& pend = p->pending;
  pend.erase(std::remove_if(pend.begin(), pend.end(),
                            [req](const std::tuple<int32_t, int32_t, int32_t>& t) {
                              return std::get<0>(t) == req;
                            }),
             pend.end());
  q = Req();
  return out.ok ? HS_POLICY_OK : HS_POLICY_ERR_INVALID_ARGUMENT;
}

hs_policy_status hs_policy_step(hs_policy* p, int32_t stamp, const int32_t* req,
                                const int32_t* ctx_len, int32_t n, const int32_t* topk,
                                int32_t k, hs_policy_edits* edits) {
  clear_counts(edits);
  hs_policy_status s = check_step(p, req, ctx_len, n);
  if (s != HS_POLICY_OK) return s;
  if (k < 0 || (k > 0 && !topk)) return HS_POLICY_ERR_INVALID_ARGUMENT;
  Out out{edits};
  publish_copies(p, out);
  // coldness from the last step's lists
  const int32_t shift = p->page_shift;
  for (int32_t i = 0; i < n && k > 0; ++i) {
    Req& q = p->reqs[req[i]];
    const int32_t* t = topk + (int64_t)i * k;
    uint32_t* use = q.last_use.data();
    for (int32_t j = 0; j < k; ++j)
      if (t[j] >= 0 && t[j] < q.ctx) use[t[j] >> shift] = (uint32_t)stamp;
  }
  return finish_step(p, req, ctx_len, n, out);
}

hs_policy_status hs_policy_step_pages(hs_policy* p, const int32_t* req, const int32_t* ctx_len,
                                      int32_t n, const uint32_t* page_use, int32_t page_stride,
                                      hs_policy_edits* edits) {
  clear_counts(edits);
  hs_policy_status s = check_step(p, req, ctx_len, n);
  if (s != HS_POLICY_OK) return s;
  if (page_stride < 0 || (n > 0 && page_stride > 0 && !page_use))
    return HS_POLICY_ERR_INVALID_ARGUMENT;
  Out out{edits};
  publish_copies(p, out);
  // coldness from the stamps the GPU wrote per page: a page keeps the later
  // of its own stamp and the table's
  for (int32_t i = 0; i < n && page_stride > 0; ++i) {
    Req& q = p->reqs[req[i]];
    const uint32_t* u = page_use + (int64_t)i * page_stride;
    const int32_t np = std::min(p->pages_of(q.ctx), page_stride);
    for (int32_t pg = 0; pg < np; ++pg) q.last_use[pg] = std::max(q.last_use[pg], u[pg]);
  }
  return finish_step(p, req, ctx_len, n, out);
}

hs_policy_status hs_policy_tables(const hs_policy* p, int32_t req, int32_t* bt, int32_t* hbt,
                                  int32_t* hot) {
  if (!p || req < 0 || req >= p->cfg.max_requests) return HS_POLICY_ERR_INVALID_ARGUMENT;
  const Req& q = p->reqs[req];
  for (int32_t pg = 0; pg < p->cfg.max_pages; ++pg) {
    if (bt) bt[pg] = q.active ? q.bt[pg] : -1;
    if (hbt) hbt[pg] = q.active ? q.hbt[pg] : -1;
  }
  for (int32_t j = 0; j < p->cfg.hot_blocks_per_request; ++j)
    if (hot) hot[j] = (q.active && !q.hot.empty()) ? q.hot[j] : -1;
  return HS_POLICY_OK;
}

int32_t hs_policy_free_blocks(const hs_policy* p) {
  return p ? (int32_t)p->free_blocks.size() : -1;
}

}  // extern "C"
