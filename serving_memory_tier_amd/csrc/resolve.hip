// The fused top-K resolver for gfx950 (CDNA4).
//
// Method: "vLLM GLM 5.3 ... Hybrid HiSparse offloading, Part 1", section
// "How it works" (mixed residency: one fused kernel resolves the indexer's
// top-K; resident tokens are read in place, hot tokens are read and their LRU
// entry refreshed, a miss copies one row from pinned host memory into the LRU
// slot; nothing waits on the CPU) and its figure (solid arrow = one-row copy
// on a miss, dotted = reuse without copy); section "Integration with the rest
// of vLLM" (a per-step replayable plan shares the request's hot state).
//
// One workgroup (16 wave64s) resolves one request-layer.  Everything the
// decision needs lives in LDS:
//   A  load the N top-K entries (one per lane per round), classify each
//      (pad / invalid / resident / non-resident) and write the rows of every
//      entry that does not need the hot buffer;
//   B  bitonic-sort the non-pad tokens in LDS; the first element of each run
//      is a distinct token; compact the distinct non-resident ones (ballot +
//      mbcnt, order kept) into an ascending list U;
//   C  every slot binary-searches its token in U: a hit records the slot
//      (the smallest slot wins if the state ever held a token twice);
//   D  hits take the new stamp; distinct misses with a host copy are
//      compacted in ascending token order;
//   E  the usable non-hit slots are compacted in slot order and stably
//      radix-sorted by stamp (one ballot split per stamp bit that varies), so
//      they end in ascending (stamp, slot) order; the j-th miss takes the
//      j-th slot; each assigned miss streams its one row from the host pool
//      into its slot (16-byte loads over the host link, four in flight per
//      lane), and the slot's token and stamp are written back;
//   H  the non-resident entries look their token up in U and write their row.
// No step depends on the order in which lanes or waves run: every result is
// fixed by the sort and the scans, so repeated runs are bitwise identical.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "hs_internal.h"

namespace hs {
namespace {

constexpr int kThreads = kResolveThreads;
constexpr int kWaves = kThreads / 64;
constexpr int32_t kNone = 0x7fffffff;   // "no slot yet" / sort padding
constexpr int32_t kRowPad = -1;
constexpr int32_t kRowOverflow = -2;
constexpr int32_t kRowInvalid = -3;

enum : int8_t { K_EMPTY = 0, K_PAD = 1, K_INVALID = 2, K_RESIDENT = 3, K_NONRES = 4 };

// LDS carve-up (byte offsets), identical on host and device.
struct LdsPlan {
  int32_t sort_n;      // power of two >= N
  uint32_t off_keys;   // int32[max(sort_n, 2 * C / 2)]: sort keys, later victim lists
  uint32_t off_unr;    // int32[N]: ascending distinct non-resident tokens
  uint32_t off_ures;   // int32[N]: per distinct token: slot, or a negative row code
  uint32_t off_mk;     // uint16[N]: miss rank -> index into the distinct list
  uint32_t off_stp;    // uint32[C]: slot stamps
  uint32_t off_flag;   // uint8[C]: 0 free, 1 hit, 2 unusable
  uint32_t off_red;    // int32[kRed]: scan / reduction scratch
  uint32_t total;
};

constexpr int kRed = 8 * kWaves + 64;

__host__ __device__ inline uint32_t align16(uint32_t x) { return (x + 15u) & ~15u; }

__host__ __device__ inline int32_t next_pow2(int32_t n) {
  int32_t s = 1;
  while (s < n) s <<= 1;
  return s < 2 ? 2 : s;
}

__host__ __device__ inline LdsPlan make_plan(int32_t N, int32_t C) {
  LdsPlan p;
  p.sort_n = next_pow2(N);
  uint32_t keys_bytes = (uint32_t)p.sort_n * 4u;
  uint32_t vict_bytes = (uint32_t)C * 2u * 2u;  // two uint16 lists of C slots
  if (vict_bytes > keys_bytes) keys_bytes = vict_bytes;
  uint32_t o = 0;
  p.off_keys = o; o = align16(o + keys_bytes);
  p.off_unr = o;  o = align16(o + (uint32_t)N * 4u);
  p.off_ures = o; o = align16(o + (uint32_t)N * 4u);
  p.off_mk = o;   o = align16(o + (uint32_t)N * 2u);
  p.off_stp = o;  o = align16(o + (uint32_t)C * 4u);
  p.off_flag = o; o = align16(o + (uint32_t)C);
  p.off_red = o;  o = align16(o + (uint32_t)kRed * 4u);
  p.total = o;
  return p;
}

__device__ inline int lane_id() { return threadIdx.x & 63; }
__device__ inline int wave_id() { return threadIdx.x >> 6; }

__device__ inline int lanes_below(uint64_t mask) {
  return __builtin_amdgcn_mbcnt_hi((uint32_t)(mask >> 32),
                                   __builtin_amdgcn_mbcnt_lo((uint32_t)mask, 0u));
}

// Stable block-wide compaction over elements e = j * kThreads + tid, j < E:
// pos[j] = number of true predicates at smaller e; returns the total.
template <int E>
__device__ int block_compact(const bool (&pred)[E], int (&pos)[E], int* red) {
  const int w = wave_id(), l = lane_id();
  int below[E];
#pragma unroll
  for (int j = 0; j < E; ++j) {
    const uint64_t b = __ballot(pred[j]);
    below[j] = lanes_below(b);
    if (l == 0) red[j * kWaves + w] = __popcll(b);
  }
  __syncthreads();
  if (w == 0) {
    constexpr int n = E * kWaves;  // <= 128: two counts per lane
    const int i0 = 2 * l, i1 = 2 * l + 1;
    const int v0 = i0 < n ? red[i0] : 0;
    const int v1 = i1 < n ? red[i1] : 0;
    const int s = v0 + v1;
    int inc = s;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
      const int t = __shfl_up(inc, d);
      if (l >= d) inc += t;
    }
    const int ex = inc - s;
    if (i0 < n) red[i0] = ex;
    if (i1 < n) red[i1] = ex + v0;
    if (l == 63) red[n] = inc;
  }
  __syncthreads();
#pragma unroll
  for (int j = 0; j < E; ++j) pos[j] = red[j * kWaves + w] + below[j];
  const int total = red[E * kWaves];
  __syncthreads();
  return total;
}

// Block-wide sums of up to four counters at once.
__device__ inline void block_sum4(int (&v)[4], int* red) {
  const int w = wave_id(), l = lane_id();
#pragma unroll
  for (int c = 0; c < 4; ++c) {
#pragma unroll
    for (int d = 32; d >= 1; d >>= 1) v[c] += __shfl_xor(v[c], d);
    if (l == 0) red[c * kWaves + w] = v[c];
  }
  __syncthreads();
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    int t = 0;
#pragma unroll
    for (int i = 0; i < kWaves; ++i) t += red[c * kWaves + i];
    v[c] = t;
  }
  __syncthreads();
}

__device__ inline void block_minmax(uint32_t& mn, uint32_t& mx, int* red) {
  const int w = wave_id(), l = lane_id();
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) {
    mn = min(mn, (uint32_t)__shfl_xor((int)mn, d));
    mx = max(mx, (uint32_t)__shfl_xor((int)mx, d));
  }
  if (l == 0) {
    red[w] = (int)mn;
    red[kWaves + w] = (int)mx;
  }
  __syncthreads();
  mn = 0xffffffffu;
  mx = 0u;
#pragma unroll
  for (int i = 0; i < kWaves; ++i) {
    mn = min(mn, (uint32_t)red[i]);
    mx = max(mx, (uint32_t)red[kWaves + i]);
  }
  __syncthreads();
}

// Ascending bitonic sort of S (a power of two) int32 keys in LDS.
__device__ void bitonic_sort(int32_t* keys, int S) {
  for (int k = 2; k <= S; k <<= 1) {
    for (int j = k >> 1; j > 0; j >>= 1) {
      for (int i = threadIdx.x; i < (S >> 1); i += kThreads) {
        const int lo = ((i & ~(j - 1)) << 1) | (i & (j - 1));
        const int hi = lo + j;
        const int32_t a = keys[lo], b = keys[hi];
        const bool up = (lo & k) == 0;
        if ((a > b) == up) {
          keys[lo] = b;
          keys[hi] = a;
        }
      }
      __syncthreads();
    }
  }
}

__device__ inline int lower_bound(const int32_t* a, int n, int32_t v) {
  int lo = 0, hi = n;
  while (lo < hi) {
    const int mid = (lo + hi) >> 1;
    if (a[mid] < v) lo = mid + 1;
    else hi = mid;
  }
  return lo;
}

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

struct KernelArgs {
  ResolveParams p;
  LdsPlan plan;
};

// E = rounds of kThreads elements needed to cover max(sort_n, C).
// PIECES = row_bytes / 16 when known at compile time, 0 for any row size.
template <int E, int PIECES>
__global__ void __launch_bounds__(kThreads) resolve_kernel(KernelArgs args) {
  extern __shared__ __attribute__((aligned(16))) unsigned char lds[];
  const ResolveParams& p = args.p;
  const LdsPlan& plan = args.plan;
  int32_t* keys = reinterpret_cast<int32_t*>(lds + plan.off_keys);
  int32_t* unr = reinterpret_cast<int32_t*>(lds + plan.off_unr);
  int32_t* ures = reinterpret_cast<int32_t*>(lds + plan.off_ures);
  uint16_t* mk = reinterpret_cast<uint16_t*>(lds + plan.off_mk);
  uint32_t* sst = reinterpret_cast<uint32_t*>(lds + plan.off_stp);
  uint8_t* sflag = reinterpret_cast<uint8_t*>(lds + plan.off_flag);
  int* red = reinterpret_cast<int*>(lds + plan.off_red);

  const int tid = threadIdx.x;
  const int rl = blockIdx.x;
  const int r = rl / p.num_layers;
  const int layer = rl - r * p.num_layers;
  const int ps = p.page_shift;
  const int32_t pm = (1 << ps) - 1;
  const int N = p.entries, C = p.hot_capacity, S = plan.sort_n;
  const int32_t ctx = p.ctx_len[r];
  const int32_t* bt = p.block_table + (int64_t)r * p.max_pages;
  const int32_t* hbt = p.host_block_table + (int64_t)r * p.max_pages;
  const int32_t* hot = p.hot_blocks + (int64_t)r * (C >> ps);
  const int32_t* topk = p.topk + (int64_t)rl * N;
  int32_t* rows = p.row_ids + (int64_t)rl * N;
  int32_t* stok = p.slot_token + (int64_t)rl * C;
  uint32_t* sstp = p.slot_stamp + (int64_t)rl * C;
  const int64_t pool_blocks = p.pool_rows >> ps;
  const int64_t host_blocks = p.host_rows >> ps;

  // ---- A: load, classify, rows of entries that need no hot lookup --------
  int32_t t[E];
  int8_t kind[E];
  int cnt[4] = {0, 0, 0, 0};  // pads
#pragma unroll
  for (int j = 0; j < E; ++j) {
    const int e = j * kThreads + tid;
    kind[j] = K_EMPTY;
    t[j] = kNone;
    if (e < N) {
      const int32_t v = topk[e];
      t[j] = v;
      int32_t row = 0;
      if (v == -1) {
        kind[j] = K_PAD;
        row = kRowPad;
        cnt[0] += 1;
      } else if (v < 0 || v >= ctx || (v >> ps) >= p.max_pages) {
        kind[j] = K_INVALID;
        row = kRowInvalid;
      } else {
        const int32_t b = bt[v >> ps];
        if (b >= 0) {
          if (b < pool_blocks) {
            kind[j] = K_RESIDENT;
            row = (b << ps) | (v & pm);
          } else {
            kind[j] = K_INVALID;
            row = kRowInvalid;
          }
        } else {
          kind[j] = K_NONRES;
        }
      }
      if (kind[j] != K_NONRES) rows[e] = row;
    }
    if (e < S) keys[e] = (kind[j] == K_PAD || kind[j] == K_EMPTY) ? kNone : t[j];
  }
  // slot stamps and usability
#pragma unroll
  for (int j = 0; j < E; ++j) {
    const int q = j * kThreads + tid;
    if (q < C) {
      sst[q] = sstp[q];
      const int32_t hb = hot[q >> ps];
      sflag[q] = (hb >= 0 && hb < pool_blocks) ? 0 : 2;
    }
  }
  block_sum4(cnt, red);  // also the barrier before the sort
  const int pads = cnt[0];
  const int n_nonpad = N - pads;

  // ---- B: sort, distinct tokens, compact the non-resident ones ----------
  bitonic_sort(keys, S);
  bool pred[E];
  int pos[E];
  int32_t sv[E];
  int ucnt[4] = {0, 0, 0, 0};  // distinct, distinct resident, distinct invalid
#pragma unroll
  for (int j = 0; j < E; ++j) {
    const int i = j * kThreads + tid;
    pred[j] = false;
    sv[j] = 0;
    if (i < n_nonpad) {
      const int32_t v = keys[i];
      sv[j] = v;
      if (i == 0 || keys[i - 1] != v) {
        ucnt[0] += 1;
        if (v < 0 || v >= ctx || (v >> ps) >= p.max_pages) {
          ucnt[2] += 1;
        } else {
          const int32_t b = bt[v >> ps];
          if (b >= 0) {
            if (b < pool_blocks) ucnt[1] += 1;
            else ucnt[2] += 1;
          } else {
            pred[j] = true;
          }
        }
      }
    }
  }
  const int n_u = block_compact<E>(pred, pos, red);
#pragma unroll
  for (int j = 0; j < E; ++j)
    if (pred[j]) unr[pos[j]] = sv[j];
  for (int k = tid; k < n_u; k += kThreads) ures[k] = kNone;
  block_sum4(ucnt, red);  // barrier: unr and ures complete

  // ---- C: hot-map lookup (each slot searches its token) -----------------
#pragma unroll
  for (int j = 0; j < E; ++j) {
    const int q = j * kThreads + tid;
    if (q < C && sflag[q] == 0) {
      const int32_t tk = stok[q];
      if (tk >= 0 && n_u > 0) {
        const int k = lower_bound(unr, n_u, tk);
        if (k < n_u && unr[k] == tk) atomicMin(&ures[k], q);
      }
    }
  }
  __syncthreads();

  // ---- D: hits refresh their stamp; misses are listed in token order ----
  int dcnt[4] = {0, 0, 0, 0};  // hits, distinct invalid (no host copy)
#pragma unroll
  for (int j = 0; j < E; ++j) {
    const int k = j * kThreads + tid;
    pred[j] = false;
    if (k < n_u) {
      const int32_t q = ures[k];
      if (q != kNone) {
        dcnt[0] += 1;
        sflag[q] = 1;
        sstp[q] = p.stamp;
      } else {
        const int32_t u = unr[k];
        const int32_t hb = hbt[u >> ps];
        if (hb >= 0 && hb < host_blocks) {
          pred[j] = true;
        } else {
          dcnt[1] += 1;
          ures[k] = kRowInvalid;
        }
      }
    }
  }
  const int M = block_compact<E>(pred, pos, red);
#pragma unroll
  for (int j = 0; j < E; ++j)
    if (pred[j]) mk[pos[j]] = (uint16_t)(j * kThreads + tid);
  block_sum4(dcnt, red);  // barrier: mk and sflag complete

  // ---- E: victims in ascending (stamp, slot), assignment, copies --------
  int A = 0;
  if (M > 0) {
    uint16_t* vbuf0 = reinterpret_cast<uint16_t*>(keys);
    uint16_t* vbuf1 = vbuf0 + C;
    uint32_t mn = 0xffffffffu, mx = 0u;
#pragma unroll
    for (int j = 0; j < E; ++j) {
      const int q = j * kThreads + tid;
      pred[j] = q < C && sflag[q] == 0;
      if (pred[j]) {
        mn = min(mn, sst[q]);
        mx = max(mx, sst[q]);
      }
    }
    const int nv = block_compact<E>(pred, pos, red);
#pragma unroll
    for (int j = 0; j < E; ++j)
      if (pred[j]) vbuf0[pos[j]] = (uint16_t)(j * kThreads + tid);
    block_minmax(mn, mx, red);  // barrier: vbuf0 complete
    const int bits = (nv == 0 || mx == mn) ? 0 : 32 - __clz((int)(mx - mn));
    uint16_t* src = vbuf0;
    uint16_t* dst = vbuf1;
    for (int bit = 0; bit < bits; ++bit) {
      uint16_t qs[E];
      bool one[E];
#pragma unroll
      for (int j = 0; j < E; ++j) {
        const int e = j * kThreads + tid;
        qs[j] = 0;
        one[j] = false;
        if (e < nv) {
          qs[j] = src[e];
          one[j] = ((sst[qs[j]] - mn) >> bit) & 1u;
        }
        pred[j] = e < nv && !one[j];
      }
      const int zeros = block_compact<E>(pred, pos, red);
#pragma unroll
      for (int j = 0; j < E; ++j) {
        const int e = j * kThreads + tid;
        if (e < nv) dst[one[j] ? zeros + (e - pos[j]) : pos[j]] = qs[j];
      }
      __syncthreads();
      uint16_t* tmp = src;
      src = dst;
      dst = tmp;
    }
    A = M < nv ? M : nv;
    for (int j = tid; j < M; j += kThreads) {
      const int k = mk[j];
      if (j < A) {
        const int q = src[j];
        ures[k] = q;
        stok[q] = unr[k];
        sstp[q] = p.stamp;
      } else {
        ures[k] = kRowOverflow;
      }
    }
    // one row per assigned miss: host row -> hot-slot row, 16 B per lane
    const int pieces = PIECES > 0 ? PIECES : (p.row_bytes >> 4);
    const int total = A * pieces;
    const uint8_t* host_l = p.host + (int64_t)layer * p.host_stride;
    uint8_t* pool_l = p.pool + (int64_t)layer * p.pool_stride;
    constexpr int U = 4;
    for (int base = tid; base < total; base += U * kThreads) {
      u32x4 v[U];
      uint8_t* dptr[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int idx = base + u * kThreads;
        dptr[u] = nullptr;
        if (idx < total) {
          const int jj = idx / pieces;
          const int pc = idx - jj * pieces;
          const int q = src[jj];
          const int32_t tok = unr[mk[jj]];
          const int64_t srow = ((int64_t)hbt[tok >> ps] << ps) | (tok & pm);
          const int64_t drow = ((int64_t)hot[q >> ps] << ps) | (q & pm);
          v[u] = *reinterpret_cast<const u32x4*>(host_l + srow * p.row_bytes + pc * 16);
          dptr[u] = pool_l + drow * p.row_bytes + pc * 16;
        }
      }
#pragma unroll
      for (int u = 0; u < U; ++u)
        if (dptr[u]) *reinterpret_cast<u32x4*>(dptr[u]) = v[u];
    }
    __syncthreads();  // ures final
  }

  // ---- H: rows of the non-resident entries ------------------------------
#pragma unroll
  for (int j = 0; j < E; ++j) {
    if (kind[j] != K_NONRES) continue;
    const int e = j * kThreads + tid;
    const int k = lower_bound(unr, n_u, t[j]);
    // every non-resident token is in the list by construction; the guard
    // keeps a broken invariant from ever indexing past hot_blocks
    const int32_t code = (k < n_u && unr[k] == t[j]) ? ures[k] : kRowInvalid;
    rows[e] = (code >= 0 && code < C) ? ((hot[code >> ps] << ps) | (code & pm))
                                      : (code >= 0 ? kRowInvalid : code);
  }

  if (tid == 0) {
    int32_t* st = p.stats + (int64_t)rl * 8;
    st[0] = ucnt[1];
    st[1] = dcnt[0];
    st[2] = A;
    st[3] = M - A;
    st[4] = ucnt[2] + dcnt[1];
    st[5] = pads;
    st[6] = n_nonpad - ucnt[0];
    st[7] = 0;
  }
}

template <int E, int PIECES>
hipError_t launch_e(const KernelArgs& a, int grid, hipStream_t stream) {
  auto fn = resolve_kernel<E, PIECES>;
  static bool attr = false;
  if (!attr) {
    hipError_t err = hipFuncSetAttribute(reinterpret_cast<const void*>(fn),
                                         hipFuncAttributeMaxDynamicSharedMemorySize,
                                         160 * 1024);
    if (err != hipSuccess) return err;
    attr = true;
  }
  hipLaunchKernelGGL(fn, dim3(grid), dim3(kThreads), a.plan.total, stream, a);
  return hipGetLastError();
}

template <int PIECES>
hipError_t launch_pieces(const KernelArgs& a, int grid, int E, hipStream_t stream) {
  switch (E) {
    case 1: return launch_e<1, PIECES>(a, grid, stream);
    case 2: return launch_e<2, PIECES>(a, grid, stream);
    case 4: return launch_e<4, PIECES>(a, grid, stream);
    default: return launch_e<8, PIECES>(a, grid, stream);
  }
}

}  // namespace

size_t resolve_lds_bytes(int32_t entries, int32_t hot_capacity) {
  return make_plan(entries, hot_capacity).total;
}

hipError_t launch_resolve(const ResolveParams& p, hipStream_t stream) {
  KernelArgs a;
  a.p = p;
  a.plan = make_plan(p.entries, p.hot_capacity);
  const int span = a.plan.sort_n > p.hot_capacity ? a.plan.sort_n : p.hot_capacity;
  int E = (span + kThreads - 1) / kThreads;
  E = E <= 1 ? 1 : E <= 2 ? 2 : E <= 4 ? 4 : 8;
  const int grid = p.num_reqs * p.num_layers;
  if (grid == 0) return hipSuccess;
  if (p.row_bytes == 656) return launch_pieces<41>(a, grid, E, stream);
  return launch_pieces<0>(a, grid, E, stream);
}

}  // namespace hs
