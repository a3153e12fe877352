// The fused top-K resolver for gfx950 (CDNA4): the decision half.
//
// Method: "vLLM GLM 5.3 ... Hybrid HiSparse offloading, Part 1", section
// "How it works" (mixed residency: one fused kernel resolves the indexer's
// top-K; resident tokens are read in place, hot tokens are read and their LRU
// entry refreshed, a miss copies one row from pinned host memory into the LRU
// slot; nothing waits on the CPU) and its figure (solid arrow = one-row copy
// on a miss, dotted = reuse without copy); section "Integration with the rest
// of vLLM" (a per-step replayable plan shares the request's hot state).
//
// One workgroup (16 wave64s, 1024 threads) decides one request-layer.  The
// row movement is not done here: with a gather output the same launch also
// carries the early fill's workgroups (fill.h: every output row, the misses'
// host-link reads included, written from the pre-call state while this
// decides), and the commit kernel in copy.hip then copies each assigned
// miss's row into its slot; without one, the row mover in copy.hip runs
// next on the same stream.  Either way the host link and HBM are driven by
// the whole chip instead of one CU per request-layer.  Phases:
//   A  load the N top-K entries in sort layout, classify each (pad / invalid
//      / resident / non-resident), write the final row of every entry that
//      does not need the hot buffer;
//   B  sort the non-pad tokens: a bitonic network run in registers, lane
//      exchanges by wave shuffles, cross-wave strides through LDS (one barrier
//      each); the first element of each run is a distinct token; the distinct
//      non-resident ones are compacted (ballot + mbcnt, order kept) into an
//      ascending list U;
//   C  every slot binary-searches its token in U: a hit records the slot
//      (the smallest slot wins if the state ever held a token twice);
//   D  hits take the new stamp; distinct misses with a host copy are
//      compacted in ascending token order;
//   E  the usable non-hit slots, in ascending (stamp, slot) order, are
//      handed to the misses: if the least-recent stamp group is large enough
//      it is taken in slot order, otherwise the candidates are stably
//      radix-sorted by stamp (one ballot split per varying stamp bit); the
//      slot's token and stamp are written back;
//   H  every non-resident entry looks its token up in U and writes its row:
//      a hit's hot row, or for an assigned miss the code -(8 + 2 slot + c)
//      where c = 1 marks the single entry (the first occurrence) that will
//      copy the row into the slot; overflow -2, invalid -3.
// Nothing depends on the order in which lanes or waves run: every result is
// fixed by the sort and the scans, so repeated runs are bitwise identical.

#include <hip/hip_runtime.h>

#include <atomic>
#include <stdint.h>

#include "fill.h"
#include "hisparse.h"
#include "hs_internal.h"

// Phase markers for timing builds; empty in the library.
#ifndef HS_PHASE_MARK
#define HS_PHASE_DECL
#define HS_PHASE_MARK(i)
#define HS_PHASE_FLUSH
#endif

namespace hs {
namespace {

constexpr int kThreads = kResolveThreads;
constexpr int kWaves = kThreads / 64;
constexpr int32_t kNone = 0x7fffffff;    // "no slot yet" / sort padding
constexpr int32_t kNoHost = 0x7ffffffe;  // not resident, no host copy (unless it hits)
// ures of an assigned miss: kMissBase | first_entry << 14 | slot, so that one
// atomicMin over the token's entries marks its first occurrence
constexpr int32_t kMissBase = 1 << 30;
constexpr int kMissSlotBits = 14;                          // slots < 16384
constexpr int32_t kMissSlotMask = (1 << kMissSlotBits) - 1;
constexpr int32_t kMissInit = kMissBase | (0x1fff << kMissSlotBits);
// stamp groups taken one at a time before falling back to a full radix sort
constexpr int kMaxGroups = 16;
constexpr int32_t kRowPad = -1;
constexpr int32_t kRowOverflow = -2;
constexpr int32_t kRowInvalid = -3;

enum : uint32_t { K_EMPTY = 0, K_PAD = 1, K_OTHER = 2, K_NONRES = 3 };

// LDS carve-up (byte offsets), identical on host and device.
struct LdsPlan {
  int32_t sort_n;      // kThreads * ES >= N
  uint32_t off_keys;   // int32[max(sort_n, C, N)]: sorted keys; then two uint16
                       // victim lists of C; then first-occurrence indices
  uint32_t off_unr;    // int32[max(N, sort_n / 2)]: distinct non-resident tokens
  uint32_t off_ures;   // int32[max(N, sort_n / 2)]: per distinct token: slot or code
                       // (unr and ures together are the sort's exchange buffer)
  uint32_t off_mk;     // uint16[N]: miss rank -> index into the distinct list
  uint32_t off_flag;   // uint8[C]: 0 free, 1 hit, 2 unusable
  uint32_t off_red;    // int32[kRed]: scan / reduction scratch
  uint32_t off_bits;   // uint32[bits_words]: membership filter of the distinct list
  int32_t bits_log2;   // log2 of the filter's size in bits
  uint32_t total;
};

constexpr int kRed = 256;

__host__ __device__ inline uint32_t align16(uint32_t x) { return (x + 15u) & ~15u; }
__host__ __device__ inline int32_t imax(int32_t a, int32_t b) { return a > b ? a : b; }

__host__ __device__ inline LdsPlan make_plan(int32_t N, int32_t C, int32_t ES) {
  LdsPlan p;
  p.sort_n = kThreads * ES;
  const int32_t half = imax(N, p.sort_n / 2);
  uint32_t o = 0;
  p.off_keys = o; o = align16(o + 4u * (uint32_t)imax(imax(p.sort_n, C), N));
  p.off_unr = o;  o += 4u * (uint32_t)half;   // contiguous with ures (sort exchange)
  p.off_ures = o; o = align16(o + 4u * (uint32_t)half);
  p.off_mk = o;   o = align16(o + 2u * (uint32_t)N);
  p.off_flag = o; o = align16(o + (uint32_t)C);
  p.off_red = o;  o = align16(o + 4u * (uint32_t)kRed);
  // 4 filter bits per possible distinct token (at least 4096): a slot whose
  // token is not in the list almost always finds its bit clear
  int32_t fb = 12;
  while ((1 << fb) < 4 * N) ++fb;
  p.bits_log2 = fb;
  p.off_bits = o; o = align16(o + (uint32_t)(1u << fb) / 8u);
  p.total = o;
  return p;
}

__device__ inline int lane_id() { return threadIdx.x & 63; }
__device__ inline int wave_id() { return threadIdx.x >> 6; }

__device__ inline int lanes_below(uint64_t mask) {
  return __builtin_amdgcn_mbcnt_hi((uint32_t)(mask >> 32),
                                   __builtin_amdgcn_mbcnt_lo((uint32_t)mask, 0u));
}

// x ^ lane distance J within a wave64, for compile-time J: DPP moves for 1, 2,
// 4 and 8 (quad permutes, half-row mirror + quad mirror, row rotate by 8),
// a swizzle for 16, a permute through the LDS crossbar for 32.
template <int J>
__device__ __forceinline__ int32_t lane_xor(int32_t v) {
  if constexpr (J == 1) {
    return __builtin_amdgcn_update_dpp(0, v, 0xB1, 0xF, 0xF, false);   // quad_perm [1,0,3,2]
  } else if constexpr (J == 2) {
    return __builtin_amdgcn_update_dpp(0, v, 0x4E, 0xF, 0xF, false);   // quad_perm [2,3,0,1]
  } else if constexpr (J == 4) {
    const int32_t m = __builtin_amdgcn_update_dpp(0, v, 0x141, 0xF, 0xF, false);  // half mirror
    return __builtin_amdgcn_update_dpp(0, m, 0x1B, 0xF, 0xF, false);   // quad_perm [3,2,1,0]
  } else if constexpr (J == 8) {
    return __builtin_amdgcn_update_dpp(0, v, 0x128, 0xF, 0xF, false);  // row_ror:8
  } else if constexpr (J == 16) {
    return __builtin_amdgcn_ds_swizzle(v, 0x401F);                     // xor 16 in 32 lanes
  } else {
    return __shfl_xor(v, J);
  }
}

// Wave64 reductions by DPP/swizzle butterflies within each 32-lane half, the
// halves joined through two lane reads; the result is wave-uniform.
__device__ __forceinline__ int wave_sum(int v) {
  v += lane_xor<1>(v);
  v += lane_xor<2>(v);
  v += lane_xor<4>(v);
  v += lane_xor<8>(v);
  v += lane_xor<16>(v);
  return __builtin_amdgcn_readlane(v, 0) + __builtin_amdgcn_readlane(v, 32);
}

// Inclusive prefix sum over the 64 lanes: row shifts within rows of 16, then
// row broadcasts of lanes 15 and 31 into the rows above.
__device__ __forceinline__ int wave_incl_scan(int v) {
  v += __builtin_amdgcn_update_dpp(0, v, 0x111, 0xF, 0xF, true);   // row_shr:1
  v += __builtin_amdgcn_update_dpp(0, v, 0x112, 0xF, 0xF, true);   // row_shr:2
  v += __builtin_amdgcn_update_dpp(0, v, 0x114, 0xF, 0xF, true);   // row_shr:4
  v += __builtin_amdgcn_update_dpp(0, v, 0x118, 0xF, 0xF, true);   // row_shr:8
  v += __builtin_amdgcn_update_dpp(0, v, 0x142, 0xA, 0xF, false);  // row_bcast:15
  v += __builtin_amdgcn_update_dpp(0, v, 0x143, 0xC, 0xF, false);  // row_bcast:31
  return v;
}

// Filter position of a token: a multiplicative hash (Knuth) on `log2` bits.
__device__ inline uint32_t filter_bit(int32_t t, int log2) {
  return ((uint32_t)t * 0x9E3779B1u) >> (32 - log2);
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
    constexpr int n = E * kWaves;            // < kRed
    constexpr int per = (n + 63) / 64;       // consecutive counts per lane
    int v[per];
    int s = 0;
#pragma unroll
    for (int k = 0; k < per; ++k) {
      const int i = per * l + k;
      v[k] = i < n ? red[i] : 0;
      s += v[k];
    }
    const int inc = wave_incl_scan(s);
    int ex = inc - s;
#pragma unroll
    for (int k = 0; k < per; ++k) {
      const int i = per * l + k;
      if (i < n) red[i] = ex;
      ex += v[k];
    }
    if (l == 63) red[n] = inc;
  }
  __syncthreads();
#pragma unroll
  for (int j = 0; j < E; ++j) pos[j] = red[j * kWaves + w] + below[j];
  const int total = red[E * kWaves];
  __syncthreads();
  return total;
}

// block_compact plus block-wide sums of NS per-thread counters, in the same
// two barriers (and the trailing one).
template <int E, int NS>
__device__ int block_compact_sum(const bool (&pred)[E], int (&pos)[E], int (&sums)[NS],
                                 int* red) {
  const int w = wave_id(), l = lane_id();
  constexpr int n = E * kWaves;
  int below[E];
#pragma unroll
  for (int j = 0; j < E; ++j) {
    const uint64_t b = __ballot(pred[j]);
    below[j] = lanes_below(b);
    if (l == 0) red[j * kWaves + w] = __popcll(b);
  }
#pragma unroll
  for (int c = 0; c < NS; ++c) {
    sums[c] = wave_sum(sums[c]);
    if (l == 0) red[n + 1 + c * kWaves + w] = sums[c];
  }
  __syncthreads();
  if (w == 0) {
    const int i0 = 2 * l, i1 = 2 * l + 1;
    const int v0 = i0 < n ? red[i0] : 0;
    const int v1 = i1 < n ? red[i1] : 0;
    const int s = v0 + v1;
    const int inc = wave_incl_scan(s);
    const int ex = inc - s;
    if (i0 < n) red[i0] = ex;
    if (i1 < n) red[i1] = ex + v0;
    if (l == 63) red[n] = inc;
  }
  __syncthreads();
#pragma unroll
  for (int j = 0; j < E; ++j) pos[j] = red[j * kWaves + w] + below[j];
  const int total = red[n];
#pragma unroll
  for (int c = 0; c < NS; ++c) sums[c] = wave_sum(l < kWaves ? red[n + 1 + c * kWaves + l] : 0);
  __syncthreads();
  return total;
}

// Block-wide (smallest value, how many hold it, sum of s): v = 0xffffffff
// with c = 0 means "none".
__device__ inline void block_mincount(uint32_t& v, int& c, int& s, int* red) {
  const int w = wave_id(), l = lane_id();
  // (value, count) combine: keep the smaller value, add counts on ties
  auto comb = [&](uint32_t ov, int oc) {
    if (ov < v) {
      v = ov;
      c = oc;
    } else if (ov == v) {
      c += oc;
    }
  };
  comb((uint32_t)lane_xor<1>((int)v), lane_xor<1>(c));
  comb((uint32_t)lane_xor<2>((int)v), lane_xor<2>(c));
  comb((uint32_t)lane_xor<4>((int)v), lane_xor<4>(c));
  comb((uint32_t)lane_xor<8>((int)v), lane_xor<8>(c));
  comb((uint32_t)lane_xor<16>((int)v), lane_xor<16>(c));
  {
    const uint32_t v0 = (uint32_t)__builtin_amdgcn_readlane((int)v, 0);
    const int c0 = __builtin_amdgcn_readlane(c, 0);
    const uint32_t v1 = (uint32_t)__builtin_amdgcn_readlane((int)v, 32);
    const int c1 = __builtin_amdgcn_readlane(c, 32);
    v = v0;
    c = c0;
    comb(v1, c1);
  }
  s = wave_sum(s);
  if (l == 0) {
    red[w] = (int)v;
    red[kWaves + w] = c;
    red[2 * kWaves + w] = s;
  }
  __syncthreads();
  v = l < kWaves ? (uint32_t)red[l] : 0xffffffffu;
  c = l < kWaves ? red[kWaves + l] : 0;
  s = wave_sum(l < kWaves ? red[2 * kWaves + l] : 0);
  comb((uint32_t)lane_xor<1>((int)v), lane_xor<1>(c));
  comb((uint32_t)lane_xor<2>((int)v), lane_xor<2>(c));
  comb((uint32_t)lane_xor<4>((int)v), lane_xor<4>(c));
  comb((uint32_t)lane_xor<8>((int)v), lane_xor<8>(c));
  comb((uint32_t)lane_xor<16>((int)v), lane_xor<16>(c));
  v = (uint32_t)__builtin_amdgcn_readlane((int)v, 0);
  c = __builtin_amdgcn_readlane(c, 0);
  __syncthreads();
}

// lower_bound of E values in the ascending list a[0..n) at once: a fixed,
// lane-uniform number of steps, so the E searches overlap their LDS latency.
template <int E>
__device__ inline void lower_bound_multi(const int32_t* a, int n, const int32_t (&v)[E],
                                         int (&k)[E]) {
  int step = 1;
  while (step * 2 <= n) step *= 2;
#pragma unroll
  for (int j = 0; j < E; ++j) k[j] = 0;
  for (; step > 0; step >>= 1) {
#pragma unroll
    for (int j = 0; j < E; ++j)
      if (k[j] + step <= n && a[k[j] + step - 1] < v[j]) k[j] += step;
  }
}

// Block-wide sums of four counters at once.
__device__ inline void block_sum4(int (&v)[4], int* red) {
  const int w = wave_id(), l = lane_id();
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    v[c] = wave_sum(v[c]);
    if (l == 0) red[c * kWaves + w] = v[c];
  }
  __syncthreads();
#pragma unroll
  for (int c = 0; c < 4; ++c) v[c] = wave_sum(l < kWaves ? red[c * kWaves + l] : 0);
  __syncthreads();
}

__device__ inline void block_minmax(uint32_t& mn, uint32_t& mx, int* red) {
  const int w = wave_id(), l = lane_id();
  mn = min(mn, (uint32_t)lane_xor<1>((int)mn));
  mx = max(mx, (uint32_t)lane_xor<1>((int)mx));
  mn = min(mn, (uint32_t)lane_xor<2>((int)mn));
  mx = max(mx, (uint32_t)lane_xor<2>((int)mx));
  mn = min(mn, (uint32_t)lane_xor<4>((int)mn));
  mx = max(mx, (uint32_t)lane_xor<4>((int)mx));
  mn = min(mn, (uint32_t)lane_xor<8>((int)mn));
  mx = max(mx, (uint32_t)lane_xor<8>((int)mx));
  mn = min(mn, (uint32_t)lane_xor<16>((int)mn));
  mx = max(mx, (uint32_t)lane_xor<16>((int)mx));
  mn = min((uint32_t)__builtin_amdgcn_readlane((int)mn, 0),
           (uint32_t)__builtin_amdgcn_readlane((int)mn, 32));
  mx = max((uint32_t)__builtin_amdgcn_readlane((int)mx, 0),
           (uint32_t)__builtin_amdgcn_readlane((int)mx, 32));
  if (l == 0) {
    red[w] = (int)mn;
    red[kWaves + w] = (int)mx;
  }
  __syncthreads();
  mn = l < kWaves ? (uint32_t)red[l] : 0xffffffffu;
  mx = l < kWaves ? (uint32_t)red[kWaves + l] : 0u;
  mn = min(mn, (uint32_t)lane_xor<1>((int)mn));
  mx = max(mx, (uint32_t)lane_xor<1>((int)mx));
  mn = min(mn, (uint32_t)lane_xor<2>((int)mn));
  mx = max(mx, (uint32_t)lane_xor<2>((int)mx));
  mn = min(mn, (uint32_t)lane_xor<4>((int)mn));
  mx = max(mx, (uint32_t)lane_xor<4>((int)mx));
  mn = min(mn, (uint32_t)lane_xor<8>((int)mn));
  mx = max(mx, (uint32_t)lane_xor<8>((int)mx));
  mn = (uint32_t)__builtin_amdgcn_readlane((int)min(mn, (uint32_t)lane_xor<16>((int)mn)), 0);
  mx = (uint32_t)__builtin_amdgcn_readlane((int)max(mx, (uint32_t)lane_xor<16>((int)mx)), 0);
  __syncthreads();
}

// One stage (k = K, j = J) of an ascending bitonic network over kThreads * ES
// keys held in registers: element i = wave * 64 * ES + s * 64 + lane is x[s].
// Strides below 64 exchange with lane_xor, strides within a thread swap
// registers, strides across waves go through LDS.  Cross-wave stages use two
// buffers in turn, so each needs one barrier: a buffer is written again only
// two cross-wave stages later, after every reader has passed the barrier in
// between.  XW counts the cross-wave stages done so far.
template <int ES, int K, int J, int XW>
__device__ __forceinline__ void bitonic_stage(int32_t (&x)[ES], int32_t* b0, int32_t* b1,
                                              int base, int l) {
  constexpr int S = kThreads * ES;
  constexpr int WSPAN = 64 * ES;
  constexpr bool cross = J >= WSPAN;
  if constexpr (cross) {
    int32_t* b = (XW & 1) ? b1 : b0;
#pragma unroll
    for (int s = 0; s < ES; ++s) b[base + s * 64 + l] = x[s];
    __syncthreads();
#pragma unroll
    for (int s = 0; s < ES; ++s) {
      const int i = base + s * 64 + l;
      const int32_t y = b[i ^ J];
      const bool up = (i & K) == 0;
      const bool lower = (i & J) == 0;
      x[s] = (lower == up) ? min(x[s], y) : max(x[s], y);
    }
  } else if constexpr (J >= 64) {
    constexpr int js = J / 64;
#pragma unroll
    for (int s = 0; s < ES; ++s) {
      if ((s & js) == 0) {
        const int i = base + s * 64 + l;
        const bool up = (i & K) == 0;
        const int32_t a = x[s], c = x[s | js];
        const int32_t lo = min(a, c), hi = max(a, c);
        x[s] = up ? lo : hi;
        x[s | js] = up ? hi : lo;
      }
    }
  } else {
    const bool lower = (l & J) == 0;
#pragma unroll
    for (int s = 0; s < ES; ++s) {
      const int i = base + s * 64 + l;
      const bool up = (i & K) == 0;
      const int32_t y = lane_xor<J>(x[s]);
      x[s] = (lower == up) ? min(x[s], y) : max(x[s], y);
    }
  }
  constexpr int XW2 = XW + (cross ? 1 : 0);
  if constexpr (J > 1) {
    bitonic_stage<ES, K, J / 2, XW2>(x, b0, b1, base, l);
  } else if constexpr (K < S) {
    bitonic_stage<ES, 2 * K, K, XW2>(x, b0, b1, base, l);
  }
}

// Ascending sort of the kThreads * ES keys; ends with a barrier, so the buffers
// may be reused at once.
template <int ES>
__device__ __forceinline__ void bitonic_sort_regs(int32_t (&x)[ES], int32_t* b0, int32_t* b1) {
  const int l = lane_id(), w = wave_id();
  bitonic_stage<ES, 2, 1, 0>(x, b0, b1, w * 64 * ES, l);
  __syncthreads();
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

struct KernelArgs {
  ResolveParams p;
  LdsPlan plan;
  FetchParams fill;  // the fused fill's workgroups (FILL launches)
  int32_t n_rl;
  uint32_t lds_bytes;
  int32_t interleave;  // FILL: resolvers and gathers alternate in groups of 8 (see below)
};

// ES: sort elements per thread (kThreads * ES >= N); EC: slots per thread
// (kThreads * EC >= C).
// All global stores happen after the last barrier, so no barrier ever waits
// for store acknowledgements.
// FILL: the launch also carries the early fill's workgroups (fill.h) -- its
// miss workgroups first, so that the host-link reads start at once, then one
// resolver workgroup per request-layer, then the fill's gather workgroups.
// The two kinds never wait on each other; they share the launch so that the
// step needs no second stream and no cross-queue join.  When the resolvers
// alone would hold more than half of one round of the chip (many
// request-layers), the resolvers and the gathers alternate in groups of 8
// workgroups (one a XCD) instead, so that HBM is busy from the start rather
// than after rounds of resolvers, whose time is latency, not bytes: position
// j after the miss workgroups is the resolver of rank (resolvers before it)
// when j % 16 < 8 and resolvers remain, otherwise gather j - (resolvers
// before it).
template <int ES, int EC, bool FILL>
__global__ void __launch_bounds__(kThreads) resolve_kernel(KernelArgs args) {
  extern __shared__ __attribute__((aligned(16))) unsigned char lds[];
  int rl = blockIdx.x;
  if constexpr (FILL) {
    const int32_t b = blockIdx.x;
    const int32_t mg = args.fill.miss_groups;
    int32_t fi = b;  // the fill's workgroup index, or -1 for a resolver
    if (b >= mg) {
      const int32_t j = b - mg;
      if (args.interleave) {
        const int32_t before = min(args.n_rl, (j >> 4) * 8 + min(j & 15, 8));
        fi = (j & 15) < 8 && before < args.n_rl ? -1 : mg + j - before;
        rl = before;
      } else {
        fi = j < args.n_rl ? -1 : b - args.n_rl;
        rl = j;
      }
    }
    if (fi >= 0) {
      fill::fill_block(args.fill, reinterpret_cast<int32_t*>(lds), fi);
      return;
    }
  }
  const ResolveParams& p = args.p;
  const LdsPlan& plan = args.plan;
  int32_t* keys = reinterpret_cast<int32_t*>(lds + plan.off_keys);
  int32_t* unr = reinterpret_cast<int32_t*>(lds + plan.off_unr);
  int32_t* ures = reinterpret_cast<int32_t*>(lds + plan.off_ures);
  uint16_t* mk = reinterpret_cast<uint16_t*>(lds + plan.off_mk);
  uint8_t* sflag = reinterpret_cast<uint8_t*>(lds + plan.off_flag);
  int* red = reinterpret_cast<int*>(lds + plan.off_red);
  uint32_t* fbits = reinterpret_cast<uint32_t*>(lds + plan.off_bits);
  const int fb = plan.bits_log2;

  const int tid = threadIdx.x;
  const int l = lane_id(), w = wave_id();
  const int r = rl / p.num_layers;
  const int ps = p.page_shift;
  const int32_t pm = (1 << ps) - 1;
  const int N = p.entries, C = p.hot_capacity;
  const int32_t ctx = p.ctx_len[r];
  const int32_t* bt = p.block_table + (int64_t)r * p.max_pages;
  const int32_t* hbt = p.host_block_table + (int64_t)r * p.max_pages;
  const int32_t* hot = p.hot_blocks + (int64_t)r * (C >> ps);
  const int32_t* topk = p.topk + (int64_t)rl * N;
  int32_t* rows = p.row_ids + (int64_t)rl * N;
  const int32_t* stok = p.slot_token + (int64_t)rl * C;
  uint32_t* sstp = p.slot_stamp + (int64_t)rl * C;
  const int64_t pool_blocks = p.pool_rows >> ps;
  const int64_t host_blocks = p.host_rows >> ps;
  const int sbase = w * 64 * ES + l;  // element s of this thread: sbase + 64 * s

  HS_PHASE_DECL;
  HS_PHASE_MARK(0);
  // ---- A: load in sort layout and classify; stage the slots ------------
  int32_t x[ES];     // sort keys
  int32_t tv[ES];    // the entries' tokens
  int32_t rowA[ES];  // final rows of entries that need no hot lookup
  uint32_t kinds = 0;  // 2 bits per entry
  int cnt[4] = {0, 0, 0, 0};
#pragma unroll
  for (int s = 0; s < ES; ++s) {
    const int i = sbase + 64 * s;
    x[s] = kNone;
    tv[s] = kNone;
    rowA[s] = 0;
    if (i < N) tv[s] = topk[i];
  }
  int32_t btv[ES], hbv[ES];
#pragma unroll
  for (int s = 0; s < ES; ++s) {
    const int32_t v = tv[s];
    const bool inrange = sbase + 64 * s < N && v >= 0 && v < ctx && (v >> ps) < p.max_pages;
    // the host-table entry is fetched with the block-table entry: it warms the
    // lines the distinct-token pass reads again
    btv[s] = inrange ? bt[v >> ps] : -1;
    hbv[s] = inrange ? hbt[v >> ps] : -1;
  }
  for (int wi = tid; wi < (1 << fb) / 32; wi += kThreads) fbits[wi] = 0u;
  // each thread keeps its slots' tokens and stamps in registers
  int32_t tokq[EC];
  uint32_t cst[EC];
#pragma unroll
  for (int j = 0; j < EC; ++j) {
    const int q = j * kThreads + tid;
    tokq[j] = -1;
    cst[j] = 0xffffffffu;
    if (q < C) {
      tokq[j] = stok[q];
      cst[j] = sstp[q];
      const int32_t hb = hot[q >> ps];
      sflag[q] = (hb >= 0 && hb < pool_blocks) ? 0 : 2;
    }
  }
#pragma unroll
  for (int s = 0; s < ES; ++s) {
    const int i = sbase + 64 * s;
    if (i >= N) continue;
    const int32_t v = tv[s];
    uint32_t kind = K_OTHER;
    if (v == -1) {
      kind = K_PAD;
      rowA[s] = kRowPad;
      cnt[0] += 1;
    } else if (v < 0 || v >= ctx || (v >> ps) >= p.max_pages) {
      rowA[s] = kRowInvalid;
    } else if (btv[s] < 0) {
      kind = K_NONRES;
      cnt[1] += hbv[s] < 0 ? 1 : 0;  // keeps the warming load alive
    } else {
      rowA[s] = btv[s] < pool_blocks ? ((btv[s] << ps) | (v & pm)) : kRowInvalid;
    }
    if (kind != K_PAD) x[s] = v;
    kinds |= kind << (2 * s);
  }

  HS_PHASE_MARK(1);
  // ---- B: sort, distinct tokens, compact the non-resident ones ----------
  bitonic_sort_regs<ES>(x, keys, unr);
#pragma unroll
  for (int s = 0; s < ES; ++s) keys[sbase + 64 * s] = x[s];
  block_sum4(cnt, red);  // barrier: keys complete
  HS_PHASE_MARK(2);
  const int pads = cnt[0];
  const int n_nonpad = N - pads;

  bool predS[ES];
  int posS[ES];
  int32_t sv[ES], sinit[ES];
  int ucnt[3] = {0, 0, 0};  // distinct, distinct resident, distinct invalid
#pragma unroll
  for (int j = 0; j < ES; ++j) {
    const int i = j * kThreads + tid;
    predS[j] = false;
    sv[j] = 0;
    sinit[j] = kNone;
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
            predS[j] = true;
            const int32_t hb = hbt[v >> ps];
            sinit[j] = (hb >= 0 && hb < host_blocks) ? kNone : kNoHost;
          }
        }
      }
    }
  }
  const int n_u = block_compact_sum<ES, 3>(predS, posS, ucnt, red);
#pragma unroll
  for (int j = 0; j < ES; ++j)
    if (predS[j]) {
      unr[posS[j]] = sv[j];
      ures[posS[j]] = sinit[j];
      const uint32_t fbit = filter_bit(sv[j], fb);
      atomicOr(&fbits[fbit >> 5], 1u << (fbit & 31));
    }
  __syncthreads();  // unr, ures and the filter complete

  HS_PHASE_MARK(3);
  // ---- C: hot-map lookup (each slot searches its token) -----------------
  if (n_u > 0) {
#pragma unroll
    for (int j = 0; j < EC; ++j) {
      const int q = j * kThreads + tid;
      const int32_t tk = tokq[j];
      if (q < C && tk >= 0 && sflag[q] == 0) {
        const uint32_t fbit = filter_bit(tk, fb);
        if ((fbits[fbit >> 5] >> (fbit & 31)) & 1u) {
          const int k = lower_bound(unr, n_u, tk);
          if (k < n_u && unr[k] == tk) atomicMin(&ures[k], q);
        }
      }
    }
  }
  __syncthreads();

  HS_PHASE_MARK(4);
  // ---- D: hits are marked; misses are listed in token order -------------
  int dcnt[2] = {0, 0};  // hits, distinct invalid (no host copy)
#pragma unroll
  for (int j = 0; j < ES; ++j) {
    const int k = j * kThreads + tid;
    predS[j] = false;
    if (k < n_u) {
      const int32_t q = ures[k];
      if (q < C) {
        dcnt[0] += 1;
        sflag[q] = 1;
      } else if (q == kNoHost) {
        dcnt[1] += 1;
        ures[k] = kRowInvalid;
      } else {
        predS[j] = true;
      }
    }
  }
  const int M = block_compact_sum<ES, 2>(predS, posS, dcnt, red);
#pragma unroll
  for (int j = 0; j < ES; ++j)
    if (predS[j]) mk[posS[j]] = (uint16_t)(j * kThreads + tid);

  HS_PHASE_MARK(5);
  // ---- E: victims in ascending (stamp, slot); assignment -----------------
  int A = 0;
  uint16_t* vict = reinterpret_cast<uint16_t*>(keys);
  if (M > 0) {
    bool predC[EC];
    int posC[EC];
    // the least-recent stamp among the usable non-hit slots, its group size,
    // and the number of such slots.  Candidacy is a bit per slot round, not a
    // stamp value: every uint32 is a legal stamp, 0xffffffff included, so no
    // stamp can mark a hit or unusable slot.
    uint32_t v = 0xffffffffu;
    int c = 0, nv = 0;
    uint32_t candm = 0;  // bit j: this thread's slot j * kThreads + tid is a candidate
    static_assert(EC <= 32, "candidate bits");
#pragma unroll
    for (int j = 0; j < EC; ++j) {
      const int q = j * kThreads + tid;
      const bool cand = q < C && sflag[q] == 0;
      candm |= cand ? (1u << j) : 0u;
      nv += cand ? 1 : 0;
      if (cand) {
        if (cst[j] < v) {
          v = cst[j];
          c = 1;
        } else if (cst[j] == v) {
          c += 1;
        }
      }
    }
    block_mincount(v, c, nv, red);
    A = M < nv ? M : nv;
    // take whole stamp groups, least recent first, each in slot order; the
    // victims of a step normally span a few groups
    int taken = 0, groups = 0;
    bool fallback = false;
#pragma unroll 1
    while (taken < A) {
      const int take = c < A - taken ? c : A - taken;
      const uint32_t gv = v;
#pragma unroll
      for (int j = 0; j < EC; ++j) predC[j] = ((candm >> j) & 1u) && cst[j] == gv;
      block_compact<EC>(predC, posC, red);
#pragma unroll
      for (int j = 0; j < EC; ++j)
        if (predC[j] && posC[j] < take) vict[taken + posC[j]] = (uint16_t)(j * kThreads + tid);
      taken += take;
      if (taken >= A) break;
      if (++groups >= kMaxGroups) {
        fallback = true;
        break;
      }
      uint32_t v2 = 0xffffffffu;
      int c2 = 0, dummy = 0;
#pragma unroll
      for (int j = 0; j < EC; ++j) {
        const uint32_t st = cst[j];
        if (((candm >> j) & 1u) && st > gv) {
          if (st < v2) {
            v2 = st;
            c2 = 1;
          } else if (st == v2) {
            c2 += 1;
          }
        }
      }
      block_mincount(v2, c2, dummy, red);
      v = v2;
      c = c2;
    }
    __syncthreads();  // vict complete
    if (fallback) {
      // many stamp groups: stable radix sort of all candidates by stamp
      uint16_t* vbuf0 = reinterpret_cast<uint16_t*>(keys);
      uint16_t* vbuf1 = vbuf0 + C;
      uint32_t mn = 0xffffffffu, mx = 0u;
#pragma unroll
      for (int j = 0; j < EC; ++j) {
        predC[j] = ((candm >> j) & 1u) != 0;
        if (predC[j]) {
          mn = min(mn, cst[j]);
          mx = max(mx, cst[j]);
        }
      }
      block_minmax(mn, mx, red);
      block_compact<EC>(predC, posC, red);
#pragma unroll
      for (int j = 0; j < EC; ++j)
        if (predC[j]) vbuf0[posC[j]] = (uint16_t)(j * kThreads + tid);
      __syncthreads();
      const int bits = mx == mn ? 0 : 32 - __clz((int)(mx - mn));
      uint16_t* srcb = vbuf0;
      uint16_t* dstb = vbuf1;
      for (int bit = 0; bit < bits; ++bit) {
        uint16_t qs[EC];
        bool one[EC];
#pragma unroll
        for (int j = 0; j < EC; ++j) {
          const int e = j * kThreads + tid;
          qs[j] = 0;
          one[j] = false;
          if (e < nv) {
            qs[j] = srcb[e];
            // the pre-call stamps: nothing is stored before the last barrier
            one[j] = ((sstp[qs[j]] - mn) >> bit) & 1u;
          }
          predC[j] = e < nv && !one[j];
        }
        const int zeros = block_compact<EC>(predC, posC, red);
#pragma unroll
        for (int j = 0; j < EC; ++j) {
          const int e = j * kThreads + tid;
          if (e < nv) dstb[one[j] ? zeros + (e - posC[j]) : posC[j]] = qs[j];
        }
        __syncthreads();
        uint16_t* tmp = srcb;
        srcb = dstb;
        dstb = tmp;
      }
      vict = srcb;
    }
    HS_PHASE_MARK(6);
    for (int j = tid; j < M; j += kThreads)
      ures[mk[j]] = j < A ? (kMissInit | (int32_t)vict[j]) : kRowOverflow;
    __syncthreads();  // ures final
  }

  HS_PHASE_MARK(7);
  // ---- H: rows of the non-resident entries ------------------------------
  int kk[ES];
#pragma unroll
  for (int s = 0; s < ES; ++s) {
    kk[s] = -1;
    if (((kinds >> (2 * s)) & 3u) != K_NONRES) continue;
    const int k = lower_bound(unr, n_u, tv[s]);
    // every non-resident token is in the list by construction; the guard
    // keeps a broken invariant from ever indexing past the slot arrays
    if (k < n_u && unr[k] == tv[s]) kk[s] = k;
    if (A > 0 && kk[s] >= 0) {
      const int32_t code = ures[kk[s]];
      if (code >= kMissBase && code != kNone)
        atomicMin(&ures[kk[s]],
                  kMissBase | ((sbase + 64 * s) << kMissSlotBits) | (code & kMissSlotMask));
    }
  }
  if (A > 0) __syncthreads();
#pragma unroll
  for (int s = 0; s < ES; ++s) {
    if (((kinds >> (2 * s)) & 3u) != K_NONRES) continue;
    const int i = sbase + 64 * s;
    int32_t row = kRowInvalid;
    if (kk[s] >= 0) {
      const int32_t code = ures[kk[s]];
      if (code >= kMissBase && code != kNone) {
        const int32_t q = code & kMissSlotMask;
        row = -(8 + 2 * q + (((code >> kMissSlotBits) & 0x1fff) == i ? 1 : 0));
      } else if (code >= 0 && code < C) {
        row = (hot[code >> ps] << ps) | (code & pm);
      } else if (code < 0) {
        row = code;
      }
    }
    rowA[s] = row;
  }

  HS_PHASE_MARK(8);
  // ---- stores: rows, the hit slots' stamps, the victims' token and stamp
#pragma unroll
  for (int s = 0; s < ES; ++s) {
    const int i = sbase + 64 * s;
    if (i < N) rows[i] = rowA[s];
  }
#pragma unroll
  for (int j = 0; j < EC; ++j) {
    const int q = j * kThreads + tid;
    if (q < C && sflag[q] == 1) sstp[q] = p.stamp;
  }
  // (a victim's new token is recorded by the row mover, on the entry that
  // fills the slot)
  for (int j = tid; j < A; j += kThreads) sstp[vict[j]] = p.stamp;
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
  HS_PHASE_FLUSH;
}

template <int ES, int EC, bool FILL>
hipError_t launch_ec(KernelArgs a, int grid, hipStream_t stream) {
  auto fn = resolve_kernel<ES, EC, FILL>;
  static std::atomic<uint64_t> raised{0};
  hipError_t err = allow_full_lds(reinterpret_cast<const void*>(fn), raised);
  if (err != hipSuccess) return err;
  if constexpr (FILL) {
    // as many gather workgroups as fit beside the resolver's and the miss
    // workgroups in one round of the chip, so that no gather range waits
    // for a CU to come free
    int64_t resident = 0;
    err = resident_groups(reinterpret_cast<const void*>(fn), kThreads, a.lds_bytes, &resident);
    if (err != hipSuccess) return err;
    const int64_t target = resident - a.n_rl - a.fill.miss_groups;
    if (!a.fill.misses_only && target >= kFetchGatherMinGroups) {
      size_t flds = 0;
      const int64_t fill_groups = prepare_fetch(a.fill, &flds, target);
      const int64_t g = a.n_rl + fill_groups;
      if (g > INT32_MAX || flds > kMaxLdsBytes) return hipErrorInvalidValue;
      grid = (int)g;
      a.lds_bytes = a.plan.total > flds ? a.plan.total : (uint32_t)flds;
    }
    // interleave where the resolvers alone would hold more than half a
    // round of the chip.  Every resolver then has its place: the last one
    // sits at position 16 * ((n_rl - 1) / 8) + (n_rl - 1) % 8, behind
    // ((n_rl - 1) / 8) * 8 < n_rl gathers, and there is at least one gather
    // a request-layer.
    a.interleave = !a.fill.misses_only && a.fill.gather_splits > 0 &&
                   2 * (int64_t)a.n_rl > resident ? 1 : 0;
  }
  return launch_kernel(fn, dim3(grid), dim3(kThreads), a.lds_bytes, stream, a);
}

// Largest rounds per thread needed: HS_MAX_ENTRIES (8192) entries and
// HS_MAX_HOT_CAPACITY (12288) slots, i.e. 8 and 12 rounds of kThreads.
constexpr int kMaxRounds = HS_MAX_ENTRIES / kThreads;
constexpr int kMaxSlotRounds = HS_MAX_HOT_CAPACITY / kThreads;
static_assert(kMaxRounds == 8 && kMaxSlotRounds == 12, "round instantiations below");
static_assert(HS_MAX_HOT_CAPACITY <= (1 << kMissSlotBits), "slot field of the miss code");

template <int ES, bool FILL>
hipError_t launch_es(const KernelArgs& a, int grid, int EC, hipStream_t stream) {
  if constexpr (ES > kMaxRounds) {
    return hipErrorInvalidValue;
  } else {
    switch (EC) {
      case 1: return launch_ec<ES, 1, FILL>(a, grid, stream);
      case 2: return launch_ec<ES, 2, FILL>(a, grid, stream);
      case 4: return launch_ec<ES, 4, FILL>(a, grid, stream);
      case 8: return launch_ec<ES, 8, FILL>(a, grid, stream);
      case 12: return launch_ec<ES, 12, FILL>(a, grid, stream);
      default: return hipErrorInvalidValue;
    }
  }
}

template <bool FILL>
hipError_t launch_rounds(const KernelArgs& a, int grid, int ES, int EC, hipStream_t stream) {
  switch (ES) {
    case 1: return launch_es<1, FILL>(a, grid, EC, stream);
    case 2: return launch_es<2, FILL>(a, grid, EC, stream);
    case 4: return launch_es<4, FILL>(a, grid, EC, stream);
    case 8: return launch_es<8, FILL>(a, grid, EC, stream);
    default: return launch_es<16, FILL>(a, grid, EC, stream);
  }
}

// Rounds of kThreads elements per thread covering n (a power of two).
int round_up_pow2_rounds(int n) {
  const int e = (n + kThreads - 1) / kThreads;
  return e <= 1 ? 1 : e <= 2 ? 2 : e <= 4 ? 4 : e <= 8 ? 8 : 16;
}

// Rounds of kThreads slots per thread covering C: 1, 2, 4, 8 or 12.
int slot_rounds(int n) {
  const int e = (n + kThreads - 1) / kThreads;
  return e <= 8 ? round_up_pow2_rounds(n) : e <= 12 ? 12 : 16;
}

}  // namespace

size_t resolve_lds_bytes(int32_t entries, int32_t hot_capacity) {
  return make_plan(entries, hot_capacity, round_up_pow2_rounds(entries)).total;
}

hipError_t launch_resolve(const ResolveParams& p, const FetchParams* fill, hipStream_t stream) {
  const int ES = round_up_pow2_rounds(p.entries);
  const int EC = slot_rounds(p.hot_capacity);
  KernelArgs a;
  a.p = p;
  a.plan = make_plan(p.entries, p.hot_capacity, ES);
  a.n_rl = p.num_reqs * p.num_layers;
  a.lds_bytes = a.plan.total;
  a.interleave = 0;
  if (a.n_rl == 0) return hipSuccess;
  if (!fill) return launch_rounds<false>(a, a.n_rl, ES, EC, stream);
  a.fill = *fill;
  size_t flds = 0;
  const int64_t fill_groups = prepare_fetch(a.fill, &flds, 0);
  const int64_t grid = a.n_rl + fill_groups;
  if (grid > INT32_MAX || flds > kMaxLdsBytes) return hipErrorInvalidValue;
  if (flds > a.lds_bytes) a.lds_bytes = (uint32_t)flds;
  return launch_rounds<true>(a, (int)grid, ES, EC, stream);
}

}  // namespace hs
