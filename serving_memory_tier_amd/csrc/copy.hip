// Streaming kernels for gfx950: the row mover (single-stride gather, fused
// with the host-link copies of the resolver's misses) and the post-forward
// prefix-page offload.
//
// Method: "vLLM GLM 5.3 ... Hybrid HiSparse offloading, Part 1", section
// "How it works": the resolver hands back a row id whether the row is
// resident or hot, and the rows are gathered at one stride; a miss copies
// one row from pinned host memory into its hot slot; completed prefix pages
// are copied to host while still served from the GPU, all sparse layers in
// one launch after the forward, ordered on the model's stream.
//
// Both kernels are bound by memory bandwidth -- HBM for the gather, the host
// link for miss rows and offloaded pages -- not by arithmetic.  They move
// 16-byte pieces, consecutive lanes on consecutive pieces, several loads in
// flight per lane before any store; the mover's grid covers all 256 CUs many
// times over, the offload's is a few workgroups that loop, which is enough
// for the link.  In the mover each wave owns kMoveEntriesPerWave whole entries:
// host-link reads of the misses and HBM reads of the resident and hot rows
// are interleaved across every wave of the chip, so the two links run at the
// same time instead of one after the other.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "hs_internal.h"

namespace hs {
namespace {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

constexpr int kT = kCopyThreads;
constexpr int kU = kCopyUnroll;
constexpr int kWavesPerBlock = kT / 64;
constexpr int kEPW = kMoveEntriesPerWave;

// PIECES = row_bytes / 16 when known at compile time (0 = runtime); MODE is
// a MoveMode.
template <int PIECES, int MODE>
__global__ void __launch_bounds__(kT) move_kernel(MoveParams p, int32_t chunks_per_rl,
                                                  int32_t total_chunks) {
  const int lane = threadIdx.x & 63;
  const int32_t c = blockIdx.x * kWavesPerBlock + (threadIdx.x >> 6);
  if (c >= total_chunks) return;  // the whole wave leaves together
  const int32_t rl = c / chunks_per_rl;
  const int32_t e0 = (c - rl * chunks_per_rl) * kEPW;
  const int32_t N = p.rows_per_rl;
  const int32_t ne = min(kEPW, N - e0);
  const int32_t r = rl / p.num_layers;
  const int32_t group = MODE == kMoveFused ? p.group : 1;
  const int32_t l0 = (rl - r * p.num_layers) * group;  // first layer of the group
  const int32_t layers = p.layers > 0 ? p.layers : p.num_layers;
  const int32_t pieces = PIECES > 0 ? PIECES : (p.row_bytes >> 4);
  const int32_t npieces = ne * pieces;
  const int ps = p.page_shift;
  const int32_t pm = (1 << ps) - 1;
  int32_t* rows = p.row_ids + (int64_t)rl * N + e0;
  const int64_t out_stride = (int64_t)N * p.row_bytes;  // between layers of the output
  constexpr bool kSlots = MODE == kMoveFused;

  // Each entry is resolved once, by lane `entry` of the wave, before any row
  // moves: its code and token are loaded together, then its host block and
  // its slot's hot block together; the piece loop below takes an entry's
  // source and slot rows from that lane (ds_bpermute), so a piece's load
  // waits on nothing but its address.
  //   kind 0: zero row (or nothing without an output); 1: pool row; 2: host row
  const bool has_e = lane < ne;
  const int32_t code = has_e ? rows[lane] : 0;
  const int32_t t = kSlots && has_e ? p.topk[(int64_t)rl * N + e0 + lane] : -1;
  int32_t kind = 0, src = 0, drow = -1;  // drow: the slot's pool row, for a first entry
  int32_t hblk = -1;                     // the slot's hot block, for an assigned miss
  const int32_t q = code <= -8 ? (-code - 8) >> 1 : 0;
  const bool copier = code <= -8 && ((-code - 8) & 1) != 0;
  if (code >= 0) {
    if (p.out && code < p.pool_rows) { kind = 1; src = code; }
  } else if (kSlots && code <= -8 && q < p.hot_capacity) {
    const int32_t* hot = p.hot_blocks + (int64_t)r * (p.hot_capacity >> ps);
    hblk = hot[q >> ps];
    int32_t hb = -1;
    if (t >= 0 && (t >> ps) < p.max_pages) hb = p.host_block_table[(int64_t)r * p.max_pages + (t >> ps)];
    if ((p.out || copier) && hb >= 0 && hb < (p.host_rows >> ps)) {
      kind = 2;
      src = (hb << ps) | (t & pm);
      if (copier && hblk >= 0 && hblk < (p.pool_rows >> ps)) drow = (hblk << ps) | (q & pm);
    }
  }

  for (int32_t lj = 0; lj < group; ++lj) {  // each layer of the group
    const int32_t layer = l0 + lj;
    const uint8_t* pool_l = p.pool + (int64_t)layer * p.pool_stride;
    uint8_t* out = p.out ? p.out + ((int64_t)r * layers + layer) * out_stride +
                               (int64_t)e0 * p.row_bytes
                         : nullptr;
    uint8_t* slot_l = kSlots ? p.pool_w + (int64_t)layer * p.pool_stride : nullptr;
    const uint8_t* host_l = kSlots ? p.host + (int64_t)layer * p.host_stride : nullptr;
    for (int32_t base = 0; base < npieces; base += 64 * kU) {
      u32x4 v[kU];
      uint8_t* slot_dst[kU];
      bool st[kU];
#pragma unroll
      for (int u = 0; u < kU; ++u) {
        const int32_t g = base + u * 64 + lane;
        const bool in = g < npieces;
        const int32_t el = in ? g / pieces : 0;
        const int32_t pc = g - el * pieces;
        // every lane takes part in the exchange (lanes past the pieces read entry 0)
        const int32_t ek = __builtin_amdgcn_ds_bpermute(el << 2, kind);
        const int32_t es = __builtin_amdgcn_ds_bpermute(el << 2, src);
        const int32_t ed = kSlots ? __builtin_amdgcn_ds_bpermute(el << 2, drow) : -1;
        v[u] = u32x4{0u, 0u, 0u, 0u};
        slot_dst[u] = nullptr;
        st[u] = in && out != nullptr;
        if (in && ek == 1)
          v[u] = *reinterpret_cast<const u32x4*>(pool_l + (int64_t)es * p.row_bytes + pc * 16);
        if (kSlots && in && ek == 2) {
          v[u] = *reinterpret_cast<const u32x4*>(host_l + (int64_t)es * p.row_bytes + pc * 16);
          if (ed >= 0) slot_dst[u] = slot_l + (int64_t)ed * p.row_bytes + pc * 16;
        }
      }
#pragma unroll
      for (int u = 0; u < kU; ++u) {
        const int32_t g = base + u * 64 + lane;
        if (st[u])
          __builtin_nontemporal_store(v[u], reinterpret_cast<u32x4*>(out + (int64_t)g * 16));
        if (kSlots && slot_dst[u]) *reinterpret_cast<u32x4*>(slot_dst[u]) = v[u];
      }
    }
  }  // layers of the group
  if (kSlots && has_e && code <= -8) {
    // only this wave reads these entries' codes, and it read them all above
    if (q < p.hot_capacity) {
      if (copier) p.slot_token[(int64_t)rl * p.hot_capacity + q] = t;
      rows[lane] = (int32_t)(((int64_t)hblk << ps) | (q & pm));
    } else {
      rows[lane] = -3;
    }
  }
}


// Entries per wave of the commit: few enough that a chunk full of misses is
// copied by a wave in a few rounds of loads (64 entries of 656-byte rows would
// be ten rounds, and a step of misses only would run on a quarter as many
// waves).
constexpr int kCommitEPW = 16;
// The C ABI bounds a launch's waves by kMoveEntriesPerWave entries a wave.
static_assert(kCommitEPW >= kMoveEntriesPerWave, "commit waves within the validated bound");

// The commit after the early fill: one wave per kCommitEPW entries of a
// request-layer.  Entries holding a first-entry code copy their output row
// into the assigned slot and record the slot's token; every code becomes the
// slot's row id; misses left without a slot get a zero row.  Only those rows
// are touched, so the work is proportional to the misses.
template <int PIECES>
__global__ void __launch_bounds__(kT) commit_kernel(MoveParams p, int32_t chunks_per_rl,
                                                    int32_t total_chunks) {
  __shared__ int32_t work_e[kWavesPerBlock][kCommitEPW];    // entry; -1 - entry for a zero row
  __shared__ int32_t work_row[kWavesPerBlock][kCommitEPW];  // the slot's pool row
  const int lane = threadIdx.x & 63;
  const int wv = threadIdx.x >> 6;
  const int32_t c = blockIdx.x * kWavesPerBlock + wv;
  if (c >= total_chunks) return;  // the whole wave leaves together
  const int32_t rl = c / chunks_per_rl;
  const int32_t e0 = (c - rl * chunks_per_rl) * kCommitEPW;
  const int32_t N = p.rows_per_rl;
  const int32_t ne = min(kCommitEPW, N - e0);
  const int32_t r = rl / p.num_layers;
  const int32_t l0 = (rl - r * p.num_layers) * p.group;  // first layer of the group
  const int32_t layers = p.layers > 0 ? p.layers : p.num_layers;
  const int32_t pieces = PIECES > 0 ? PIECES : (p.row_bytes >> 4);
  const int ps = p.page_shift;
  const int32_t pm = (1 << ps) - 1;
  int32_t* rows = p.row_ids + (int64_t)rl * N + e0;
  const int64_t out_stride = (int64_t)N * p.row_bytes;  // between layers of the output
  uint8_t* out0 = p.out + ((int64_t)r * layers + l0) * out_stride + (int64_t)e0 * p.row_bytes;
  const int32_t* topk = p.topk + (int64_t)rl * N + e0;
  const int32_t* hot = p.hot_blocks + (int64_t)r * (p.hot_capacity >> ps);
  uint8_t* slot0 = p.pool_w + (int64_t)l0 * p.pool_stride;
  int32_t* stok = p.slot_token + (int64_t)rl * p.hot_capacity;

  // the codes, the entries' tokens and (up to 64 of them) the request's hot
  // blocks are loaded together, so a miss's slot row waits on one load
  const int32_t code = lane < ne ? rows[lane] : 0;
  const int32_t tk = lane < ne ? topk[lane] : -1;
  const int32_t nhb = p.hot_capacity >> ps;
  const bool hot_in_lanes = nhb <= 64;  // the same for the whole launch
  const int32_t hreg = hot_in_lanes && lane < nhb ? hot[lane] : -1;
  const int32_t qq = code <= -8 ? (-code - 8) >> 1 : 0;
  // every lane takes part in the exchange; lanes without a miss read lane 0
  const int32_t hlane = hot_in_lanes
      ? __builtin_amdgcn_ds_bpermute(((qq < p.hot_capacity ? qq >> ps : 0) & 63) << 2, hreg)
      : -1;
  int32_t drow = -1;  // the slot's pool row, for a first entry
  bool copier = false;
  if (code <= -8) {
    const int32_t q = qq;
    if (q < p.hot_capacity) {
      const int32_t hblk = hot_in_lanes ? hlane : hot[q >> ps];
      const int32_t row = (hblk << ps) | (q & pm);
      copier = ((-code - 8) & 1) != 0 && hblk >= 0 && hblk < (p.pool_rows >> ps);
      if (copier) {
        drow = row;
        stok[q] = tk;
      }
      rows[lane] = row;
    } else {
      rows[lane] = -3;
    }
  }
  const bool zero = code == -2;
  const uint64_t m = __ballot(copier || zero);
  if (m == 0) return;
  if (copier || zero) {
    const int32_t rank = __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32),
                                                   __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
    work_e[wv][rank] = zero ? -1 - lane : lane;
    work_row[wv][rank] = drow;
  }
  // the work lists are written and read by this wave only
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
  const int32_t n = __popcll(m);
  const int32_t total = n * pieces;
  const int64_t dst_stride = p.row_bytes;
  for (int32_t l = 0; l < p.group; ++l) {  // each layer of the group
    uint8_t* out = out0 + l * out_stride;
    uint8_t* slot_l = slot0 + l * p.pool_stride;
    for (int32_t g0 = 0; g0 < total; g0 += 64 * kU) {
      u32x4 v[kU];
      uint8_t* dst[kU];
#pragma unroll
      for (int u = 0; u < kU; ++u) {
        const int32_t g = g0 + u * 64 + lane;
        dst[u] = nullptr;
        v[u] = u32x4{0u, 0u, 0u, 0u};
        if (g < total) {
          const int32_t j = g / pieces;
          const int32_t pc = g - j * pieces;
          const int32_t w = work_e[wv][j];
          if (w < 0) {
            dst[u] = out + (int64_t)(-1 - w) * dst_stride + pc * 16;
          } else {
            v[u] = *reinterpret_cast<const u32x4*>(out + (int64_t)w * dst_stride + pc * 16);
            dst[u] = slot_l + (int64_t)work_row[wv][j] * dst_stride + pc * 16;
          }
        }
      }
#pragma unroll
      for (int u = 0; u < kU; ++u)
        if (dst[u]) *reinterpret_cast<u32x4*>(dst[u]) = v[u];
    }
  }
}

// Workgroup b copies the pages of (pair, layer) items b, b + G, b + 2G, ...
// (G workgroups, item = layer * n + pair); G is bounded, so that an offload
// running beside other kernels leaves them most of the chip -- the link, not
// the number of workgroups, sets its rate.
__global__ void __launch_bounds__(kT) offload_kernel(OffloadParams p) {
  const int64_t items = (int64_t)p.n * p.num_layers;
  const int32_t n = (int32_t)(p.page_bytes >> 4);
  for (int64_t it = blockIdx.x; it < items; it += gridDim.x) {
    const int32_t layer = (int32_t)(it / p.n);
    const int32_t i = (int32_t)(it - (int64_t)layer * p.n);
    const int64_t db = p.pairs[2 * i];
    const int64_t hb = p.pairs[2 * i + 1];
    if (db < 0 || db >= p.pool_blocks || hb < 0 || hb >= p.host_blocks) continue;
    const uint8_t* src = p.pool + (int64_t)layer * p.pool_stride + db * p.page_bytes;
    uint8_t* dst = p.host + (int64_t)layer * p.host_stride + hb * p.page_bytes;
    for (int32_t b = threadIdx.x; b < n; b += kT * kU) {
      u32x4 v[kU];
#pragma unroll
      for (int u = 0; u < kU; ++u) {
        const int32_t g = b + u * kT;
        if (g < n) v[u] = *reinterpret_cast<const u32x4*>(src + (int64_t)g * 16);
      }
#pragma unroll
      for (int u = 0; u < kU; ++u) {
        const int32_t g = b + u * kT;
        if (g < n) *reinterpret_cast<u32x4*>(dst + (int64_t)g * 16) = v[u];
      }
    }
  }
}

template <int PIECES>
hipError_t launch_move_pieces(const MoveParams& p, MoveMode mode, int32_t chunks_per_rl,
                              int32_t total, uint32_t grid, hipStream_t stream) {
  void (*fn)(MoveParams, int32_t, int32_t) = nullptr;
  switch (mode) {
    case kMoveGather: fn = move_kernel<PIECES, kMoveGather>; break;
    case kMoveFused: fn = move_kernel<PIECES, kMoveFused>; break;
    case kMoveCommit: break;  // commit_kernel
  }
  if (!fn) return hipErrorInvalidValue;
  return launch_kernel(fn, dim3(grid), dim3(kT), 0, stream, p, chunks_per_rl, total);
}

}  // namespace

hipError_t launch_move(const MoveParams& p, MoveMode mode, hipStream_t stream) {
  const int64_t n_rl = (int64_t)p.num_reqs * p.num_layers;
  if (n_rl == 0 || p.rows_per_rl == 0) return hipSuccess;
  if (mode == kMoveCommit) {
    const int32_t cpr = (p.rows_per_rl + kCommitEPW - 1) / kCommitEPW;
    const int64_t total = n_rl * cpr;
    const uint32_t grid = (uint32_t)((total + kWavesPerBlock - 1) / kWavesPerBlock);
    auto fn = p.row_bytes == 656 ? commit_kernel<41> : commit_kernel<0>;
    return launch_kernel(fn, dim3(grid), dim3(kT), 0, stream, p, cpr, (int32_t)total);
  }
  const int32_t chunks_per_rl = (p.rows_per_rl + kEPW - 1) / kEPW;
  const int64_t total = n_rl * chunks_per_rl;
  const uint32_t grid = (uint32_t)((total + kWavesPerBlock - 1) / kWavesPerBlock);
  if (p.row_bytes == 656)
    return launch_move_pieces<41>(p, mode, chunks_per_rl, (int32_t)total, grid, stream);
  return launch_move_pieces<0>(p, mode, chunks_per_rl, (int32_t)total, grid, stream);
}

hipError_t launch_offload(const OffloadParams& p, hipStream_t stream) {
  if (p.n == 0 || p.num_layers == 0) return hipSuccess;
  const int64_t items = (int64_t)p.n * p.num_layers;
  const int64_t grid = items < kOffloadGroups ? items : kOffloadGroups;
  return launch_kernel(offload_kernel, dim3((uint32_t)grid), dim3(kT), 0, stream, p);
}

}  // namespace hs
