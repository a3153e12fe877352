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
// flight per lane before any store, on grids that cover all 256 CUs many
// times over.  In the mover each wave owns kMoveEntriesPerWave whole entries:
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

// PIECES = row_bytes / 16 when known at compile time (0 = runtime).
template <int PIECES, bool FUSED>
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
  const int32_t layer = rl - r * p.num_layers;
  const int32_t pieces = PIECES > 0 ? PIECES : (p.row_bytes >> 4);
  const int32_t npieces = ne * pieces;
  const int ps = p.page_shift;
  const int32_t pm = (1 << ps) - 1;
  int32_t* rows = p.row_ids + (int64_t)rl * N + e0;
  const uint8_t* pool_l = p.pool + (int64_t)layer * p.pool_stride;
  uint8_t* out = p.out ? p.out + ((int64_t)rl * N + e0) * p.row_bytes : nullptr;

  const int32_t* topk = nullptr;
  const int32_t* hbt = nullptr;
  const int32_t* hot = nullptr;
  const uint8_t* host_l = nullptr;
  uint8_t* slot_l = nullptr;
  int64_t host_blocks = 0;
  if (FUSED) {
    topk = p.topk + (int64_t)rl * N + e0;
    hbt = p.host_block_table + (int64_t)r * p.max_pages;
    hot = p.hot_blocks + (int64_t)r * (p.hot_capacity >> ps);
    host_l = p.host + (int64_t)layer * p.host_stride;
    slot_l = p.pool_w + (int64_t)layer * p.pool_stride;
    host_blocks = p.host_rows >> ps;
  }

  for (int32_t base = 0; base < npieces; base += 64 * kU) {
    u32x4 v[kU];
    uint8_t* slot_dst[kU];
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const int32_t g = base + u * 64 + lane;
      v[u] = u32x4{0u, 0u, 0u, 0u};
      slot_dst[u] = nullptr;
      if (g < npieces) {
        const int32_t el = g / pieces;
        const int32_t pc = g - el * pieces;
        const int32_t code = rows[el];
        if (code >= 0) {
          if (out && code < p.pool_rows)
            v[u] = *reinterpret_cast<const u32x4*>(pool_l + (int64_t)code * p.row_bytes +
                                                   pc * 16);
        } else if (FUSED && code <= -8) {
          const int32_t q = (-code - 8) >> 1;
          const bool copier = ((-code - 8) & 1) != 0;
          if (out || copier) {
            const int32_t t = topk[el];
            if (t >= 0 && (t >> ps) < p.max_pages && q < p.hot_capacity) {
              const int32_t hb = hbt[t >> ps];
              if (hb >= 0 && hb < host_blocks) {
                const int64_t srow = ((int64_t)hb << ps) | (t & pm);
                v[u] = *reinterpret_cast<const u32x4*>(host_l + srow * p.row_bytes + pc * 16);
                const int32_t hblk = hot[q >> ps];
                if (copier && hblk >= 0 && hblk < (p.pool_rows >> ps)) {
                  const int64_t drow = ((int64_t)hblk << ps) | (q & pm);
                  slot_dst[u] = slot_l + drow * p.row_bytes + pc * 16;
                }
              }
            }
          }
        }
      }
    }
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const int32_t g = base + u * 64 + lane;
      if (g < npieces) {
        if (out)
          __builtin_nontemporal_store(v[u], reinterpret_cast<u32x4*>(out + (int64_t)g * 16));
        if (FUSED && slot_dst[u]) *reinterpret_cast<u32x4*>(slot_dst[u]) = v[u];
      }
    }
  }
  if (FUSED && lane < ne) {
    // only this wave reads these entries' codes, and all its reads are done
    const int32_t code = rows[lane];
    if (code <= -8) {
      const int32_t q = (-code - 8) >> 1;
      rows[lane] = q < p.hot_capacity ? (int32_t)(((int64_t)hot[q >> ps] << ps) | (q & pm))
                                      : -3;
    }
  }
}

// One workgroup copies one page of one layer: blockIdx.x = pair, blockIdx.y = layer.
__global__ void __launch_bounds__(kT) offload_kernel(OffloadParams p) {
  const int32_t i = blockIdx.x;
  const int32_t layer = blockIdx.y;
  const int64_t db = p.pairs[2 * i];
  const int64_t hb = p.pairs[2 * i + 1];
  if (db < 0 || db >= p.pool_blocks || hb < 0 || hb >= p.host_blocks) return;
  const uint8_t* src = p.pool + (int64_t)layer * p.pool_stride + db * p.page_bytes;
  uint8_t* dst = p.host + (int64_t)layer * p.host_stride + hb * p.page_bytes;
  const int32_t n = (int32_t)(p.page_bytes >> 4);
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

template <int PIECES>
void launch_move_pieces(const MoveParams& p, bool fused, int32_t chunks_per_rl, int32_t total,
                        uint32_t grid, hipStream_t stream) {
  if (fused)
    hipLaunchKernelGGL((move_kernel<PIECES, true>), dim3(grid), dim3(kT), 0, stream, p,
                       chunks_per_rl, total);
  else
    hipLaunchKernelGGL((move_kernel<PIECES, false>), dim3(grid), dim3(kT), 0, stream, p,
                       chunks_per_rl, total);
}

}  // namespace

hipError_t launch_move(const MoveParams& p, bool fused, hipStream_t stream) {
  const int64_t n_rl = (int64_t)p.num_reqs * p.num_layers;
  if (n_rl == 0 || p.rows_per_rl == 0) return hipSuccess;
  const int32_t chunks_per_rl = (p.rows_per_rl + kEPW - 1) / kEPW;
  const int64_t total = n_rl * chunks_per_rl;
  const uint32_t grid = (uint32_t)((total + kWavesPerBlock - 1) / kWavesPerBlock);
  if (p.row_bytes == 656)
    launch_move_pieces<41>(p, fused, chunks_per_rl, (int32_t)total, grid, stream);
  else
    launch_move_pieces<0>(p, fused, chunks_per_rl, (int32_t)total, grid, stream);
  return hipGetLastError();
}

hipError_t launch_offload(const OffloadParams& p, hipStream_t stream) {
  if (p.n == 0 || p.num_layers == 0) return hipSuccess;
  hipLaunchKernelGGL(offload_kernel, dim3((uint32_t)p.n, (uint32_t)p.num_layers), dim3(kT), 0,
                     stream, p);
  return hipGetLastError();
}

}  // namespace hs
