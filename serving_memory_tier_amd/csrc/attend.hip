// Sparse MLA decode over resolved rows read in place ("vLLM GLM 5.3 ...
// Hybrid HiSparse offloading, Part 1": hot pages sit in the same KV-cache
// tensor as resident pages, so the sparse MLA kernel reads every selected
// row by its HMA row id, "Use sparsity when needed" and "How it works").
// The rows are never copied to a gathered buffer first.
//
// Row format (656 bytes): 512 latent values in OCP FP8 E4M3, 4 float32
// scales (one per 128 latent values), 64 rope values in bfloat16.  A row's
// key is its scaled latent values and its rope values (576), its value the
// scaled latent values (512).
//
// Work split: one workgroup of 8 waves per (query token, 64 heads, key
// split); the two head groups of a (token, split) run side by side on one
// XCD, so each selected row comes from HBM about once.  Blocks of 32
// selected rows stream through LDS as they are in the pool (FP8 latent
// bytes, scales, bf16 rope), three blocks resident: the block computed, the
// next one being stored from registers, and the one before, which every wave
// is done with; the block after next is loaded by row id into registers.
// One barrier a block.  Wave w takes 16 heads (w & 3) and one half (w >> 2),
// which picks its 16 keys for the scores and its 256 value dimensions:
//   S^T (16 keys x 16 heads) = K Q^T with 16x16x32 bf16 MFMAs, the key
//     operand read from LDS as FP8, 16 bytes a lane for two steps (within
//     each 64-value chunk the contraction runs over lane g's 16 values, 8 a
//     step, and the queries are loaded in that order), and converted exactly
//     to bf16 (every E4M3 value is a bf16 value), one accumulator per
//     128-value latent tile and one for the rope, so the per-row scales are
//     applied in float32 after the products; the two halves swap their
//     scores through LDS (rows of 20 floats for 16 heads: the four lane
//     groups of a write or read land on distinct banks);
//   online softmax per head over the 32 keys (each lane owns one head column);
//   O^T (256 dims x 16 heads) += V^T P'^T, where P' = p * scale of the latent
//     tile: the probabilities are the B operand straight from registers, and
//     the value operand comes from the row-major block through the
//     transposing LDS read (ds_read_b64_tr_b8), converted to bf16 likewise.
// Reading FP8 from LDS and converting per use halves the LDS bytes against
// converting once into bf16 copies; half the value dimensions per wave keep
// a wave under 256 registers, so two waves share each SIMD.
// Key splits write their outputs divided by their own sums, in half
// precision, with their running max and sum to the workspace; a combine
// kernel merges them in float32.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <atomic>
#include <mutex>

#include "hs_internal.h"

// Timing hooks (per-workgroup time per phase of the block loop), empty unless
// a profiling build defines them.
#ifndef HS_ATTEND_MARK
#define HS_ATTEND_DECL
#define HS_ATTEND_MARK(i)
#define HS_ATTEND_FLUSH
#endif

namespace hs {
namespace {

constexpr int kT = kAttendThreads;          // 8 waves
constexpr int kBlockKeys = 32;
constexpr int kLatent = 512;
constexpr int kRope = 64;
constexpr int kDim = kLatent + kRope;       // 576
constexpr int kRowBytes = 656;
constexpr int kPieces = kRowBytes / 16;     // 41
constexpr int kBufs = 3;                    // blocks resident in LDS: computed, stored, free
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kStaleMax = 8.f;            // log2 of the largest unnormalised probability

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(4))) _Float16 f16x4;
typedef __attribute__((ext_vector_type(4))) uint32_t u32x4;
typedef __attribute__((ext_vector_type(2))) uint32_t u32x2;

// A block's rows as they are in the pool, 656 bytes each; key k of the
// block sits in row slot(k), which spreads both the key-fragment reads and the
// transposing value reads over distinct banks.
struct AttendBlock {
  uint8_t rows[kBlockKeys * kRowBytes];
};

__device__ __forceinline__ int slot(int k) { return k ^ ((k >> 4) << 3); }

struct AttendLds {
  AttendBlock blk[kBufs];
  int32_t ids[kAttendMaxSplitKeys];         // the split's row ids, -1 where nothing is selected
  float xs[2][4][kBlockKeys][20];           // scores per (head tile, key, head) for the exchange
};

typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;

// Two FP8 E4M3 bytes (the low or high half of w) to two bf16 in one word:
// exact, every E4M3 value is a bf16 value (the conversion's scale is 1).
template <bool HI>
__device__ __forceinline__ uint32_t fp8x2_to_bf16x2(uint32_t w) {
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, HI));
}

// ds_read_b64_tr_b8: within each group of 16 lanes, lane c receives byte
// c % 8 of the 8-byte vectors at the addresses of lanes 2 j + c / 8 of its
// group, j = 0..7 (an 8-byte-aligned LDS address a lane).
typedef __attribute__((ext_vector_type(2))) int i32x2;
typedef __attribute__((address_space(3))) i32x2 lds_i32x2;
__device__ __forceinline__ u32x2 tr8_read(const uint8_t* p) {
  const i32x2 v = __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_i32x2*)(const_cast<uint8_t*>(p)));
  return __builtin_bit_cast(u32x2, v);
}

// Eight FP8 E4M3 bytes to eight bf16, exactly, in byte order.
__device__ __forceinline__ bf16x8 fp8x8_to_bf16x8(u32x2 w) {
  return __builtin_bit_cast(bf16x8, u32x4{fp8x2_to_bf16x2<false>(w[0]), fp8x2_to_bf16x2<true>(w[0]),
                                          fp8x2_to_bf16x2<false>(w[1]), fp8x2_to_bf16x2<true>(w[1])});
}

// A block's rows are moved one 16-byte piece a thread (41 consecutive
// threads read one row): the loads are issued two blocks ahead of the
// block computed, into registers, and stored one block ahead.
constexpr int kBlockPieces = kBlockKeys * kPieces;                // 1312
constexpr int kFetchRounds = (kBlockPieces + kT - 1) / kT;        // 3

struct BlockRegs {
  u32x4 v[kFetchRounds];
  int32_t id[kFetchRounds];
};

// Global loads of the rows of keys [k0, k0 + 32) of the split (row ids from
// LDS) into registers.  Loads are unconditional where the pool has rows (an
// unselected key reads row 0 and is stored as zeros), so nothing waits
// between issuing them.
__device__ __forceinline__ void fetch_block(const AttendParams& p, const AttendLds& s,
                                            int32_t k0, BlockRegs& b) {
  const int tid = threadIdx.x;
  // every round's row id first (a key inside the block for each lane, so the
  // reads need no branch and are issued together), then the row loads
  int32_t ids[kFetchRounds];
#pragma unroll
  for (int i = 0; i < kFetchRounds; ++i) {
    const int q = tid + kT * i;
    ids[i] = s.ids[k0 + (q < kBlockPieces ? q / kPieces : 0)];
  }
#pragma unroll
  for (int i = 0; i < kFetchRounds; ++i) {
    const int q = tid + kT * i;
    const int k = q / kPieces, pc = q - k * kPieces;
    const int32_t id = q < kBlockPieces ? ids[i] : -1;
    b.id[i] = id;
    if (p.pool_rows > 0 && q < kBlockPieces)
      b.v[i] = *reinterpret_cast<const u32x4*>(p.kv + (int64_t)(id >= 0 ? id : 0) * kRowBytes +
                                               pc * 16);
    else
      b.v[i] = u32x4{0u, 0u, 0u, 0u};
  }
}

// The fetched rows into an LDS block as they are (zeros for unselected keys).
__device__ __forceinline__ void store_block(AttendBlock& s, const BlockRegs& b) {
  const int tid = threadIdx.x;
#pragma unroll
  for (int i = 0; i < kFetchRounds; ++i) {
    const int q = tid + kT * i;
    if (q >= kBlockPieces) continue;
    const int k = q / kPieces, pc = q - k * kPieces;
    *reinterpret_cast<u32x4*>(s.rows + slot(k) * kRowBytes + pc * 16) =
        b.id[i] >= 0 ? b.v[i] : u32x4{0u, 0u, 0u, 0u};
  }
}


// 8 waves: wave w takes head tile ht = w & 3 (16 heads) and half = w >> 2,
// which picks both its key tile for the scores (keys 16 half ..) and its
// value dimensions (256 half ..); the two halves swap scores through LDS.
__global__ void __launch_bounds__(kT) attend_kernel(AttendParams p) {
  extern __shared__ __attribute__((aligned(16))) unsigned char lds_raw[];
  AttendLds& s = *reinterpret_cast<AttendLds*>(lds_raw);
  // workgroup -> (token, split, head group): the head groups of one (token,
  // split) are 8 workgroups apart -- the XCD stride -- and dispatched
  // together, so the rows one of them fetches are in that XCD's L2 when the
  // other reads them
  const int32_t L = blockIdx.x;
  const int hg = (L >> 3) % p.head_groups;
  const int32_t pair = (L / (8 * p.head_groups)) * 8 + (L & 7);
  if (pair >= p.num_tokens * p.splits) return;   // the grid's rounding: the whole workgroup
  const int t = pair % p.num_tokens, split = pair / p.num_tokens;
  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63;
  const int col = l & 15, g = l >> 4;
  const int ht = w & 3, half = w >> 2;
  const int head = hg * 64 + ht * 16 + col;
  const bool head_ok = head < p.num_heads;
  const int32_t key_lo = split * p.keys_per_split;
  const int32_t key_end = min(p.top_k, key_lo + p.keys_per_split);
  const int32_t* ids = p.row_ids + (int64_t)t * p.top_k;

  bf16x8 qb[kDim / 32];
  {
    const uint16_t* qh = p.q + ((int64_t)t * p.num_heads + (head_ok ? head : 0)) * kDim;
#pragma unroll
    for (int ks = 0; ks < kDim / 32; ++ks) {
      // latent steps in the keys' read order: step kk of tile tl takes
      // values 128 tl + 64 (kk / 2) + 16 g + 8 (kk % 2) ..; rope as it is
      const int off = ks < 16 ? (ks / 4) * 128 + 64 * ((ks % 4) >> 1) + 16 * g + 8 * (ks & 1)
                              : ks * 32 + 8 * g;
      u32x4 v = head_ok ? *reinterpret_cast<const u32x4*>(qh + off) : u32x4{0, 0, 0, 0};
      qb[ks] = __builtin_bit_cast(bf16x8, v);
    }
  }
  f32x4 o[16];                               // O^T: dims 256 half + 16 dt + 4 g + r
#pragma unroll
  for (int dt = 0; dt < 16; ++dt) o[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY, l_run = 0.f;
  const float qk_scale = p.sm_scale * kLog2e;

  const int32_t n_keys = key_end > key_lo ? key_end - key_lo : 0;
  const int32_t n_pad = (n_keys + kBlockKeys - 1) / kBlockKeys * kBlockKeys;
  for (int k = tid; k < n_pad; k += kT) {
    int32_t id = k < n_keys ? ids[key_lo + k] : -1;
    if (id >= 0 && (int64_t)id >= p.pool_rows) id = -1;
    s.ids[k] = id;
  }
  __syncthreads();
  HS_ATTEND_DECL;
  const int32_t nblk = n_pad / kBlockKeys;
  BlockRegs regs;
  if (nblk > 0) {
    fetch_block(p, s, 0, regs);
    store_block(s.blk[0], regs);
    if (nblk > 1) fetch_block(p, s, kBlockKeys, regs);
  }
  __syncthreads();
  // Block i is computed from buffer i % 3 while block i + 1 is stored into
  // buffer (i + 1) % 3 and block i + 2 is loaded into registers.  One barrier
  // a block: past it, block i's scores and block i + 1's rows are complete,
  // and every wave is done with block i - 1, whose buffer is stored next.
  int cur = 0;
  for (int32_t bi = 0; bi < nblk; ++bi) {
    HS_ATTEND_MARK(0);
    const AttendBlock& cb = s.blk[cur];
    const int nxt = cur == kBufs - 1 ? 0 : cur + 1;
    float (*xs)[kBlockKeys][20] = s.xs[bi & 1];
    // ---- scores of this wave's key tile: S^T[key 16 half + ..][head]
    {
      f32x4 acc[5];
#pragma unroll
      for (int tl = 0; tl < 5; ++tl) acc[tl] = f32x4{0.f, 0.f, 0.f, 0.f};
      // key half * 16 + col: latent bytes 128 tl + 32 kk + 8 g .. converted
      // to bf16, rope values 32 kk + 8 g .. as they are
      const uint8_t* krow = cb.rows + slot(half * 16 + col) * kRowBytes;
      // latent: one 16-byte read a tile covers two steps (the contraction's
      // order within a 64-value chunk is lane g's 16 values, 8 a step; the
      // queries were loaded in the same order)
#pragma unroll
      for (int kk2 = 0; kk2 < 2; ++kk2) {
        u32x4 kr[4];
#pragma unroll
        for (int tl = 0; tl < 4; ++tl)
          kr[tl] = *reinterpret_cast<const u32x4*>(krow + tl * 128 + kk2 * 64 + 16 * g);
        bf16x8 rp[2];
        if (kk2 == 0) {
#pragma unroll
          for (int h = 0; h < 2; ++h)
            rp[h] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(
                        krow + kLatent + 16 + h * 64 + 16 * g));
        }
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const int kk = 2 * kk2 + h;
#pragma unroll
          for (int tl = 0; tl < 4; ++tl)
            acc[tl] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                fp8x8_to_bf16x8(u32x2{kr[tl][2 * h], kr[tl][2 * h + 1]}), qb[tl * 4 + kk], acc[tl],
                0, 0, 0);
          if (kk2 == 0)
            acc[4] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(rp[h], qb[16 + h], acc[4], 0, 0, 0);
        }
      }
      // the four keys' scales and row ids read together, before any score
      // is written (the writes would otherwise order each read after them)
      f32x4 sc4[4];
      int32_t sel[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int key = half * 16 + 4 * g + r;
        sc4[r] = *reinterpret_cast<const f32x4*>(cb.rows + slot(key) * kRowBytes + kLatent);
        sel[r] = s.ids[bi * kBlockKeys + key];
      }
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int key = half * 16 + 4 * g + r;
        float v = acc[4][r];
#pragma unroll
        for (int tl = 0; tl < 4; ++tl) v += sc4[r][tl] * acc[tl][r];
        xs[ht][key][col] = sel[r] >= 0 ? v * qk_scale : -INFINITY;
      }
    }
    HS_ATTEND_MARK(1);
    // ---- the next block into the next buffer, the one after into registers
    if (bi + 1 < nblk) {
      store_block(s.blk[nxt], regs);
      if (bi + 2 < nblk) fetch_block(p, s, (bi + 2) * kBlockKeys, regs);
    }
    HS_ATTEND_MARK(2);
    __syncthreads();
    HS_ATTEND_MARK(3);
    // ---- online softmax over the block's 32 keys (both halves alike)
    float sc[2][4];
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
      for (int r = 0; r < 4; ++r) sc[mt][r] = xs[ht][mt * 16 + 4 * g + r][col];
    float mb = -INFINITY;
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
      for (int r = 0; r < 4; ++r) mb = fmaxf(mb, sc[mt][r]);
    mb = fmaxf(mb, __shfl_xor(mb, 16));
    mb = fmaxf(mb, __shfl_xor(mb, 32));
    const bool grow = mb > m_run + kStaleMax;
    const float m_new = grow ? mb : m_run;
    // the hardware base-2 exponential: arguments here are <= kStaleMax, and
    // results below 2^-126 (weights far below the block's largest) go to 0
    const float alpha = grow ? __builtin_amdgcn_exp2f(m_run - m_new) : 1.f;
    float pr[2][4], ls = 0.f;
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        pr[mt][r] = m_new == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(sc[mt][r] - m_new);
        ls += pr[mt][r];
      }
    ls += __shfl_xor(ls, 16);
    ls += __shfl_xor(ls, 32);
    l_run = l_run * alpha + ls;
    m_run = m_new;
    if (__any(grow)) {
#pragma unroll
      for (int dt = 0; dt < 16; ++dt) o[dt] *= alpha;
    }
    // ---- O^T += V^T P'^T for this wave's two latent tiles.  The value
    // operand is read transposed from the key-major rows: in each 16-lane
    // group g, lane c supplies the address of key 4 g + c / 4 (and 16 more),
    // dimensions 4 (c % 4) ..; the transposing read hands lane c dimension c
    // of keys 4 g .. 4 g + 3
#pragma unroll
    for (int t2 = 0; t2 < 2; ++t2) {
      const int tl = half * 2 + t2;
      bf16x8 b;
#pragma unroll
      for (int mt = 0; mt < 2; ++mt)
#pragma unroll
        for (int r = 0; r < 4; ++r)
          b[4 * mt + r] = (__bf16)(pr[mt][r] * *reinterpret_cast<const float*>(
                                        cb.rows + slot(mt * 16 + 4 * g + r) * kRowBytes +
                                        kLatent + 4 * tl));
      bf16x8 va[8];
      // lane c of group g supplies key kv(c / 2) (4 g + j, then 16 + 4 g + j)
      // at dimensions 8 (c % 2) ..; the transposing read hands lane c
      // dimension c of the group's eight keys
      const int j = col >> 1;
      const int kv = (j < 4 ? 0 : 12) + 4 * g + j;
      const uint8_t* vbase = cb.rows + slot(kv) * kRowBytes + 8 * (col & 1);
#pragma unroll
      for (int d8 = 0; d8 < 8; ++d8)
        va[d8] = fp8x8_to_bf16x8(tr8_read(vbase + (tl * 8 + d8) * 16));
#pragma unroll
      for (int d8 = 0; d8 < 8; ++d8)
        o[t2 * 8 + d8] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va[d8], b, o[t2 * 8 + d8], 0, 0, 0);
    }
    HS_ATTEND_MARK(4);
    cur = nxt;
  }
  HS_ATTEND_MARK(5);
  HS_ATTEND_FLUSH;

  if (!head_ok) return;
  const int64_t th = (int64_t)t * p.num_heads + head;
  const int d0 = half * 256;
  if (p.splits == 1) {
    const float inv = l_run > 0.f ? 1.f / l_run : 0.f;
    float* out = p.out + th * kLatent + d0;
#pragma unroll
    for (int dt = 0; dt < 16; ++dt)
      *reinterpret_cast<f32x4*>(out + dt * 16 + 4 * g) = o[dt] * inv;
    if (g == 0 && half == 0)
      p.lse[th] = l_run > 0.f ? (m_run + log2f(l_run)) / kLog2e : -INFINITY;
    return;
  }
  // the split's output divided by its own sum, in half precision: values
  // within the rows' range, a relative 2^-11 each, half the bytes of float32
  // for the merge to read back
  const int64_t ps = ((int64_t)t * p.splits + split) * p.num_heads + head;
  const float inv = l_run > 0.f ? 1.f / l_run : 0.f;
  uint16_t* po = p.part_o + ps * kLatent + d0;
#pragma unroll
  for (int dt = 0; dt < 16; ++dt) {
    const f32x4 v = o[dt] * inv;
    const f16x4 h = {(_Float16)v[0], (_Float16)v[1], (_Float16)v[2], (_Float16)v[3]};
    *reinterpret_cast<f16x4*>(po + dt * 16 + 4 * g) = h;
  }
  if (g == 0 && half == 0) {
    p.part_ml[2 * ps] = m_run;
    p.part_ml[2 * ps + 1] = l_run;
  }
}

// Merges the key splits of one (token, head): with w_s = 2^(m_s - M) l_s and
// the splits' normalised outputs O_s / l_s, out = sum_s w_s (O_s / l_s) /
// sum_s w_s, lse = (M + log2 L) / log2 e, L = sum_s w_s.
__global__ void __launch_bounds__(128) attend_combine_kernel(AttendParams p) {
  const int t = blockIdx.y, head = blockIdx.x;
  const int64_t th = (int64_t)t * p.num_heads + head;
  float M = -INFINITY;
  for (int sp = 0; sp < p.splits; ++sp)
    M = fmaxf(M, p.part_ml[2 * (((int64_t)t * p.splits + sp) * p.num_heads + head)]);
  float L = 0.f;
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  for (int sp = 0; sp < p.splits; ++sp) {
    const int64_t ps = ((int64_t)t * p.splits + sp) * p.num_heads + head;
    const float m = p.part_ml[2 * ps];
    if (m == -INFINITY) continue;
    const float wgt = exp2f(m - M) * p.part_ml[2 * ps + 1];
    L += wgt;
    const f16x4 h = *reinterpret_cast<const f16x4*>(p.part_o + ps * kLatent + 4 * threadIdx.x);
    acc += wgt * f32x4{(float)h[0], (float)h[1], (float)h[2], (float)h[3]};
  }
  const float inv = L > 0.f ? 1.f / L : 0.f;
  *reinterpret_cast<f32x4*>(p.out + th * kLatent + 4 * threadIdx.x) = acc * inv;
  if (threadIdx.x == 0) p.lse[th] = L > 0.f ? (M + log2f(L)) / kLog2e : -INFINITY;
}

// The workspace of the allocation-free entry point: one array per device
// that holds the key splits' partial outputs of whichever call runs, kept
// until the process ends.  Host code never uses the array's name as an
// address (on the host it only names the symbol); the device address comes
// from hipGetSymbolAddress, once per device, on that device.
static __device__ __align__(256) unsigned char scratch[kAttendScratchBytes];

}  // namespace

hipError_t attend_scratch(void** ptr) {
  static std::mutex mu;
  static void* addr[64] = {};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= 64) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (!addr[dev]) {
    void* a = nullptr;
    e = hipGetSymbolAddress(&a, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!a) return hipErrorInvalidSymbol;
    addr[dev] = a;
  }
  *ptr = addr[dev];
  return hipSuccess;
}

size_t attend_lds_bytes() { return sizeof(AttendLds); }

void plan_attend(AttendParams& p, int64_t target_groups) {
  const int32_t hg = (p.num_heads + kAttendHeadsPerGroup - 1) / kAttendHeadsPerGroup;
  const int64_t base = (int64_t)p.num_tokens * hg;
  const int32_t blocks = (p.top_k + kBlockKeys - 1) / kBlockKeys;
  int64_t s = base > 0 ? (target_groups + base - 1) / base : 1;
  const int64_t s_min = (blocks + kAttendMaxSplitKeys / kBlockKeys - 1) /
                        (kAttendMaxSplitKeys / kBlockKeys);   // the split's ids fit in LDS
  if (s < s_min) s = s_min;
  if (s > blocks) s = blocks;
  if (s > kAttendMaxSplits) s = kAttendMaxSplits;   // top_k is validated against this bound
  if (s < 1) s = 1;
  const int32_t per = (int32_t)(((blocks + s - 1) / s) * kBlockKeys);
  p.head_groups = hg;
  p.keys_per_split = per;
  p.splits = per > 0 ? (p.top_k + per - 1) / per : 1;
  if (p.splits < 1) p.splits = 1;
}

hipError_t launch_attend(const AttendParams& p, hipStream_t stream) {
  if (p.num_tokens == 0 || p.num_heads == 0) return hipSuccess;
  static_assert(kAttendHeadsPerGroup == 64, "64 heads per workgroup");
  auto fn = attend_kernel;
  static std::atomic<uint64_t> raised{0};
  hipError_t e = allow_full_lds(reinterpret_cast<const void*>(fn), raised);
  if (e != hipSuccess) return e;
  // (token, split) pairs in rounds of 8, each round once per head group
  const int64_t pairs = (int64_t)p.num_tokens * p.splits;
  const int64_t grid = (pairs + 7) / 8 * 8 * p.head_groups;
  if (grid > INT32_MAX) return hipErrorInvalidValue;
  e = launch_kernel(fn, dim3((uint32_t)grid), dim3(kT), sizeof(AttendLds), stream, p);
  if (e != hipSuccess || p.splits == 1) return e;
  return launch_kernel(attend_combine_kernel, dim3((uint32_t)p.num_heads, (uint32_t)p.num_tokens),
                       dim3(128), 0, stream, p);
}

}  // namespace hs
