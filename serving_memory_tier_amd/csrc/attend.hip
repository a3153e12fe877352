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
// Work split: one workgroup of 4 waves per (query token, 64 heads, key
// split).  Per block of 32 selected rows the workgroup loads the rows by id,
// converts the latent bytes exactly to bfloat16 (FP8 E4M3 fits bfloat16)
// into LDS twice -- key-major for the scores, dimension-major for the
// values -- and each wave takes 16 heads:
//   S^T (32 keys x 16 heads) = K Q^T with 16x16x32 bf16 MFMAs, one
//     accumulator per 128-value latent tile and one for the rope, so the
//     per-row scales are applied in float32 after the products;
//   online softmax per head (each lane owns one head column);
//   O^T (512 dims x 16 heads) += V^T P'^T, where P' = p * scale of the
//     latent tile: the probabilities are the B operand straight from the
//     score accumulators' registers, no LDS round trip.
// Key splits write unnormalised partial outputs with their running max and
// sum to the caller's workspace; a combine kernel merges them.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <atomic>

#include "hs_internal.h"

namespace hs {
namespace {

constexpr int kT = kAttendThreads;          // 4 waves
constexpr int kHeadsPerWave = 16;
constexpr int kBlockKeys = 32;
constexpr int kLatent = 512;
constexpr int kRope = 64;
constexpr int kDim = kLatent + kRope;       // 576
constexpr int kRowBytes = 656;
constexpr int kPieces = kRowBytes / 16;     // 41
constexpr int kKdStride = kDim + 8;         // bf16 per key row in LDS (padded)
constexpr int kVtStride = kBlockKeys + 8;   // bf16 per dimension row in LDS (padded)
constexpr float kLog2e = 1.4426950408889634f;

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(4))) uint32_t u32x4;
typedef __attribute__((ext_vector_type(2))) uint32_t u32x2;

struct AttendLds {
  uint16_t kd[kBlockKeys * kKdStride];      // keys, key-major, bf16 bits
  uint16_t vt[kLatent * kVtStride];         // latent values, dimension-major
  float scale[kBlockKeys][4];
  int32_t valid[kBlockKeys];
};

__device__ __forceinline__ uint32_t bf16_bits(float f) { return __float_as_uint(f) >> 16; }

// Two FP8 E4M3 bytes (the low or high half of w) to two bf16 in one word:
// exact, every E4M3 value is a bf16 value.
template <bool HI>
__device__ __forceinline__ uint32_t fp8x2_to_bf16x2(uint32_t w) {
  const auto f = __builtin_amdgcn_cvt_pk_f32_fp8((int)w, HI);
  return bf16_bits(f[0]) | (bf16_bits(f[1]) << 16);
}

// Loads the block of rows [key0, key0 + 32) of token t into LDS.
__device__ void load_block(const AttendParams& p, AttendLds& s, const int32_t* ids, int32_t key0,
                           int32_t key_end) {
  const int tid = threadIdx.x;
  if (tid < kBlockKeys) {
    const int32_t k = key0 + tid;
    const int32_t id = k < key_end ? ids[k] : -1;
    s.valid[tid] = (id >= 0 && (int64_t)id < p.pool_rows) ? id : -1;
  }
  __syncthreads();
  for (int piece = tid; piece < kBlockKeys * kPieces; piece += kT) {
    const int j = piece / kPieces;
    const int pc = piece - j * kPieces;
    const int32_t id = s.valid[j];
    u32x4 v = {0u, 0u, 0u, 0u};
    if (id >= 0) v = *reinterpret_cast<const u32x4*>(p.kv + (int64_t)id * kRowBytes + pc * 16);
    if (pc < kLatent / 16) {
      // 16 latent values: key-major copy and dimension-major copy
      uint32_t w[8];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        w[2 * i] = fp8x2_to_bf16x2<false>(v[i]);
        w[2 * i + 1] = fp8x2_to_bf16x2<true>(v[i]);
      }
      uint16_t* kd = s.kd + j * kKdStride + pc * 16;
      *reinterpret_cast<u32x4*>(kd) = u32x4{w[0], w[1], w[2], w[3]};
      *reinterpret_cast<u32x4*>(kd + 8) = u32x4{w[4], w[5], w[6], w[7]};
#pragma unroll
      for (int d = 0; d < 16; ++d)
        s.vt[(pc * 16 + d) * kVtStride + j] = (uint16_t)(w[d >> 1] >> (16 * (d & 1)));
    } else if (pc == kLatent / 16) {
      *reinterpret_cast<u32x4*>(&s.scale[j][0]) = v;       // four float32 scales
    } else {
      *reinterpret_cast<u32x4*>(s.kd + j * kKdStride + kLatent + (pc - 33) * 8) = v;  // rope
    }
  }
  __syncthreads();
}

__global__ void __launch_bounds__(kT) attend_kernel(AttendParams p) {
  extern __shared__ __attribute__((aligned(16))) unsigned char lds_raw[];
  AttendLds& s = *reinterpret_cast<AttendLds*>(lds_raw);
  const int split = blockIdx.x, hg = blockIdx.y, t = blockIdx.z;
  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63;
  const int col = l & 15, g = l >> 4;
  const int head = hg * (kHeadsPerWave * (kT / 64)) + w * kHeadsPerWave + col;
  const bool head_ok = head < p.num_heads;
  const int32_t key_lo = split * p.keys_per_split;
  const int32_t key_end = min(p.top_k, key_lo + p.keys_per_split);
  const int32_t* ids = p.row_ids + (int64_t)t * p.top_k;

  // Q^T as the B operand of the scores: this lane's head, dims 32 ks + 8 g ..
  bf16x8 qb[kDim / 32];
  const uint16_t* qh = p.q + ((int64_t)t * p.num_heads + (head_ok ? head : 0)) * kDim;
#pragma unroll
  for (int ks = 0; ks < kDim / 32; ++ks) {
    u32x4 v = head_ok ? *reinterpret_cast<const u32x4*>(qh + ks * 32 + 8 * g) : u32x4{0, 0, 0, 0};
    qb[ks] = __builtin_bit_cast(bf16x8, v);
  }
  f32x4 o[kLatent / 16];                     // O^T: dims 16 dt + 4 g + r, this lane's head
#pragma unroll
  for (int dt = 0; dt < kLatent / 16; ++dt) o[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY, l_run = 0.f;      // log2 domain
  const float qk_scale = p.sm_scale * kLog2e;

  for (int32_t key0 = key_lo; key0 < key_end; key0 += kBlockKeys) {
    load_block(p, s, ids, key0, key_end);
    // ---- scores: S^T[key][head] for the 32 keys, tiles mt of 16 keys
    float sc[2][4];
#pragma unroll
    for (int mt = 0; mt < 2; ++mt) {
      f32x4 acc[5];
#pragma unroll
      for (int i = 0; i < 5; ++i) acc[i] = f32x4{0.f, 0.f, 0.f, 0.f};
      const uint16_t* krow = s.kd + (mt * 16 + col) * kKdStride + 8 * g;
#pragma unroll
      for (int ks = 0; ks < kDim / 32; ++ks) {
        const bf16x8 a = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(krow + ks * 32));
        const int tile = ks < 16 ? ks / 4 : 4;
        acc[tile] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, qb[ks], acc[tile], 0, 0, 0);
      }
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int key = mt * 16 + 4 * g + r;
        float v = acc[4][r];
#pragma unroll
        for (int tl = 0; tl < 4; ++tl) v += s.scale[key][tl] * acc[tl][r];
        sc[mt][r] = s.valid[key] >= 0 ? v * qk_scale : -INFINITY;
      }
    }
    // ---- online softmax for this lane's head over the block's 32 keys
    float mb = -INFINITY;
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
      for (int r = 0; r < 4; ++r) mb = fmaxf(mb, sc[mt][r]);
    mb = fmaxf(mb, __shfl_xor(mb, 16));
    mb = fmaxf(mb, __shfl_xor(mb, 32));
    const float m_new = fmaxf(m_run, mb);
    const float alpha = m_new == -INFINITY ? 1.f : exp2f(m_run - m_new);
    float pr[2][4], ls = 0.f;
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        pr[mt][r] = m_new == -INFINITY ? 0.f : exp2f(sc[mt][r] - m_new);
        ls += pr[mt][r];
      }
    ls += __shfl_xor(ls, 16);
    ls += __shfl_xor(ls, 32);
    l_run = l_run * alpha + ls;
    m_run = m_new;
#pragma unroll
    for (int dt = 0; dt < kLatent / 16; ++dt) o[dt] *= alpha;
    // ---- O^T += V^T P'^T, one latent tile (8 dimension tiles) at a time;
    // this lane's 8 keys are 4 g .. 4 g + 3 and 16 + 4 g .. 16 + 4 g + 3
#pragma unroll
    for (int tl = 0; tl < 4; ++tl) {
      bf16x8 b;   // P' rounded to nearest bf16
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int r = 0; r < 4; ++r)
          b[4 * h + r] = (__bf16)(pr[h][r] * s.scale[h * 16 + 4 * g + r][tl]);
#pragma unroll
      for (int d8 = 0; d8 < 8; ++d8) {
        const int dt = tl * 8 + d8;
        const uint16_t* vrow = s.vt + (dt * 16 + col) * kVtStride;
        const u32x2 lo = *reinterpret_cast<const u32x2*>(vrow + 4 * g);
        const u32x2 hi = *reinterpret_cast<const u32x2*>(vrow + 16 + 4 * g);
        const bf16x8 a = __builtin_bit_cast(bf16x8, u32x4{lo[0], lo[1], hi[0], hi[1]});
        o[dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, o[dt], 0, 0, 0);
      }
    }
    __syncthreads();   // every wave is done with the block before the next load
  }

  if (!head_ok) return;
  const int64_t th = (int64_t)t * p.num_heads + head;
  if (p.splits == 1) {
    const float inv = l_run > 0.f ? 1.f / l_run : 0.f;
    float* out = p.out + th * kLatent;
#pragma unroll
    for (int dt = 0; dt < kLatent / 16; ++dt)
      *reinterpret_cast<f32x4*>(out + dt * 16 + 4 * g) = o[dt] * inv;
    if (g == 0) p.lse[th] = l_run > 0.f ? (m_run + log2f(l_run)) / kLog2e : -INFINITY;
    return;
  }
  const int64_t ps = ((int64_t)t * p.splits + split) * p.num_heads + head;
  float* po = p.part_o + ps * kLatent;
#pragma unroll
  for (int dt = 0; dt < kLatent / 16; ++dt)
    *reinterpret_cast<f32x4*>(po + dt * 16 + 4 * g) = o[dt];
  if (g == 0) {
    p.part_ml[2 * ps] = m_run;
    p.part_ml[2 * ps + 1] = l_run;
  }
}

// Merges the key splits of one (token, head): out = sum_s 2^(m_s - M) O_s /
// sum_s 2^(m_s - M) l_s, lse = (M + log2 L) / log2 e.
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
    const float f = exp2f(m - M);
    L += f * p.part_ml[2 * ps + 1];
    acc += f * *reinterpret_cast<const f32x4*>(p.part_o + ps * kLatent + 4 * threadIdx.x);
  }
  const float inv = L > 0.f ? 1.f / L : 0.f;
  *reinterpret_cast<f32x4*>(p.out + th * kLatent + 4 * threadIdx.x) = acc * inv;
  if (threadIdx.x == 0) p.lse[th] = L > 0.f ? (M + log2f(L)) / kLog2e : -INFINITY;
}

}  // namespace

size_t attend_lds_bytes() { return sizeof(AttendLds); }

void plan_attend(AttendParams& p, int64_t target_groups) {
  const int32_t hg = (p.num_heads + kAttendHeadsPerGroup - 1) / kAttendHeadsPerGroup;
  const int64_t base = (int64_t)p.num_tokens * hg;
  const int32_t blocks = (p.top_k + kBlockKeys - 1) / kBlockKeys;
  int64_t s = base > 0 ? (target_groups + base - 1) / base : 1;
  if (s < 1) s = 1;
  if (s > blocks) s = blocks;
  if (s > kAttendMaxSplits) s = kAttendMaxSplits;
  if (s < 1) s = 1;
  const int32_t per = (int32_t)(((blocks + s - 1) / s) * kBlockKeys);
  p.keys_per_split = per;
  p.splits = per > 0 ? (p.top_k + per - 1) / per : 1;
  if (p.splits < 1) p.splits = 1;
}

hipError_t launch_attend(const AttendParams& p, hipStream_t stream) {
  if (p.num_tokens == 0 || p.num_heads == 0) return hipSuccess;
  static std::atomic<uint64_t> raised{0};
  hipError_t e = allow_full_lds(reinterpret_cast<const void*>(attend_kernel), raised);
  if (e != hipSuccess) return e;
  const uint32_t hg = (uint32_t)((p.num_heads + kAttendHeadsPerGroup - 1) / kAttendHeadsPerGroup);
  e = launch_kernel(attend_kernel, dim3((uint32_t)p.splits, hg, (uint32_t)p.num_tokens), dim3(kT),
                    sizeof(AttendLds), stream, p);
  if (e != hipSuccess || p.splits == 1) return e;
  return launch_kernel(attend_combine_kernel, dim3((uint32_t)p.num_heads, (uint32_t)p.num_tokens),
                       dim3(128), 0, stream, p);
}

}  // namespace hs
