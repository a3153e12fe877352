// Measurement kernels for the benchmark: a plain streaming device copy, the
// practical HBM ceiling that the gathers are compared with.  Built into a
// library of its own (libhs_probe.so); nothing on the hot path uses it.
//
// Each thread moves 16-byte pieces, U loads in flight before its stores.
// Layouts: grid-stride (consecutive lanes on consecutive pieces, the whole
// grid sweeping the buffer), or one contiguous chunk per workgroup.

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

constexpr int kT = 256;

template <int U, bool NT, bool CHUNK>
__global__ void __launch_bounds__(kT) copy_kernel(const u32x4* __restrict__ src,
                                                  u32x4* __restrict__ dst, int64_t n) {
  int64_t lo = 0, hi = n, step = (int64_t)gridDim.x * kT;
  int64_t i0 = (int64_t)blockIdx.x * kT + threadIdx.x;
  if (CHUNK) {
    const int64_t per = (n + gridDim.x - 1) / gridDim.x;
    lo = (int64_t)blockIdx.x * per;
    hi = lo + per < n ? lo + per : n;
    step = kT;
    i0 = lo + threadIdx.x;
  }
  (void)lo;
  for (int64_t i = i0; i < hi; i += step * U) {
    u32x4 v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t j = i + u * step;
      if (j < hi) v[u] = src[j];
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t j = i + u * step;
      if (j < hi) {
        if (NT) __builtin_nontemporal_store(v[u], dst + j);
        else dst[j] = v[u];
      }
    }
  }
}

}  // namespace

extern "C" {

// Copies `bytes` (a multiple of 16; both pointers 16-byte aligned) from src
// to dst on `stream` with `grid` workgroups of 256 threads.  variant: 0
// grid-stride, 4 loads in flight; 1 the same with non-temporal stores; 2
// grid-stride, 8 in flight, non-temporal; 3 one chunk per workgroup, 8 in
// flight, non-temporal.  Returns the launch's hipError_t.
int hs_probe_copy(const void* src, void* dst, size_t bytes, int grid, int variant,
                  hipStream_t stream) {
  if (bytes % 16 || ((uintptr_t)src | (uintptr_t)dst) % 16 || grid < 1) return (int)hipErrorInvalidValue;
  const int64_t n = (int64_t)(bytes / 16);
  const u32x4* s = static_cast<const u32x4*>(src);
  u32x4* d = static_cast<u32x4*>(dst);
  void (*fn)(const u32x4*, u32x4*, int64_t) = nullptr;
  switch (variant) {
    case 0: fn = copy_kernel<4, false, false>; break;
    case 1: fn = copy_kernel<4, true, false>; break;
    case 2: fn = copy_kernel<8, true, false>; break;
    case 3: fn = copy_kernel<8, true, true>; break;
    default: return (int)hipErrorInvalidValue;
  }
  void* args[] = {&s, &d, const_cast<int64_t*>(&n)};
  return (int)hipLaunchKernel(reinterpret_cast<const void*>(fn), dim3(grid), dim3(kT), args, 0,
                              stream);
}

}  // extern "C"
