// kvq_quant_common.h — small helpers shared by the cache-write kernels
// (packed fp16 min / max, fp16 → fp32 unpacking, non-temporal stores).
#pragma once
#include <hip/hip_fp16.h>
#include <hip/hip_runtime.h>

namespace kvq {

__device__ __forceinline__ void halves_to_float(const uint4& raw, float* f) {
  const __half2* h = reinterpret_cast<const __half2*>(&raw);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    float2 v = __half22float2(h[i]);
    f[2 * i] = v.x;
    f[2 * i + 1] = v.y;
  }
}

typedef _Float16 h2v __attribute__((ext_vector_type(2)));

__device__ __forceinline__ h2v as_h2(uint32_t u) { return __builtin_bit_cast(h2v, u); }
__device__ __forceinline__ uint32_t as_u(h2v h) { return __builtin_bit_cast(uint32_t, h); }
__device__ __forceinline__ h2v h2max(h2v a, h2v b) { return __builtin_elementwise_max(a, b); }
__device__ __forceinline__ h2v h2min(h2v a, h2v b) { return __builtin_elementwise_min(a, b); }

// Stores of KIVI cache data (codes, scales, zero-points), non-temporal: the
// decode reads them much later, so they need not stay in the caches, and a
// prefill leaves no dirty lines behind for the next kernel's reads to evict
// and write back. The empty asm keeps the optimizer from merging a store
// with its copy on another path, which drops the non-temporal mark.
template <typename T>
__device__ __forceinline__ void store_nt(T* p, T x) {
  asm volatile("" ::: "memory");
  __builtin_nontemporal_store(x, p);
}
// two 32-bit words at an 8-byte aligned address
typedef unsigned int u32x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ void store_nt2(void* p, uint32_t x0, uint32_t x1) {
  store_nt(static_cast<u32x2_t*>(p), u32x2_t{x0, x1});
}

}  // namespace kvq
