// kvq_quant_common.h — small fp16 helpers shared by the cache-write kernels
// (packed fp16 min / max, fp16 → fp32 unpacking).
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

}  // namespace kvq
