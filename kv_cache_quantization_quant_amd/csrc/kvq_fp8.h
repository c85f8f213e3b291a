// kvq_fp8.h — FP8 encoding shared by the cache writers (kvq_quant.hip) and
// the query quantizer of the FP8-domain decode (kvq_decode_mfma.hip), so that
// both produce the codes of one definition. Not part of the public interface.
//
// Encoding ("大模型量化从0到1（十三）：KV Cache 量化", §十 FP8 formula, and
// "LLM推理加速KV Cache量化压缩实战方案", section 自定义KV Cache量化的实现路径):
// code = fp8(clamp(x / s, ±FMAX)), round to nearest even, OCP E4M3 ("fn",
// FMAX = 448) or E5M2 (FMAX = 57344, §十八.4 of the first page).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kvq_internal.h"

namespace kvq {

// x / s correctly rounded, from rs = RN(1 / s) (one IEEE division per
// thread): q = RN(x·rs) is within an ulp of x / s, the residual x − q·s is
// exact in one fma, and RN(q + residual·rs) is the correctly rounded quotient
// (Markstein's theorem for round-to-nearest; it needs no overflow or underflow
// in these steps, which holds for fp16 x and a scale amax / FMAX ≥ 2⁻²⁴ /
// 57344, and for fp32 x with a scale ≥ 2⁻¹⁰⁰). The quotient takes the sign
// of x, which keeps −0 / s = −0 (the sum above would give +0).
__device__ __forceinline__ float div_by_scale(float x, float s, float rs) {
  const float q = x * rs;
  const float res = fmaf(-q, s, x);
  return __builtin_copysignf(fmaf(res, rs, q), x);
}

// Largest finite value of each FP8 format: E4M3 "fn" 1.75·2^8, E5M2 1.75·2^15.
template <int FMT>
constexpr float kFp8Max = FMT == kE5M2 ? 57344.0f : 448.0f;

// Two clamped quotients into byte pair `high` of w (RNE hardware conversion).
template <int FMT>
__device__ __forceinline__ uint32_t fp8_pack2(float t0, float t1, uint32_t w, bool high) {
  constexpr float M = kFp8Max<FMT>;
  t0 = fminf(fmaxf(t0, -M), M);
  t1 = fminf(fmaxf(t1, -M), M);
  if (FMT == kE5M2)
    return high ? __builtin_amdgcn_cvt_pk_bf8_f32(t0, t1, w, true)
                : __builtin_amdgcn_cvt_pk_bf8_f32(t0, t1, w, false);
  return high ? __builtin_amdgcn_cvt_pk_fp8_f32(t0, t1, w, true)
              : __builtin_amdgcn_cvt_pk_fp8_f32(t0, t1, w, false);
}

// Four codes: t = clamp(x / s, ±FMAX), then the conversion, two per instruction.
template <int FMT>
__device__ __forceinline__ uint32_t fp8_encode4(const float* x, float s, float rs) {
  uint32_t w = fp8_pack2<FMT>(div_by_scale(x[0], s, rs), div_by_scale(x[1], s, rs), 0u, false);
  return fp8_pack2<FMT>(div_by_scale(x[2], s, rs), div_by_scale(x[3], s, rs), w, true);
}

// Per-row query scale and quotients (FP8-domain attention): s = amax / 448;
// a scale below 2⁻¹⁰⁰ (possible for fp32 queries, never for the fp16 cache)
// takes the IEEE division per element instead of the reciprocal form.
__device__ __forceinline__ float query_quotient(float x, float s, float rs, bool tiny) {
  return tiny ? x / s : div_by_scale(x, s, rs);
}
constexpr float kTinyQueryScale = 0x1p-100f;

}  // namespace kvq
