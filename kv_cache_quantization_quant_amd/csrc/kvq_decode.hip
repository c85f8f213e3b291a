// kvq_decode.hip — split-K merge and dispatch of the decode attention.
//
// Attention ("大模型量化从0到1（十三）：KV Cache 量化", §二): score_t = q·k̂_t / √D,
// p = softmax(score), out = Σ_t p_t v̂_t over every cached token. The split
// kernels (kvq_decode_mfma.hip: KIVI groups and window on the matrix cores,
// FP8 / FP16 tiles on the matrix cores) each write one partial (o[D], m, l)
// per (b, query head, split), with m a log2-domain maximum and o, l relative
// to it; this file merges them (log-sum-exp) into the output.
#include <hip/hip_fp16.h>
#include <hip/hip_runtime.h>

#include <math.h>

#include "kvq_internal.h"

namespace kvq {
namespace {

constexpr int kPart = kHeadDim + 2;   // partial record: o[D], m, l

__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) x = fmaxf(x, __shfl_xor(x, off));
  return x;
}
__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) x += __shfl_xor(x, off);
  return x;
}

// out[b, hq, :] = Σ_s o_s·2^(m_s − M) / Σ_s l_s·2^(m_s − M), one wave per
// (b, hq): the split maxima and sums are read by all lanes at once, then the
// weighted partial outputs with independent loads.
__global__ __launch_bounds__(64) void decode_merge_kernel(DecodeArgs a) {
  const int64_t row = blockIdx.x;   // b·Hq + hq
  const int lane = threadIdx.x;
  const float* part = a.ws + row * a.n_split * kPart;
  float mloc = -INFINITY;
  for (int s = lane; s < a.n_split; s += 64) mloc = fmaxf(mloc, part[s * kPart + kHeadDim]);
  const float M = wave_max(mloc);
  float lloc = 0.0f;
  for (int s = lane; s < a.n_split; s += 64) {
    const float ms = part[s * kPart + kHeadDim];
    if (ms != -INFINITY) lloc = fmaf(exp2f(ms - M), part[s * kPart + kHeadDim + 1], lloc);
  }
  const float L = wave_sum(lloc);
  float o0 = 0.0f, o1 = 0.0f;
#pragma unroll 8
  for (int s = 0; s < a.n_split; ++s) {
    const float ms = part[s * kPart + kHeadDim];
    const float2 os = *reinterpret_cast<const float2*>(part + s * kPart + 2 * lane);
    const float f = ms == -INFINITY ? 0.0f : exp2f(ms - M);
    o0 = fmaf(f, os.x, o0);
    o1 = fmaf(f, os.y, o1);
  }
  *reinterpret_cast<float2*>(a.out + row * kHeadDim + 2 * lane) = make_float2(o0 / L, o1 / L);
}

}  // namespace

// The split kernel of the cache's format, then the merge.
hipError_t launch_decode(const DecodeArgs& a_in, hipStream_t s) {
  DecodeArgs a = a_in;
  a.split_offset = 0;
  hipError_t e = hipSuccess;
  switch (a.src) {
    case kSrcKivi2:
    case kSrcKivi4:
      e = launch_kivi_mfma(a, s);
      break;
    case kSrcFp16:
    case kSrcFp8:
      e = launch_dense_mfma(a, s);
      break;
    default:
      return hipErrorInvalidValue;
  }
  if (e != hipSuccess) return e;
  decode_merge_kernel<<<a.B * a.Hq, 64, 0, s>>>(a);
  return hipGetLastError();
}

}  // namespace kvq
