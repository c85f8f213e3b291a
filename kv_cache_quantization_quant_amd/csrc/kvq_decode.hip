// kvq_decode.hip — split-K merge and dispatch of the decode attention.
//
// Attention ("大模型量化从0到1（十三）：KV Cache 量化", §二): score_t = q·k̂_t / √D,
// p = softmax(score), out = Σ_t p_t v̂_t over every cached token. The split
// kernels (kvq_decode_mfma.hip: KIVI groups and window on the matrix cores,
// FP8 / FP16 tiles on the matrix cores) each write one partial (o[D], m, l)
// per (b, query head, split), with m a log2-domain maximum and o, l relative
// to it; this file merges them (log-sum-exp) into the output. With one split
// per row the split kernels write o / l to the output themselves.
#include <hip/hip_fp16.h>
#include <hip/hip_runtime.h>

#include <math.h>

#include <mutex>

#include "../../include/kvq.h"
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
// (b, hq). The loads are issued together: lane s reads split s's (m, l), and
// every lane reads its two channels of up to kBatch partial outputs at once,
// so a head costs about one memory round trip per kBatch splits.
constexpr int kBatch = 32;
// The merge's own launch arguments (a few bytes instead of the split
// kernels' block with its ragged-batch table).
struct MergeArgs {
  const float* ws;        // [rows][n_split][D + 2] partials
  float* out;             // [rows][D]
  int n_split;
};

__global__ __launch_bounds__(64) void decode_merge_kernel(MergeArgs a) {
  const int64_t row = blockIdx.x;   // b·Hq + hq
  const int lane = threadIdx.x;
  const float* part = a.ws + row * a.n_split * kPart;
  float M = -INFINITY, L = 0.0f, o0 = 0.0f, o1 = 0.0f;
  for (int s0 = 0; s0 < a.n_split; s0 += kBatch) {
    const int n = min(kBatch, a.n_split - s0);
    float2 os[kBatch];
#pragma unroll
    for (int j = 0; j < kBatch; ++j)
      if (j < n) os[j] = *reinterpret_cast<const float2*>(part + (s0 + j) * kPart + 2 * lane);
    float2 ml = make_float2(-INFINITY, 0.0f);
    if (lane < n) ml = *reinterpret_cast<const float2*>(part + (s0 + lane) * kPart + kHeadDim);
    // this batch's maximum, then everything so far relative to the new one
    const float Mb = fmaxf(M, wave_max(ml.x));
    const float fl = ml.x == -INFINITY ? 0.0f : exp2f(ml.x - Mb);
    const float fo = M == -INFINITY ? 0.0f : exp2f(M - Mb);
    L = L * fo + wave_sum(fl * ml.y);
    o0 *= fo;
    o1 *= fo;
#pragma unroll
    for (int j = 0; j < kBatch; ++j) {
      if (j < n) {
        const float f = __shfl(fl, j);
        o0 = fmaf(f, os[j].x, o0);
        o1 = fmaf(f, os[j].y, o1);
      }
    }
    M = Mb;
  }
  *reinterpret_cast<float2*>(a.out + row * kHeadDim + 2 * lane) = make_float2(o0 / L, o1 / L);
}

// Split partials of kvq_decode_attention_static: one array per GPU (each
// device that loads this code object gets its own copy), never passed to a
// kernel by name — host code takes its device address from static_workspace.
static __device__ __align__(256) unsigned char scratch[KVQ_STATIC_WORKSPACE_BYTES];

}  // namespace

hipError_t static_workspace(void** ptr) {
  constexpr int kMaxDevices = 64;
  static std::mutex mu;
  static void* addr[kMaxDevices] = {};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (addr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (p == nullptr) return hipErrorInvalidSymbol;
    addr[dev] = p;
  }
  *ptr = addr[dev];
  return hipSuccess;
}

// The split kernel of the cache's format, then the merge (none with one split
// per row: the split kernel writes the output).
hipError_t launch_decode(const DecodeArgs& a_in, hipStream_t s) {
  const DecodeArgs& a = a_in;
  hipError_t e = hipSuccess;
  switch (a.src) {
    case kSrcKivi2:
    case kSrcKivi4:
      e = launch_kivi_mfma(a, s);
      break;
    case kSrcFp16:
    case kSrcFp8:
    case kSrcE5M2:
      e = launch_dense_mfma(a, s);
      break;
    default:
      return hipErrorInvalidValue;
  }
  if (e != hipSuccess) return e;
  if (KVQ_DIRECT_SINGLE_SPLIT && a.n_split == 1) return hipSuccess;   // written by the split
  MergeArgs m;
  m.ws = a.ws;
  m.out = a.out;
  m.n_split = a.n_split;
  decode_merge_kernel<<<a.B * a.Hq, 64, 0, s>>>(m);
  return hipGetLastError();
}

}  // namespace kvq
