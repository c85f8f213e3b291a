// kvq_quant.hip — cache-write kernels for gfx950: token copies into the FP16
// window / FP16 cache, and FP8 (E4M3 or E5M2) quantization with per-tensor or
// per-KV-head scales. (KIVI group quantization is in kvq_quant_kivi.hip.)
//
// FP8 ("LLM推理加速KV Cache量化压缩实战方案", section 自定义KV Cache量化的实现路径;
// "大模型量化从0到1（十三）：KV Cache 量化", §十八.4 and §十八.6):
//   s = amax(|x|) / FMAX per tensor or per KV head, FMAX = 448 (E4M3) or
//   57344 (E5M2); code = fp8(clamp(x / s, ±FMAX)) with the native gfx950 OCP
//   conversion (round to nearest even).
#include <hip/hip_fp16.h>
#include <hip/hip_runtime.h>

#include <algorithm>

#include "kvq_fp8.h"
#include "kvq_internal.h"
#include "kvq_quant_common.h"

namespace kvq {
namespace {

constexpr int kThreads = 256;

// Copies n_tokens tokens of K and V (16 bytes per thread); V is skipped when
// v_dst is null.
__global__ __launch_bounds__(kThreads) void copy_tokens_kernel(CopyTokensArgs a) {
  const int64_t idx = int64_t(blockIdx.x) * kThreads + threadIdx.x;  // uint4 index
  const int bh = blockIdx.y;
  constexpr int kChunks = kHeadDim / 8;                                // uint4 per token
  int64_t n = a.n_tokens, s0 = 0, d0 = a.dst_t0;
  if (a.ragged) {
    const int b = bh / a.H;
    s0 = a.seq.x[b];
    n = a.seq.y[b];
    d0 = a.seq.z[b];
  }
  if (idx >= n * kChunks) return;
  const int64_t tok = idx / kChunks;
  const int c = int(idx % kChunks);
  const int64_t s = bh * a.src_bh_stride + (s0 + tok) * kHeadDim + c * 8;
  const int64_t d = bh * a.dst_bh_stride + (d0 + tok) * kHeadDim + c * 8;
  *reinterpret_cast<uint4*>(a.k_dst + d) = *reinterpret_cast<const uint4*>(a.k_src + s);
  if (a.v_dst != nullptr)
    *reinterpret_cast<uint4*>(a.v_dst + d) = *reinterpret_cast<const uint4*>(a.v_src + s);
}

// V of the FP8 / FP16 caches, one workgroup per (tile, b·h): the tile's
// tokens are read token-major into LDS and written channel-major (a row of
// the tile's kGroup tokens per channel), as fp16 or as FP8 codes (the
// encoding of the row-major path: clamp to ±FMAX, then RNE) with the V scale
// of the block's KV head.
__global__ __launch_bounds__(kThreads) void v_tile_kernel(VTileArgs a) {
  __shared__ float tile[kGroup][kHeadDim + 1];
  const int bh = blockIdx.y;
  const int64_t g = a.dst_t0 / kGroup + blockIdx.x;
  const int64_t t_first = g * kGroup;
  const int64_t lo = max(a.dst_t0, t_first);
  const int64_t hi = min(a.dst_t0 + a.n_tokens, t_first + kGroup);
  const int64_t wr_hi = a.zero_tail ? t_first + kGroup : hi;
  const int tid = threadIdx.x;
  {
    // thread: token j of the tile, channels 16·(tid % 8) + [0, 16)
    const int j = tid / 8, c0 = 16 * (tid % 8);
    const int64_t t = t_first + j;
    if (t >= lo && t < hi) {
      const __half* src = a.v_src + bh * a.src_bh_stride + (t - a.dst_t0) * kHeadDim + c0;
      float f[16];
      halves_to_float(*reinterpret_cast<const uint4*>(src), f);
      halves_to_float(*reinterpret_cast<const uint4*>(src + 8), f + 8);
#pragma unroll
      for (int e = 0; e < 16; ++e) tile[j][c0 + e] = f[e];
    }
  }
  __syncthreads();
  // thread: channel d, tokens j0 + [0, 16)
  const int d = tid / 2, j0 = 16 * (tid % 2);
  const float sv = a.fp8 ? a.tensor_scale[a.scale_stride * (bh % a.H) + 1] : 1.0f;
  float x[16];
#pragma unroll
  for (int k = 0; k < 16; ++k) {
    const int64_t t = t_first + j0 + k;
    x[k] = (t >= lo && t < hi) ? tile[j0 + k][d] : 0.0f;
  }
  const int64_t row = ((int64_t(bh) * a.NT + g) * kHeadDim + d) * kGroup + j0;
  const bool full = lo <= t_first + j0 && t_first + j0 + 16 <= wr_hi;
  if (a.fp8) {
    uint8_t* dst = static_cast<uint8_t*>(a.v_dst) + row;
    uint32_t w[4] = {0u, 0u, 0u, 0u};
    if (sv != 0.0f) {
      const float rsv = 1.0f / sv;
      if (a.fmt == kE5M2) {
#pragma unroll
        for (int q = 0; q < 4; ++q) w[q] = fp8_encode4<kE5M2>(x + 4 * q, sv, rsv);
      } else {
#pragma unroll
        for (int q = 0; q < 4; ++q) w[q] = fp8_encode4<kE4M3>(x + 4 * q, sv, rsv);
      }
    }
    if (full) {
      *reinterpret_cast<uint4*>(dst) = make_uint4(w[0], w[1], w[2], w[3]);
    } else {
      for (int k = 0; k < 16; ++k) {
        const int64_t t = t_first + j0 + k;
        if (t >= lo && t < wr_hi) dst[k] = uint8_t(w[k / 4] >> (8 * (k % 4)));
      }
    }
  } else {
    __half* dst = static_cast<__half*>(a.v_dst) + row;
    if (full) {
      uint32_t w[8];
#pragma unroll
      for (int q = 0; q < 8; ++q)
        w[q] = uint32_t(__half_as_ushort(__float2half(x[2 * q]))) |
               (uint32_t(__half_as_ushort(__float2half(x[2 * q + 1]))) << 16);
      *reinterpret_cast<uint4*>(dst) = make_uint4(w[0], w[1], w[2], w[3]);
      *reinterpret_cast<uint4*>(dst + 8) = make_uint4(w[4], w[5], w[6], w[7]);
    } else {
      for (int k = 0; k < 16; ++k) {
        const int64_t t = t_first + j0 + k;
        if (t >= lo && t < wr_hi) dst[k] = __float2half(x[k]);
      }
    }
  }
}

// ------------------------------------------------------------------- FP8 ---

// zeroes the amax slots of `rows` scale rows
__global__ void fp8_clear_amax_kernel(float* ts, int rows) {
  for (int r = threadIdx.x; r < rows; r += blockDim.x) {
    ts[4 * r + 2] = 0.0f;
    ts[4 * r + 3] = 0.0f;
  }
}

// amax(|K|) and amax(|V|) over the source tokens: grid (blocks per (b, h),
// B·H), each thread a running packed-fp16 max of |x| (exact: the maximum of
// fp16 magnitudes is one of them); non-negative fp32 values order like their
// bit patterns, so an unsigned atomic max combines the wavefronts into the
// tensor's row, or the row of the block's KV head.
__global__ __launch_bounds__(kThreads) void fp8_amax_kernel(Fp8QuantArgs a) {
  constexpr int kChunks = kHeadDim / 8;                 // uint4 per token
  const int64_t n = a.n_tokens * kChunks;               // consecutive uint4 per (b, h)
  const __half* ks = a.k_src + int64_t(blockIdx.y) * a.src_bh_stride;
  const __half* vs = a.v_src + int64_t(blockIdx.y) * a.src_bh_stride;
  h2v mk = h2v{0, 0}, mv = h2v{0, 0};
  const int64_t stride = int64_t(gridDim.x) * kThreads;
  // four chunks of K and of V per step, all eight loads in flight together
  constexpr int kUnroll = 4;
  int64_t i = int64_t(blockIdx.x) * kThreads + threadIdx.x;
  for (; i + (kUnroll - 1) * stride < n; i += kUnroll * stride) {
    uint4 k[kUnroll], v[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      k[u] = *reinterpret_cast<const uint4*>(ks + 8 * (i + u * stride));
      v[u] = *reinterpret_cast<const uint4*>(vs + 8 * (i + u * stride));
    }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      mk = h2max(h2max(mk, as_h2(k[u].x & 0x7FFF7FFFu)), as_h2(k[u].y & 0x7FFF7FFFu));
      mk = h2max(h2max(mk, as_h2(k[u].z & 0x7FFF7FFFu)), as_h2(k[u].w & 0x7FFF7FFFu));
      mv = h2max(h2max(mv, as_h2(v[u].x & 0x7FFF7FFFu)), as_h2(v[u].y & 0x7FFF7FFFu));
      mv = h2max(h2max(mv, as_h2(v[u].z & 0x7FFF7FFFu)), as_h2(v[u].w & 0x7FFF7FFFu));
    }
  }
  for (; i < n; i += stride) {
    const uint4 k = *reinterpret_cast<const uint4*>(ks + 8 * i);
    const uint4 v = *reinterpret_cast<const uint4*>(vs + 8 * i);
    mk = h2max(h2max(mk, as_h2(k.x & 0x7FFF7FFFu)), as_h2(k.y & 0x7FFF7FFFu));
    mk = h2max(h2max(mk, as_h2(k.z & 0x7FFF7FFFu)), as_h2(k.w & 0x7FFF7FFFu));
    mv = h2max(h2max(mv, as_h2(v.x & 0x7FFF7FFFu)), as_h2(v.y & 0x7FFF7FFFu));
    mv = h2max(h2max(mv, as_h2(v.z & 0x7FFF7FFFu)), as_h2(v.w & 0x7FFF7FFFu));
  }
  float fk = fmaxf(float(mk[0]), float(mk[1]));
  float fv = fmaxf(float(mv[0]), float(mv[1]));
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) {
    fk = fmaxf(fk, __shfl_xor(fk, off));
    fv = fmaxf(fv, __shfl_xor(fv, off));
  }
  if ((threadIdx.x & 63) == 0) {
    float* row = a.tensor_scale + (a.per_head ? 4 * (int(blockIdx.y) % a.H) : 0);
    atomicMax(reinterpret_cast<unsigned int*>(row + 2), __float_as_uint(fk));
    atomicMax(reinterpret_cast<unsigned int*>(row + 3), __float_as_uint(fv));
  }
}

// Encodes n_tokens tokens per (b, h). FROM_AMAX: the prefill pass, scales come
// from the amax slots and are stored (by the blocks of batch row 0, one per
// scale row); otherwise the stored scales are reused.
template <bool FROM_AMAX, int FMT>
__global__ __launch_bounds__(kThreads) void fp8_encode_kernel(Fp8QuantArgs a) {
  constexpr int kChunks = kHeadDim / 8;
  const int bh = blockIdx.y;
  float* row = a.tensor_scale + (a.per_head ? 4 * (bh % a.H) : 0);
  float sk, sv;
  if (FROM_AMAX) {
    sk = row[2] / kFp8Max<FMT>;
    sv = row[3] / kFp8Max<FMT>;
    if (blockIdx.x == 0 && bh < (a.per_head ? a.H : 1) && threadIdx.x == 0) {
      row[0] = sk;
      row[1] = sv;
    }
  } else {
    sk = row[0];
    sv = row[1];
  }
  const int64_t idx = int64_t(blockIdx.x) * kThreads + threadIdx.x;
  if (idx >= a.n_tokens * kChunks) return;
  const int64_t tok = idx / kChunks;
  const int c = int(idx % kChunks);
  const int64_t s = bh * a.src_bh_stride + tok * kHeadDim + c * 8;
  const int64_t d = bh * a.dst_bh_stride + (a.dst_t0 + tok) * kHeadDim + c * 8;
  float fk[8];
  halves_to_float(*reinterpret_cast<const uint4*>(a.k_src + s), fk);
  uint2 ck = make_uint2(0u, 0u);
  if (sk != 0.0f) {
    const float rsk = 1.0f / sk;
    ck = make_uint2(fp8_encode4<FMT>(fk, sk, rsk), fp8_encode4<FMT>(fk + 4, sk, rsk));
  }
  *reinterpret_cast<uint2*>(a.k_codes + d) = ck;
  if (a.v_codes != nullptr) {
    float fv[8];
    halves_to_float(*reinterpret_cast<const uint4*>(a.v_src + s), fv);
    uint2 cv = make_uint2(0u, 0u);
    if (sv != 0.0f) {
      const float rsv = 1.0f / sv;
      cv = make_uint2(fp8_encode4<FMT>(fv, sv, rsv), fp8_encode4<FMT>(fv + 4, sv, rsv));
    }
    *reinterpret_cast<uint2*>(a.v_codes + d) = cv;
  }
}

// Query rows to E4M3 (attention in the FP8 domain): one wavefront per row of
// D = 128 fp32 values, two per lane; s = amax / 448 from a wavefront max.
__global__ __launch_bounds__(kThreads) void query_fp8_kernel(QueryQuantArgs a) {
  const int64_t row = int64_t(blockIdx.x) * (kThreads / 64) + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (row >= a.rows) return;                 // whole wavefronts leave together
  const float2 x = *reinterpret_cast<const float2*>(a.q + row * kHeadDim + 2 * lane);
  float amax = fmaxf(fabsf(x.x), fabsf(x.y));
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) amax = fmaxf(amax, __shfl_xor(amax, off));
  const float s = amax / kFp8Max<kE4M3>;
  uint32_t w = 0u;
  if (s != 0.0f) {
    const float rs = 1.0f / s;
    const bool tiny = s < kTinyQueryScale;
    w = fp8_pack2<kE4M3>(query_quotient(x.x, s, rs, tiny), query_quotient(x.y, s, rs, tiny),
                         0u, false);
  }
  *reinterpret_cast<uint16_t*>(a.codes + row * kHeadDim + 2 * lane) = uint16_t(w & 0xFFFFu);
  if (lane == 0) a.scales[row] = s;
}

}  // namespace

hipError_t launch_copy_tokens(const CopyTokensArgs& a, hipStream_t s) {
  if (a.n_tokens <= 0) return hipSuccess;
  const int64_t chunks = a.n_tokens * (kHeadDim / 8);
  dim3 grid(unsigned((chunks + kThreads - 1) / kThreads), a.bh_count);
  copy_tokens_kernel<<<grid, kThreads, 0, s>>>(a);
  return hipGetLastError();
}

hipError_t launch_v_tiles(const VTileArgs& a, hipStream_t s) {
  if (a.n_tokens <= 0) return hipSuccess;
  const int64_t first = a.dst_t0 / kGroup;
  const int64_t last = (a.dst_t0 + a.n_tokens - 1) / kGroup;
  dim3 grid(unsigned(last - first + 1), a.bh_count);
  v_tile_kernel<<<grid, kThreads, 0, s>>>(a);
  return hipGetLastError();
}

hipError_t launch_fp8_prefill(const Fp8QuantArgs& a, hipStream_t s) {
  fp8_clear_amax_kernel<<<1, 64, 0, s>>>(a.tensor_scale, a.per_head ? a.H : 1);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  // one workgroup per compute unit in all (at least one per (b, h), at most
  // one per 256 chunks of it): each (b, h) is then read by a few workgroups
  // sweeping it together, in windows of a few tens of KiB. Same-box A/B of the
  // 128K layer's FP8 prefill: 4096 workgroups 1069 µs, 1024 956, 512 928,
  // 256 902, 128 965.
  const int64_t per_bh_chunks = a.n_tokens * (kHeadDim / 8);
  const int64_t cus = std::max(1, device_compute_units());
  int64_t per_bh = (cus + a.bh_count - 1) / a.bh_count;
  per_bh = std::max<int64_t>(1, std::min<int64_t>(per_bh, (per_bh_chunks + kThreads - 1) / kThreads));
  fp8_amax_kernel<<<dim3(unsigned(per_bh), a.bh_count), kThreads, 0, s>>>(a);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  dim3 grid(unsigned((a.n_tokens * (kHeadDim / 8) + kThreads - 1) / kThreads), a.bh_count);
  if (a.fmt == kE5M2) fp8_encode_kernel<true, kE5M2><<<grid, kThreads, 0, s>>>(a);
  else fp8_encode_kernel<true, kE4M3><<<grid, kThreads, 0, s>>>(a);
  return hipGetLastError();
}

hipError_t launch_query_fp8(const QueryQuantArgs& a, hipStream_t s) {
  if (a.rows <= 0) return hipSuccess;
  constexpr int kRowsPerBlock = kThreads / 64;
  query_fp8_kernel<<<unsigned((a.rows + kRowsPerBlock - 1) / kRowsPerBlock), kThreads, 0, s>>>(a);
  return hipGetLastError();
}

hipError_t launch_fp8_append(const Fp8QuantArgs& a, hipStream_t s) {
  dim3 grid(unsigned((a.n_tokens * (kHeadDim / 8) + kThreads - 1) / kThreads), a.bh_count);
  if (a.fmt == kE5M2) fp8_encode_kernel<false, kE5M2><<<grid, kThreads, 0, s>>>(a);
  else fp8_encode_kernel<false, kE4M3><<<grid, kThreads, 0, s>>>(a);
  return hipGetLastError();
}

}  // namespace kvq
