// kvq_quant.hip — cache-write kernels for gfx950: KIVI group quantization
// (prefill and window flush), token copies into the FP16 window / FP16 cache,
// and FP8 E4M3 per-tensor quantization.
//
// KIVI ("4.4 KV Cache 量化：KIVI 2-bit 与 FP8 KV Cache", §2 and §3.2;
// "大模型量化从0到1（十三）：KV Cache 量化", §九 and the affine formula of §十):
// K gets one (scale, zero) per (group of 32 tokens, channel), V one per token.
// Quantizer, each op in fp32 and correctly rounded (no contraction; the
// library is built with -ffp-contract=off):
//   s = (max − min) / (2^b − 1), z = min,
//   code = clamp(rint((x − min) / s), 0, 2^b − 1), code = 0 when s == 0.
//
// FP8 ("LLM推理加速KV Cache量化压缩实战方案", section 自定义KV Cache量化的实现路径):
//   s = amax(|x|) / 448 per tensor; code = E4M3(clamp(x / s, ±448)) with the
//   native gfx950 OCP conversion (round to nearest even).
#include <hip/hip_fp16.h>
#include <hip/hip_runtime.h>

#include "kvq_internal.h"

namespace kvq {
namespace {

constexpr int kThreads = 256;

__device__ __forceinline__ uint32_t affine_code(float x, float mn, float s, float qmax) {
  if (s == 0.0f) return 0u;
  float r = rintf((x - mn) / s);
  r = fminf(fmaxf(r, 0.0f), qmax);
  return static_cast<uint32_t>(r);
}

__device__ __forceinline__ void halves_to_float(const uint4& raw, float* f) {
  const __half2* h = reinterpret_cast<const __half2*>(&raw);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    float2 v = __half22float2(h[i]);
    f[2 * i] = v.x;
    f[2 * i + 1] = v.y;
  }
}

// One workgroup quantizes one group (32 tokens × 128 channels) of K and of V
// for one (b, h). Thread (t = tid / 8, j = tid % 8) holds channels
// [16j, 16j + 16) of token t: the loads cover 256 contiguous bytes per token.
template <int BITS>
__global__ __launch_bounds__(kThreads) void kivi_quantize_kernel(KiviQuantArgs a) {
  constexpr int PER = 32 / BITS;           // codes per 32-bit word
  constexpr int KW = kHeadDim / PER;       // K words per token
  constexpr int VW = kGroup / PER;         // V words per (group, channel)
  constexpr float QMAX = float((1 << BITS) - 1);

  __shared__ __half tile_k[kGroup][kHeadDim];
  __shared__ float s_k[kHeadDim];
  __shared__ float z_k[kHeadDim];
  __shared__ uint8_t vcode[kHeadDim][kGroup + 4];

  const int g = blockIdx.x;
  const int bh = blockIdx.y;
  const int tid = threadIdx.x;
  const int t = tid >> 3;
  const int j = tid & 7;
  const int64_t gg = a.g0 + g;
  const int64_t CT = a.NG * kGroup;

  const int64_t src = bh * a.src_bh_stride + int64_t(g * kGroup + t) * kHeadDim + j * 16;
  const uint4 k0 = *reinterpret_cast<const uint4*>(a.k_src + src);
  const uint4 k1 = *reinterpret_cast<const uint4*>(a.k_src + src + 8);
  const uint4 v0 = *reinterpret_cast<const uint4*>(a.v_src + src);
  const uint4 v1 = *reinterpret_cast<const uint4*>(a.v_src + src + 8);
  *reinterpret_cast<uint4*>(&tile_k[t][j * 16]) = k0;
  *reinterpret_cast<uint4*>(&tile_k[t][j * 16 + 8]) = k1;

  // ---- V: per-token statistics over the 128 channels (8 consecutive lanes).
  float vx[16];
  halves_to_float(v0, vx);
  halves_to_float(v1, vx + 8);
  float vmn = vx[0], vmx = vx[0];
#pragma unroll
  for (int i = 1; i < 16; ++i) {
    vmn = fminf(vmn, vx[i]);
    vmx = fmaxf(vmx, vx[i]);
  }
#pragma unroll
  for (int off = 1; off < 8; off <<= 1) {
    vmn = fminf(vmn, __shfl_xor(vmn, off));
    vmx = fmaxf(vmx, __shfl_xor(vmx, off));
  }
  const float vs = (vmx - vmn) / QMAX;
  if (j == 0) {
    a.v_scale[bh * CT + gg * kGroup + t] = vs;
    a.v_zero[bh * CT + gg * kGroup + t] = vmn;
  }
#pragma unroll
  for (int i = 0; i < 16; ++i) vcode[j * 16 + i][t] = uint8_t(affine_code(vx[i], vmn, vs, QMAX));
  __syncthreads();

  // ---- K: per-channel statistics over the group's 32 tokens.
  if (tid < kHeadDim) {
    const int d = tid;
    float mn = __half2float(tile_k[0][d]);
    float mx = mn;
#pragma unroll 8
    for (int tt = 1; tt < kGroup; ++tt) {
      const float x = __half2float(tile_k[tt][d]);
      mn = fminf(mn, x);
      mx = fmaxf(mx, x);
    }
    const float s = (mx - mn) / QMAX;
    s_k[d] = s;
    z_k[d] = mn;
    a.k_scale[(bh * a.NG + gg) * kHeadDim + d] = s;
    a.k_zero[(bh * a.NG + gg) * kHeadDim + d] = mn;
  }
  __syncthreads();

  // ---- K codes: token t, channels [16j, 16j + 16), packed along channels.
  float kx[16];
  halves_to_float(k0, kx);
  halves_to_float(k1, kx + 8);
  uint32_t w0 = 0, w1 = 0;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int d = j * 16 + i;
    const uint32_t c = affine_code(kx[i], z_k[d], s_k[d], QMAX);
    if (BITS == 2) {
      w0 |= c << (2 * i);
    } else if (i < 8) {
      w0 |= c << (4 * i);
    } else {
      w1 |= c << (4 * (i - 8));
    }
  }
  uint32_t* kdst = a.k_codes + (bh * CT + gg * kGroup + t) * KW;
  if (BITS == 2) {
    kdst[j] = w0;
  } else {
    *reinterpret_cast<uint2*>(kdst + 2 * j) = make_uint2(w0, w1);
  }

  // ---- V codes: per channel, the group's 32 token codes packed along tokens;
  // within a word, even tokens fill the low half-word and odd tokens the high.
  uint32_t* vdst = a.v_codes + (bh * a.NG + gg) * kHeadDim * VW;
  for (int idx = tid; idx < kHeadDim * VW; idx += kThreads) {
    const int d = idx / VW;
    const int w = idx % VW;
    uint32_t word = 0;
#pragma unroll
    for (int i = 0; i < PER; ++i)
      word |= uint32_t(vcode[d][w * PER + i]) << (BITS * (i / 2) + 16 * (i % 2));
    vdst[idx] = word;
  }
}

__device__ __forceinline__ uint32_t fp8_encode4(const float* x, float s) {
  // t = clamp(x / s, ±448), then the hardware RNE conversion, two per call.
  float t[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) t[e] = fminf(fmaxf(x[e] / s, -448.0f), 448.0f);
  uint32_t w = __builtin_amdgcn_cvt_pk_fp8_f32(t[0], t[1], 0, false);
  w = __builtin_amdgcn_cvt_pk_fp8_f32(t[2], t[3], w, true);
  return w;
}

// Copies n_tokens tokens of K and V (16 bytes per thread); V is skipped when
// v_dst is null.
__global__ __launch_bounds__(kThreads) void copy_tokens_kernel(CopyTokensArgs a) {
  const int64_t idx = int64_t(blockIdx.x) * kThreads + threadIdx.x;  // uint4 index
  const int bh = blockIdx.y;
  constexpr int kChunks = kHeadDim / 8;                                // uint4 per token
  if (idx >= a.n_tokens * kChunks) return;
  const int64_t tok = idx / kChunks;
  const int c = int(idx % kChunks);
  const int64_t s = bh * a.src_bh_stride + tok * kHeadDim + c * 8;
  const int64_t d = bh * a.dst_bh_stride + (a.dst_t0 + tok) * kHeadDim + c * 8;
  *reinterpret_cast<uint4*>(a.k_dst + d) = *reinterpret_cast<const uint4*>(a.k_src + s);
  if (a.v_dst != nullptr)
    *reinterpret_cast<uint4*>(a.v_dst + d) = *reinterpret_cast<const uint4*>(a.v_src + s);
}

// V of the FP8 / FP16 caches, one workgroup per (tile, b·h): the tile's
// tokens are read token-major into LDS and written channel-major (a row of
// the tile's kGroup tokens per channel), as fp16 or as E4M3 codes (the FP8
// encoding of the row-major path: clamp to ±448, then RNE).
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
  const float sv = a.fp8 ? a.tensor_scale[1] : 1.0f;
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
#pragma unroll
      for (int q = 0; q < 4; ++q) w[q] = fp8_encode4(x + 4 * q, sv);
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

__global__ void fp8_clear_amax_kernel(float* ts) {
  if (threadIdx.x == 0) {
    ts[2] = 0.0f;
    ts[3] = 0.0f;
  }
}

// amax(|K|) and amax(|V|) over the source tokens; non-negative fp32 values
// order like their bit patterns, so an unsigned atomic max suffices.
__global__ __launch_bounds__(kThreads) void fp8_amax_kernel(Fp8QuantArgs a) {
  constexpr int kChunks = kHeadDim / 8;
  const int64_t per_bh = a.n_tokens * kChunks;
  const int64_t total = per_bh * a.bh_count;
  float mk = 0.0f, mv = 0.0f;
  for (int64_t i = int64_t(blockIdx.x) * kThreads + threadIdx.x; i < total;
       i += int64_t(gridDim.x) * kThreads) {
    const int64_t bh = i / per_bh;
    const int64_t r = i % per_bh;
    const int64_t s = bh * a.src_bh_stride + (r / kChunks) * kHeadDim + (r % kChunks) * 8;
    float fk[8], fv[8];
    halves_to_float(*reinterpret_cast<const uint4*>(a.k_src + s), fk);
    halves_to_float(*reinterpret_cast<const uint4*>(a.v_src + s), fv);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      mk = fmaxf(mk, fabsf(fk[e]));
      mv = fmaxf(mv, fabsf(fv[e]));
    }
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) {
    mk = fmaxf(mk, __shfl_xor(mk, off));
    mv = fmaxf(mv, __shfl_xor(mv, off));
  }
  if ((threadIdx.x & 63) == 0) {
    atomicMax(reinterpret_cast<unsigned int*>(a.tensor_scale + 2), __float_as_uint(mk));
    atomicMax(reinterpret_cast<unsigned int*>(a.tensor_scale + 3), __float_as_uint(mv));
  }
}


// Encodes n_tokens tokens per (b, h). FROM_AMAX: the prefill pass, scales come
// from the amax slots and are stored; otherwise the stored scales are reused.
template <bool FROM_AMAX>
__global__ __launch_bounds__(kThreads) void fp8_encode_kernel(Fp8QuantArgs a) {
  constexpr int kChunks = kHeadDim / 8;
  float sk, sv;
  if (FROM_AMAX) {
    sk = a.tensor_scale[2] / 448.0f;
    sv = a.tensor_scale[3] / 448.0f;
    if (blockIdx.x == 0 && blockIdx.y == 0 && threadIdx.x == 0) {
      a.tensor_scale[0] = sk;
      a.tensor_scale[1] = sv;
    }
  } else {
    sk = a.tensor_scale[0];
    sv = a.tensor_scale[1];
  }
  const int64_t idx = int64_t(blockIdx.x) * kThreads + threadIdx.x;
  const int bh = blockIdx.y;
  if (idx >= a.n_tokens * kChunks) return;
  const int64_t tok = idx / kChunks;
  const int c = int(idx % kChunks);
  const int64_t s = bh * a.src_bh_stride + tok * kHeadDim + c * 8;
  const int64_t d = bh * a.dst_bh_stride + (a.dst_t0 + tok) * kHeadDim + c * 8;
  float fk[8], fv[8];
  halves_to_float(*reinterpret_cast<const uint4*>(a.k_src + s), fk);
  halves_to_float(*reinterpret_cast<const uint4*>(a.v_src + s), fv);
  uint2 ck = make_uint2(0u, 0u), cv = make_uint2(0u, 0u);
  if (sk != 0.0f) ck = make_uint2(fp8_encode4(fk, sk), fp8_encode4(fk + 4, sk));
  if (sv != 0.0f) cv = make_uint2(fp8_encode4(fv, sv), fp8_encode4(fv + 4, sv));
  *reinterpret_cast<uint2*>(a.k_codes + d) = ck;
  if (a.v_codes != nullptr) *reinterpret_cast<uint2*>(a.v_codes + d) = cv;
}

}  // namespace

hipError_t launch_kivi_quantize(const KiviQuantArgs& a, hipStream_t s) {
  if (a.n_groups <= 0) return hipSuccess;
  dim3 grid(a.n_groups, a.bh_count);
  if (a.bits == 2) {
    kivi_quantize_kernel<2><<<grid, kThreads, 0, s>>>(a);
  } else {
    kivi_quantize_kernel<4><<<grid, kThreads, 0, s>>>(a);
  }
  return hipGetLastError();
}

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
  fp8_clear_amax_kernel<<<1, 64, 0, s>>>(a.tensor_scale);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int64_t chunks = a.n_tokens * (kHeadDim / 8) * a.bh_count;
  int64_t blocks = (chunks + kThreads - 1) / kThreads;
  if (blocks > 4096) blocks = 4096;
  fp8_amax_kernel<<<unsigned(blocks), kThreads, 0, s>>>(a);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  dim3 grid(unsigned((a.n_tokens * (kHeadDim / 8) + kThreads - 1) / kThreads), a.bh_count);
  fp8_encode_kernel<true><<<grid, kThreads, 0, s>>>(a);
  return hipGetLastError();
}

hipError_t launch_fp8_append(const Fp8QuantArgs& a, hipStream_t s) {
  dim3 grid(unsigned((a.n_tokens * (kHeadDim / 8) + kThreads - 1) / kThreads), a.bh_count);
  fp8_encode_kernel<false><<<grid, kThreads, 0, s>>>(a);
  return hipGetLastError();
}

}  // namespace kvq
