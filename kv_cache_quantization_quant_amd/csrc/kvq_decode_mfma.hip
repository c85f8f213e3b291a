// kvq_decode_mfma.hip — decode attention over the KIVI grouped region on the
// gfx950 matrix cores (MFMA 16x16x32).
//
// Attention as in "大模型量化从0到1（十三）：KV Cache 量化", §二 (score = q·k̂/√D,
// softmax, Σ p·v̂), over KIVI groups ("4.4 KV Cache 量化：KIVI 2-bit 与 FP8 KV
// Cache", §3.2: K per channel, V per token, groups of 32 tokens). The
// dequantization is folded so that the codes enter the matrix cores as exact
// small integers:
//   q·k̂_t = Σ_d (q_d·s[g,d])·c[t,d] + Σ_d q_d·z[g,d]          (K per channel)
//   Σ_t p_t·v̂_t[d] = Σ_t (p_t·s_t)·c[t,d] + Σ_t p_t·z_t         (V per token)
//
// One wavefront processes one 32-token group at a time; lane l has r = l%16,
// u = l/16, head slot hs = r%8 (up to 8 query heads of one KV head), and
// part = r/8 (0: high, 1: low half of a two-term split).
//
// Scores, Sᵀ[token][col] = Σ_d code[token][d] · Q'[d][col], as f16 MFMA:
//   A = K codes of token 16·tile + r as fp16 subnormals code·f·2⁻²⁴ (f a power
//       of 4 or 16 given by the code's bit position, so that only AND masks are
//       needed), B = Q' for column r: head hs, the fp16 high (part 0) or low
//       (part 1) term of q_d·s[g,d]·log2(e)/√D / f. C starts at the head's
//       z-term Σ_d q_d·z[g,d] (times 2⁻²⁴). The two parts of a head sit in
//       columns hs and hs+8 of the same lane row; a DPP rotate adds them.
// The Sᵀ accumulator layout (lane holds column r, tokens 4u..4u+3 of a tile)
// is exactly the B-operand layout of the value product, so no transpose is
// needed:
//   Oᵀ[d][col] = Σ_t (128 + f'·code[t][d]) · P'[t][col]   (bf16 MFMA, 8 tiles
//       of 16 channels), with A = codes OR-ed into the mantissa of 128.0 and
//       B = P' = p_t·s_t/f' as a bf16 high + low split (columns hs, hs+8);
//   Σ_t P'[t][col] from one more MFMA with A = 1 removes the 128 offset.
// Online softmax in the log2 domain with a per-head reference maximum that
// is only raised (with rescaling) when a score exceeds it by more than 16.
#include <hip/hip_fp16.h>
#include <hip/hip_runtime.h>

#include <math.h>

#include "kvq_internal.h"

namespace kvq {
namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / 64;
constexpr int kPart = kHeadDim + 2;
constexpr float kLazy = 16.0f;                 // log2-domain slack before rescaling
constexpr float kTwo24 = 16777216.0f;
constexpr float kTwoM24 = 1.0f / 16777216.0f;

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ f16x8 as_f16x8(u32x4 v) { return __builtin_bit_cast(f16x8, v); }
__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

// value of lane l ^ 8 (rotate by 8 inside each row of 16 lanes)
__device__ __forceinline__ float xor8(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x128, 0xF, 0xF, false));
}
__device__ __forceinline__ uint32_t xor8u(uint32_t x) {
  return uint32_t(__builtin_amdgcn_update_dpp(0, int(x), 0x128, 0xF, 0xF, false));
}
// sum / max over the 8 lanes sharing l % 8 (xor 8, 16, 32)
__device__ __forceinline__ float head_sum(float x) {
  x += xor8(x);
  x += __shfl_xor(x, 16);
  x += __shfl_xor(x, 32);
  return x;
}
__device__ __forceinline__ float head_max(float x) {
  x = fmaxf(x, xor8(x));
  x = fmaxf(x, __shfl_xor(x, 16));
  x = fmaxf(x, __shfl_xor(x, 32));
  return x;
}

__device__ __forceinline__ uint32_t f16_bits(float x) {
  return uint32_t(__builtin_bit_cast(unsigned short, (_Float16)x));
}
// fp16 high + low split of x; returns the requested term's bits.
__device__ __forceinline__ uint32_t split_f16(float x, bool low) {
  const _Float16 hi = (_Float16)x;
  const float rest = x - (float)hi;
  return low ? uint32_t(__builtin_bit_cast(unsigned short, (_Float16)rest))
             : uint32_t(__builtin_bit_cast(unsigned short, hi));
}

// ---- K code positions (see the header comment). For local k-step sl (0..3)
// and k-slot j (0..7) of a lane whose 32 channels start at 32·u:
//   2-bit: word sl/2 of the lane's two words; pair m = 4·(sl%2) + j/2 of
//          that word, code position m + 8·(j%2); factor 4^q(m).
//   4-bit: word sl of the lane's four words; pair m = j/2, position
//          m + 4·(j%2); factor 16^(m%2).
template <int BITS>
__device__ __forceinline__ constexpr int k_channel(int sl, int j) {
  if (BITS == 2) return 16 * (sl / 2) + (4 * (sl % 2) + j / 2) + 8 * (j % 2);
  return 8 * sl + j / 2 + 4 * (j % 2);
}
template <int BITS>
__device__ __forceinline__ constexpr float k_factor(int sl, int j) {
  if (BITS == 2) {
    const int m = 4 * (sl % 2) + j / 2;
    const int q = (m < 3) ? m : (m < 6 ? m - 3 : m - 6);
    return float(1 << (2 * q));
  }
  return ((j / 2) % 2) ? 16.0f : 1.0f;
}

// A operand of one token: 4 k-steps × 4 dwords of fp16 subnormal pairs.
template <int BITS>
__device__ __forceinline__ void k_unpack(const uint32_t* w, u32x4* A) {
  if (BITS == 2) {
#pragma unroll
    for (int x = 0; x < 2; ++x) {
      const uint32_t t0 = w[x], t6 = w[x] >> 6, t12 = w[x] >> 12;
      const uint32_t d[8] = {t0 & 0x00030003u,  t0 & 0x000C000Cu,  t0 & 0x00300030u,
                             t6 & 0x00030003u,  t6 & 0x000C000Cu,  t6 & 0x00300030u,
                             t12 & 0x00030003u, t12 & 0x000C000Cu};
      A[2 * x] = u32x4{d[0], d[1], d[2], d[3]};
      A[2 * x + 1] = u32x4{d[4], d[5], d[6], d[7]};
    }
  } else {
#pragma unroll
    for (int x = 0; x < 4; ++x) {
      const uint32_t t0 = w[x], t8 = w[x] >> 8;
      A[x] = u32x4{t0 & 0x000F000Fu, t0 & 0x00F000F0u, t8 & 0x000F000Fu, t8 & 0x00F000F0u};
    }
  }
}

template <int BITS>
__global__ __launch_bounds__(kThreads) void kivi_mfma_split_kernel(DecodeArgs a) {
  constexpr int KW = kHeadDim * BITS / 32;     // K words per token
  constexpr int VW = kGroup * BITS / 32;       // V words per (group, channel)
  constexpr int LW = 32 * BITS / 32;           // K words per lane (32 channels)

  __shared__ float mo[kWaves][8][kHeadDim];
  __shared__ float ml[kWaves][8][2];

  const int split = blockIdx.x;
  const int bh = blockIdx.y;
  const int b = bh / a.H;
  const int h_kv = bh % a.H;
  const int hq0 = h_kv * a.nq + int(blockIdx.z) * a.heads_per_chunk;
  const int nh = min(a.heads_per_chunk, a.nq - int(blockIdx.z) * a.heads_per_chunk);
  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int r = lane & 15;
  const int u = lane >> 4;
  const int hs = r & 7;
  const bool low = r >= 8;
  const int64_t CT = a.main_bh_tokens;

  // ---- per-lane constants: this lane's 32 channels [32u, 32u+32) of head hs
  float qf[4][8];          // q_d·log2e/√D / f, by (k-step, k-slot)
  float qz[16];            // q_d·log2e/√D for the z-term: channels 32u + 16·part + c
  {
    const bool valid = hs < nh;
    const float* qrow = a.q + (int64_t(b) * a.Hq + hq0 + (valid ? hs : 0)) * kHeadDim + 32 * u;
#pragma unroll
    for (int sl = 0; sl < 4; ++sl)
#pragma unroll
      for (int j = 0; j < 8; ++j)
        qf[sl][j] = valid ? qrow[k_channel<BITS>(sl, j)] * a.qscale / k_factor<BITS>(sl, j) : 0.0f;
#pragma unroll
    for (int c = 0; c < 16; ++c) qz[c] = valid ? qrow[16 * (low ? 1 : 0) + c] * a.qscale : 0.0f;
  }
  // V: lane tokens 16·tile + 4u + i; factor f' and shift of the code fields
  float vfac[4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
    vfac[i] = (BITS == 2) ? ((i / 2) ? 0.25f : 1.0f) : 1.0f;
  const uint32_t vsh = (BITS == 2) ? uint32_t(4 * u) : uint32_t(8 * (u % 2));
  const u32x4 ones = u32x4{0x3F803F80u, 0x3F803F80u, 0x3F803F80u, 0x3F803F80u};

  float m_ref = -INFINITY;
  float l_acc = 0.0f, pz_acc = 0.0f;
  f32x4 cv[8];
#pragma unroll
  for (int n = 0; n < 8; ++n) cv[n] = f32x4{0.f, 0.f, 0.f, 0.f};
  f32x4 cones = f32x4{0.f, 0.f, 0.f, 0.f};

  const int64_t n_groups = a.n_main / kGroup;
  const int64_t g0 = int64_t(split) * a.tiles_per_split;
  const int64_t g1 = min(g0 + int64_t(a.tiles_per_split), n_groups);
  const uint32_t* kcodes = static_cast<const uint32_t*>(a.k_main);
  const uint32_t* vcodes = static_cast<const uint32_t*>(a.v_main);

  for (int64_t g = g0 + wave; g < g1; g += kWaves) {
    // ---------------------------------------------------------------- loads
    uint32_t kw[2][LW];
#pragma unroll
    for (int tile = 0; tile < 2; ++tile) {
      const uint32_t* row = kcodes + (int64_t(bh) * CT + g * kGroup + 16 * tile + r) * KW + LW * u;
      if (BITS == 2) {
        const uint2 x = *reinterpret_cast<const uint2*>(row);
        kw[tile][0] = x.x;
        kw[tile][1] = x.y;
      } else {
        const uint4 x = *reinterpret_cast<const uint4*>(row);
        kw[tile][0] = x.x;
        kw[tile][1] = x.y;
        kw[tile][2] = x.z;
        kw[tile][3] = x.w;
      }
    }
    const float* ksp = a.k_scale + (int64_t(bh) * a.NG + g) * kHeadDim + 32 * u;
    const float* kzp = a.k_zero + (int64_t(bh) * a.NG + g) * kHeadDim + 32 * u + 16 * (low ? 1 : 0);
    float ks[32], kz[16];
#pragma unroll
    for (int c = 0; c < 32; c += 4) {
      const float4 x = *reinterpret_cast<const float4*>(ksp + c);
      ks[c] = x.x; ks[c + 1] = x.y; ks[c + 2] = x.z; ks[c + 3] = x.w;
    }
#pragma unroll
    for (int c = 0; c < 16; c += 4) {
      const float4 x = *reinterpret_cast<const float4*>(kzp + c);
      kz[c] = x.x; kz[c + 1] = x.y; kz[c + 2] = x.z; kz[c + 3] = x.w;
    }
    uint32_t vw[8][2];
#pragma unroll
    for (int n = 0; n < 8; ++n) {
      const uint32_t* cw = vcodes + ((int64_t(bh) * a.NG + g) * kHeadDim + 16 * n + r) * VW;
      if (BITS == 2) {
        const uint2 x = *reinterpret_cast<const uint2*>(cw);
        vw[n][0] = x.x;
        vw[n][1] = x.y;
      } else {
        vw[n][0] = cw[u / 2];
        vw[n][1] = cw[2 + u / 2];
      }
    }
    const int64_t tok0 = int64_t(bh) * CT + g * kGroup + 16 * (low ? 1 : 0) + 4 * u;
    const float4 vs4 = *reinterpret_cast<const float4*>(a.v_scale + tok0);
    const float4 vz4 = *reinterpret_cast<const float4*>(a.v_zero + tok0);

    // --------------------------------------------------------- scores (QK)
    u32x4 bq[4];
#pragma unroll
    for (int sl = 0; sl < 4; ++sl) {
      uint32_t d[4];
#pragma unroll
      for (int p = 0; p < 4; ++p) {
        const int j0 = 2 * p, j1 = 2 * p + 1;
        const float x0 = qf[sl][j0] * ks[k_channel<BITS>(sl, j0)];
        const float x1 = qf[sl][j1] * ks[k_channel<BITS>(sl, j1)];
        d[p] = split_f16(x0, low) | (split_f16(x1, low) << 16);
      }
      bq[sl] = u32x4{d[0], d[1], d[2], d[3]};
    }
    float zt = 0.0f;
#pragma unroll
    for (int c = 0; c < 16; ++c) zt = fmaf(qz[c], kz[c], zt);
    zt = head_sum(zt);                          // Σ_d q_d·z[g,d] for head hs
    const float c0 = low ? 0.0f : zt * kTwoM24;
    f32x4 s0 = f32x4{c0, c0, c0, c0}, s1 = s0;
    {
      u32x4 A0[4], A1[4];
      k_unpack<BITS>(kw[0], A0);
      k_unpack<BITS>(kw[1], A1);
#pragma unroll
      for (int sl = 0; sl < 4; ++sl) {
        s0 = __builtin_amdgcn_mfma_f32_16x16x32_f16(as_f16x8(A0[sl]), as_f16x8(bq[sl]), s0, 0, 0, 0);
        s1 = __builtin_amdgcn_mfma_f32_16x16x32_f16(as_f16x8(A1[sl]), as_f16x8(bq[sl]), s1, 0, 0, 0);
      }
    }
    // high + low parts: lane keeps tile `low` (tokens 16·low + 4u + i)
    float sc[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float send = low ? s0[i] : s1[i];
      const float mine = low ? s1[i] : s0[i];
      sc[i] = (mine + xor8(send)) * kTwo24;
    }

    // ------------------------------------------------------ online softmax
    float lmax = fmaxf(fmaxf(sc[0], sc[1]), fmaxf(sc[2], sc[3]));
    if (__any(lmax > m_ref + kLazy)) {          // wave-uniform slow path
      const float gm = head_max(lmax);
      const float m_new = fmaxf(m_ref, gm);
      const float alpha = exp2f(m_ref - m_new);
      l_acc *= alpha;
      pz_acc *= alpha;
#pragma unroll
      for (int n = 0; n < 8; ++n) cv[n] *= alpha;
      cones *= alpha;
      m_ref = m_new;
    }
    float pp[4];
    const float vsa[4] = {vs4.x, vs4.y, vs4.z, vs4.w};
    const float vza[4] = {vz4.x, vz4.y, vz4.z, vz4.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float p = exp2f(sc[i] - m_ref);
      l_acc += p;
      pz_acc = fmaf(p, vza[i], pz_acc);
      pp[i] = p * vsa[i] * vfac[i];
    }
    // bf16 high / low terms of P' (truncation split), exchanged with lane ^ 8
    uint32_t keep[2], send[2];
#pragma unroll
    for (int p = 0; p < 2; ++p) {
      uint32_t hb[2], lb[2];
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        const uint32_t xb = __float_as_uint(pp[2 * p + e]);
        hb[e] = xb & 0xFFFF0000u;
        lb[e] = __float_as_uint(pp[2 * p + e] - __uint_as_float(hb[e])) & 0xFFFF0000u;
      }
      const uint32_t hpair = (hb[0] >> 16) | hb[1];
      const uint32_t lpair = (lb[0] >> 16) | lb[1];
      keep[p] = low ? lpair : hpair;
      send[p] = low ? hpair : lpair;
    }
    const uint32_t recv0 = xor8u(send[0]), recv1 = xor8u(send[1]);
    // k-slots 0..3: tile 0 tokens 4u..4u+3; k-slots 4..7: tile 1 tokens
    const u32x4 bp = low ? u32x4{recv0, recv1, keep[0], keep[1]}
                         : u32x4{keep[0], keep[1], recv0, recv1};

    // ------------------------------------------------------------ P·V
#pragma unroll
    for (int n = 0; n < 8; ++n) {
      uint32_t d[4];
      if (BITS == 2) {
        const uint32_t w0 = vw[n][0] >> vsh, w1 = vw[n][1] >> vsh;
        d[0] = (w0 & 0x00030003u) | 0x43004300u;
        d[1] = (w0 & 0x000C000Cu) | 0x43004300u;
        d[2] = (w1 & 0x00030003u) | 0x43004300u;
        d[3] = (w1 & 0x000C000Cu) | 0x43004300u;
      } else {
        d[0] = ((vw[n][0] >> vsh) & 0x000F000Fu) | 0x43004300u;
        d[1] = ((vw[n][0] >> (vsh + 4)) & 0x000F000Fu) | 0x43004300u;
        d[2] = ((vw[n][1] >> vsh) & 0x000F000Fu) | 0x43004300u;
        d[3] = ((vw[n][1] >> (vsh + 4)) & 0x000F000Fu) | 0x43004300u;
      }
      cv[n] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(u32x4{d[0], d[1], d[2], d[3]}),
                                                       as_bf16x8(bp), cv[n], 0, 0, 0);
    }
    cones = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(ones), as_bf16x8(bp), cones, 0, 0, 0);
  }

  // ---- wave epilogue: head totals, offset removal, high + low columns
  const float l_tot = head_sum(l_acc);
  const float pz_tot = head_sum(pz_acc);
  const float off = 128.0f * (cones[0] + xor8(cones[0]));
#pragma unroll
  for (int n = 0; n < 8; ++n) {
    f32x4 o;
#pragma unroll
    for (int i = 0; i < 4; ++i) o[i] = cv[n][i] + xor8(cv[n][i]) - off + pz_tot;
    if (!low) *reinterpret_cast<f32x4*>(&mo[wave][hs][16 * n + 4 * u]) = o;
  }
  if (lane < 8) {
    ml[wave][hs][0] = m_ref;
    ml[wave][hs][1] = l_tot;
  }
  __syncthreads();

  // ---- merge the four wave states, write this split's partials
  for (int i = tid; i < nh * kHeadDim; i += kThreads) {
    const int h = i / kHeadDim;
    const int d = i % kHeadDim;
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) M = fmaxf(M, ml[w][h][0]);
    float O = 0.0f, L = 0.0f;
    if (M != -INFINITY) {
#pragma unroll
      for (int w = 0; w < kWaves; ++w) {
        const float mw = ml[w][h][0];
        const float f = mw == -INFINITY ? 0.0f : exp2f(mw - M);
        O = fmaf(f, mo[w][h][d], O);
        L = fmaf(f, ml[w][h][1], L);
      }
    }
    float* part = a.ws + ((int64_t(b) * a.Hq + hq0 + h) * a.n_split + split) * kPart;
    part[d] = O;
    if (d == 0) {
      part[kHeadDim] = M;
      part[kHeadDim + 1] = L;
    }
  }
}

}  // namespace

hipError_t launch_kivi_mfma(const DecodeArgs& a, hipStream_t s) {
  if (a.n_split_main <= 0) return hipSuccess;
  const dim3 grid(a.n_split_main, a.B * a.H, a.nq / a.heads_per_chunk);
  if (a.src == kSrcKivi2) {
    kivi_mfma_split_kernel<2><<<grid, kThreads, 0, s>>>(a);
  } else {
    kivi_mfma_split_kernel<4><<<grid, kThreads, 0, s>>>(a);
  }
  return hipGetLastError();
}

}  // namespace kvq
