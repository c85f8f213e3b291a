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
//   A = K codes of token 16·tile + r as exact small fp16 integers, made by the
//       gfx950 scaled conversions (2-bit codes as fp4 E2M1 nibbles c/2 scaled
//       by 2, 4-bit codes as fp8 E4M3 bytes c·2⁻⁹ scaled by 2⁹), B = Q' for
//       column r: head hs, the fp16 high (part 0) or low (part 1) term of
//       q_d·s[g,d]·log2(e)/√D. C starts at the head's z-term Σ_d q_d·z[g,d].
//       The two parts of a head sit in columns hs and hs+8 of the same lane
//       row; a DPP rotate adds them. The operands are normal fp16 numbers on
//       purpose: the matrix core aligns the 32 products of a k-step to the
//       largest product built from the operands' exponent fields, so a
//       subnormal operand (exponent field 0, read as 2⁻¹⁴) would cost up to
//       ten bits of the sum's precision.
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

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ f16x8 as_f16x8(u32x4 v) { return __builtin_bit_cast(f16x8, v); }
__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

__device__ __forceinline__ void wave_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

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

// {f16(a0·b0), f16(a1·b1)}: fp32 products rounded once to fp16, packed.
__device__ __forceinline__ uint32_t mix_pair(float a0, float b0, float a1, float b1) {
  uint32_t d;
  asm("v_fma_mixlo_f16 %0, %1, %2, 0 op_sel_hi:[0,0,0]" : "=v"(d) : "v"(a0), "v"(b0));
  asm("v_fma_mixhi_f16 %0, %1, %2, 0 op_sel_hi:[0,0,0]" : "+v"(d) : "v"(a1), "v"(b1));
  return d;
}
// {f16(a0·b0 − c.lo), f16(a1·b1 − c.hi)} with c an fp16 pair; each term is a
// fused fp32 multiply-subtract rounded once to fp16.
__device__ __forceinline__ uint32_t mix_pair_sub(float a0, float b0, float a1, float b1,
                                                 uint32_t c) {
  uint32_t d;
  asm("v_fma_mixlo_f16 %0, %1, %2, -%3 op_sel_hi:[0,0,1]" : "=v"(d) : "v"(a0), "v"(b0), "v"(c));
  asm("v_fma_mixhi_f16 %0, %1, %2, -%3 op_sel:[0,0,1] op_sel_hi:[0,0,1]"
      : "+v"(d) : "v"(a1), "v"(b1), "v"(c));
  return d;
}
// (mask & x) | (~mask & y) in one instruction
__device__ __forceinline__ uint32_t bfi(uint32_t mask, uint32_t x, uint32_t y) {
  uint32_t d;
  asm("v_bfi_b32 %0, %1, %2, %3" : "=v"(d) : "v"(mask), "v"(x), "v"(y));
  return d;
}

// ---- K code positions. The conversions turn one byte (two fp4 nibbles) or
// one half-word (two fp8 bytes) into an fp16 pair, so in k-step sl the k-slots
// j = 0..7 of a lane whose 32 channels start at 32·u hold channels
// 8·sl + {0, 2, 1, 3, 4, 6, 5, 7}[j] (for both widths):
//   2-bit: word sl/2; m0 = w & 0x33333333 has code 2n in nibble n, m1 =
//          (w >> 2) & 0x33333333 code 2n+1; byte k of m0 / m1 gives codes
//          {4k, 4k+2} / {4k+1, 4k+3}; k-step sl uses bytes 2·(sl%2) + {0, 1}.
//   4-bit: word sl; m0 = w & 0x0F0F0F0F has code 2n in byte n, m1 =
//          (w >> 4) & 0x0F0F0F0F code 2n+1; half-word 0 / 1 of m0 gives codes
//          {0, 2} / {4, 6}, of m1 {1, 3} / {5, 7}.
__device__ __forceinline__ constexpr int k_channel(int sl, int j) {
  return 8 * sl + 4 * (j / 4) + (j / 2) % 2 + 2 * (j % 2);
}

__device__ __forceinline__ uint32_t fp4x2_to_f16x2(uint32_t w, int byte) {
  typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
  f16x2 r;
  switch (byte) {  // the byte select is an immediate
    case 0: r = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 2.0f, 0); break;
    case 1: r = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 2.0f, 1); break;
    case 2: r = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 2.0f, 2); break;
    default: r = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 2.0f, 3); break;
  }
  return __builtin_bit_cast(uint32_t, r);
}
__device__ __forceinline__ uint32_t fp8x2_to_f16x2(uint32_t w, bool high) {
  typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
  const f16x2 r = high ? __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 512.0f, true)
                       : __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 512.0f, false);
  return __builtin_bit_cast(uint32_t, r);
}

// A operand of one token: 4 k-steps × 4 dwords of fp16 code pairs.
template <int BITS>
__device__ __forceinline__ void k_unpack(const uint32_t* w, u32x4* A) {
  if (BITS == 2) {
#pragma unroll
    for (int x = 0; x < 2; ++x) {
      const uint32_t m0 = w[x] & 0x33333333u, m1 = (w[x] >> 2) & 0x33333333u;
#pragma unroll
      for (int h = 0; h < 2; ++h)
        A[2 * x + h] = u32x4{fp4x2_to_f16x2(m0, 2 * h), fp4x2_to_f16x2(m1, 2 * h),
                             fp4x2_to_f16x2(m0, 2 * h + 1), fp4x2_to_f16x2(m1, 2 * h + 1)};
    }
  } else {
#pragma unroll
    for (int x = 0; x < 4; ++x) {
      const uint32_t m0 = w[x] & 0x0F0F0F0Fu, m1 = (w[x] >> 4) & 0x0F0F0F0Fu;
      A[x] = u32x4{fp8x2_to_f16x2(m0, false), fp8x2_to_f16x2(m1, false),
                   fp8x2_to_f16x2(m0, true), fp8x2_to_f16x2(m1, true)};
    }
  }
}

// Raw data of one group for one lane (loaded one group ahead).
template <int BITS>
struct GroupRegs {
  uint32_t kw[2][BITS];        // K words of tokens r and 16 + r (32 channels)
  float4 ksz;                  // 16-byte chunk of the group's K scale | zero block
  uint32_t vw[8][2];           // V words (tile-0 and tile-1 tokens) of channel 16n + r
  float vs[4], vz[4];          // V scale / zero of tokens 16·part + 4u + i
};

template <int BITS>
__device__ __forceinline__ void load_group(GroupRegs<BITS>& G, const DecodeArgs& a, int bh,
                                           int64_t g, int lane, int r, int u, bool low) {
  constexpr int KW = kHeadDim * BITS / 32;
  constexpr int VW = kGroup * BITS / 32;
  const int64_t CT = a.main_bh_tokens;
  const uint32_t* kcodes = static_cast<const uint32_t*>(a.k_main);
  const uint32_t* vcodes = static_cast<const uint32_t*>(a.v_main);
#pragma unroll
  for (int tile = 0; tile < 2; ++tile) {
    const uint32_t* row = kcodes + (int64_t(bh) * CT + g * kGroup + 16 * tile + r) * KW + BITS * u;
    if (BITS == 2) {
      const uint2 x = *reinterpret_cast<const uint2*>(row);
      G.kw[tile][0] = x.x;
      G.kw[tile][1] = x.y;
    } else {
      const uint4 x = *reinterpret_cast<const uint4*>(row);
      G.kw[tile][0] = x.x;
      G.kw[tile][1] = x.y;
      G.kw[tile][2] = x.z;
      G.kw[tile][3] = x.w;
    }
  }
  // lanes 0..31: scales 4l..4l+3; lanes 32..63: zero-points
  const float* meta = (lane < 32 ? a.k_scale : a.k_zero) + (int64_t(bh) * a.NG + g) * kHeadDim;
  G.ksz = *reinterpret_cast<const float4*>(meta + 4 * (lane & 31));
#pragma unroll
  for (int n = 0; n < 8; ++n) {
    const uint32_t* cw = vcodes + ((int64_t(bh) * a.NG + g) * kHeadDim + 16 * n + r) * VW;
    if (BITS == 2) {
      const uint2 x = *reinterpret_cast<const uint2*>(cw);
      G.vw[n][0] = x.x;
      G.vw[n][1] = x.y;
    } else {
      G.vw[n][0] = cw[u / 2];
      G.vw[n][1] = cw[2 + u / 2];
    }
  }
  const int64_t tok0 = int64_t(bh) * CT + g * kGroup + (low ? 16 : 0) + 4 * u;
  const float4 s4 = *reinterpret_cast<const float4*>(a.v_scale + tok0);
  const float4 z4 = *reinterpret_cast<const float4*>(a.v_zero + tok0);
  G.vs[0] = s4.x; G.vs[1] = s4.y; G.vs[2] = s4.z; G.vs[3] = s4.w;
  G.vz[0] = z4.x; G.vz[1] = z4.y; G.vz[2] = z4.z; G.vz[3] = z4.w;
}

// Per-lane state of one wavefront across its groups.
struct WaveAcc {
  float m_ref, l_acc, pz_acc;
  f32x4 cv[8];
  f32x4 cones;
};

template <int BITS>
__device__ __forceinline__ void process_group(const GroupRegs<BITS>& G, WaveAcc& W,
                                              float* ksz_lds, int lane, int u,
                                              const float (&qf)[4][8], const float (&qz)[16],
                                              uint32_t selmask, bool low, uint32_t vsh,
                                              uint32_t vm0, uint32_t vm1, uint32_t magic) {
  // ---- stage the group's K scales (ksz_lds[0..127]) and zero-points
  // (ksz_lds[128..255]) in this wavefront's LDS slot
  wave_sync();
  *reinterpret_cast<float4*>(ksz_lds + 4 * lane) = G.ksz;
  wave_sync();
  const float* ks = ksz_lds + 32 * u;
  const float* kz = ksz_lds + 128 + 32 * u + (low ? 16 : 0);
  // ---- z-term Σ_d q_d·z[g, d] of head hs (8 lanes × 16 channels)
  float zt = 0.0f;
#pragma unroll
  for (int c = 0; c < 16; ++c) zt = fmaf(qz[c], kz[c], zt);
  zt = head_sum(zt);
  const float c0 = low ? 0.0f : zt;
  f32x4 s0 = f32x4{c0, c0, c0, c0}, s1 = s0;
  // ---- scores, one k-step (32 channels) at a time
  u32x4 A0[4], A1[4];
  k_unpack<BITS>(G.kw[0], A0);
  k_unpack<BITS>(G.kw[1], A1);
#pragma unroll
  for (int sl = 0; sl < 4; ++sl) {
    uint32_t d[4];
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      const int j0 = 2 * p, j1 = 2 * p + 1;
      const float a0 = qf[sl][j0], b0 = ks[k_channel(sl, j0)];
      const float a1 = qf[sl][j1], b1 = ks[k_channel(sl, j1)];
      const uint32_t hi = mix_pair(a0, b0, a1, b1);
      d[p] = mix_pair_sub(a0, b0, a1, b1, hi & selmask);
    }
    const u32x4 bq = u32x4{d[0], d[1], d[2], d[3]};
    s0 = __builtin_amdgcn_mfma_f32_16x16x32_f16(as_f16x8(A0[sl]), as_f16x8(bq), s0, 0, 0, 0);
    s1 = __builtin_amdgcn_mfma_f32_16x16x32_f16(as_f16x8(A1[sl]), as_f16x8(bq), s1, 0, 0, 0);
  }
  // ---- both parts of the head's score; this lane keeps tile `low`
  float sc[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float send = low ? s0[i] : s1[i];
    const float mine = low ? s1[i] : s0[i];
    sc[i] = mine + xor8(send);
  }
  // ---- online softmax (log2 domain)
  const float lmax = fmaxf(fmaxf(sc[0], sc[1]), fmaxf(sc[2], sc[3]));
  if (__any(lmax > W.m_ref + kLazy)) {           // wave-uniform, rare
    const float m_new = fmaxf(W.m_ref, head_max(lmax));
    const float alpha = exp2f(W.m_ref - m_new);
    W.l_acc *= alpha;
    W.pz_acc *= alpha;
#pragma unroll
    for (int n = 0; n < 8; ++n) W.cv[n] *= alpha;
    W.cones *= alpha;
    W.m_ref = m_new;
  }
  float pp[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float p = exp2f(sc[i] - W.m_ref);
    W.l_acc += p;
    W.pz_acc = fmaf(p, G.vz[i], W.pz_acc);
    pp[i] = p * ((BITS == 2 && i >= 2) ? G.vs[i] * 0.25f : G.vs[i]);
  }
  // ---- bf16 high / low terms of P' (truncation split), exchanged with lane ^ 8
  uint32_t keep[2], send[2];
#pragma unroll
  for (int p = 0; p < 2; ++p) {
    const float x0 = pp[2 * p], x1 = pp[2 * p + 1];
    const float l0 = x0 - __uint_as_float(__float_as_uint(x0) & 0xFFFF0000u);
    const float l1 = x1 - __uint_as_float(__float_as_uint(x1) & 0xFFFF0000u);
    const uint32_t hpair = __builtin_amdgcn_perm(__float_as_uint(x1), __float_as_uint(x0), 0x07060302u);
    const uint32_t lpair = __builtin_amdgcn_perm(__float_as_uint(l1), __float_as_uint(l0), 0x07060302u);
    keep[p] = low ? lpair : hpair;
    send[p] = low ? hpair : lpair;
  }
  const uint32_t recv0 = xor8u(send[0]), recv1 = xor8u(send[1]);
  const u32x4 bp = low ? u32x4{recv0, recv1, keep[0], keep[1]}
                       : u32x4{keep[0], keep[1], recv0, recv1};
  // ---- P·V: 8 tiles of 16 channels, codes in the mantissa of 128.0
#pragma unroll
  for (int n = 0; n < 8; ++n) {
    uint32_t d[4];
    if (BITS == 2) {
      const uint32_t w0 = G.vw[n][0] >> vsh, w1 = G.vw[n][1] >> vsh;
      d[0] = bfi(vm0, w0, magic);
      d[1] = bfi(vm1, w0, magic);
      d[2] = bfi(vm0, w1, magic);
      d[3] = bfi(vm1, w1, magic);
    } else {
      d[0] = bfi(vm0, G.vw[n][0] >> vsh, magic);
      d[1] = bfi(vm0, G.vw[n][0] >> (vsh + 4), magic);
      d[2] = bfi(vm0, G.vw[n][1] >> vsh, magic);
      d[3] = bfi(vm0, G.vw[n][1] >> (vsh + 4), magic);
    }
    W.cv[n] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(u32x4{d[0], d[1], d[2], d[3]}),
                                                       as_bf16x8(bp), W.cv[n], 0, 0, 0);
  }
  const u32x4 ones = u32x4{0x3F803F80u, 0x3F803F80u, 0x3F803F80u, 0x3F803F80u};
  W.cones = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(ones), as_bf16x8(bp), W.cones,
                                                    0, 0, 0);
}


// One 32-token tile of the FP16 window ("4.4 KV Cache 量化：KIVI 2-bit 与 FP8
// KV Cache", §3.2: the newest tokens stay unquantized). Scores: A = K values
// (fp16, exact), B = fp16 high/low terms of q·log2e/√D (channels 32s + 8u + j
// in k-step s). Values: V enters as two exact bf16 terms (fp16 has 11
// significant bits, a bf16 pair holds 16), P' = p as a bf16 high/low pair.
// Tokens past n_win are masked (score −∞, value 0).
__device__ __forceinline__ void process_window_tile(const DecodeArgs& a, WaveAcc& W, int bh,
                                                    int64_t tile, const u32x4 (&bqw)[4],
                                                    int r, int u, bool low) {
  const __half* kw = a.k_win + (int64_t(bh) * a.win_cap + tile * kGroup) * kHeadDim;
  const __half* vwp = a.v_win + (int64_t(bh) * a.win_cap + tile * kGroup) * kHeadDim;
  const int n_in = int(min<int64_t>(kGroup, a.n_win - tile * kGroup));
  f32x4 s0 = f32x4{0.f, 0.f, 0.f, 0.f}, s1 = s0;
#pragma unroll
  for (int sl = 0; sl < 4; ++sl) {
    const uint4 k0 = *reinterpret_cast<const uint4*>(kw + r * kHeadDim + 32 * sl + 8 * u);
    const uint4 k1 = *reinterpret_cast<const uint4*>(kw + (16 + r) * kHeadDim + 32 * sl + 8 * u);
    s0 = __builtin_amdgcn_mfma_f32_16x16x32_f16(as_f16x8(u32x4{k0.x, k0.y, k0.z, k0.w}),
                                                as_f16x8(bqw[sl]), s0, 0, 0, 0);
    s1 = __builtin_amdgcn_mfma_f32_16x16x32_f16(as_f16x8(u32x4{k1.x, k1.y, k1.z, k1.w}),
                                                as_f16x8(bqw[sl]), s1, 0, 0, 0);
  }
  float sc[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    // the cross-lane add runs in every lane (its partner may hold a masked
    // token); the mask is applied afterwards
    const float send = low ? s0[i] : s1[i];
    const float mine = low ? s1[i] : s0[i];
    const float both = mine + xor8(send);
    const int t = (low ? 16 : 0) + 4 * u + i;
    sc[i] = t < n_in ? both : -INFINITY;
  }
  const float lmax = fmaxf(fmaxf(sc[0], sc[1]), fmaxf(sc[2], sc[3]));
  if (__any(lmax > W.m_ref + kLazy)) {
    const float m_new = fmaxf(W.m_ref, head_max(lmax));
    const float alpha = exp2f(W.m_ref - m_new);
    W.l_acc *= alpha;
    W.pz_acc *= alpha;
#pragma unroll
    for (int n = 0; n < 8; ++n) W.cv[n] *= alpha;
    W.cones *= alpha;
    W.m_ref = m_new;
  }
  float pp[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    pp[i] = exp2f(sc[i] - W.m_ref);          // 0 for masked tokens
    W.l_acc += pp[i];
  }
  uint32_t keep[2], send[2];
#pragma unroll
  for (int p = 0; p < 2; ++p) {
    const float x0 = pp[2 * p], x1 = pp[2 * p + 1];
    const float l0 = x0 - __uint_as_float(__float_as_uint(x0) & 0xFFFF0000u);
    const float l1 = x1 - __uint_as_float(__float_as_uint(x1) & 0xFFFF0000u);
    const uint32_t hpair = __builtin_amdgcn_perm(__float_as_uint(x1), __float_as_uint(x0), 0x07060302u);
    const uint32_t lpair = __builtin_amdgcn_perm(__float_as_uint(l1), __float_as_uint(l0), 0x07060302u);
    keep[p] = low ? lpair : hpair;
    send[p] = low ? hpair : lpair;
  }
  const uint32_t recv0 = xor8u(send[0]), recv1 = xor8u(send[1]);
  const u32x4 bp = low ? u32x4{recv0, recv1, keep[0], keep[1]}
                       : u32x4{keep[0], keep[1], recv0, recv1};
  // V^T tiles: lane (r, u) needs channel 16n + r at tokens 4u + j (j < 4) and
  // 16 + 4u + j - 4; masked tokens read as 0.
#pragma unroll
  for (int n = 0; n < 8; ++n) {
    float v[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int t = (j < 4) ? 4 * u + j : 16 + 4 * u + (j - 4);
      v[j] = t < n_in ? __half2float(vwp[t * kHeadDim + 16 * n + r]) : 0.0f;
    }
    uint32_t hi[4], lo[4];
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      const float x0 = v[2 * p], x1 = v[2 * p + 1];
      const float l0 = x0 - __uint_as_float(__float_as_uint(x0) & 0xFFFF0000u);
      const float l1 = x1 - __uint_as_float(__float_as_uint(x1) & 0xFFFF0000u);
      hi[p] = __builtin_amdgcn_perm(__float_as_uint(x1), __float_as_uint(x0), 0x07060302u);
      lo[p] = __builtin_amdgcn_perm(__float_as_uint(l1), __float_as_uint(l0), 0x07060302u);
    }
    W.cv[n] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(u32x4{hi[0], hi[1], hi[2], hi[3]}),
                                                       as_bf16x8(bp), W.cv[n], 0, 0, 0);
    W.cv[n] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(u32x4{lo[0], lo[1], lo[2], lo[3]}),
                                                       as_bf16x8(bp), W.cv[n], 0, 0, 0);
  }
}

template <int BITS>
__global__ __launch_bounds__(kThreads) void kivi_mfma_split_kernel(DecodeArgs a) {
  __shared__ float mo[kWaves][8][kHeadDim];
  __shared__ float ml[kWaves][8][2];
  __shared__ float ksz_slot[kWaves][2 * kHeadDim];

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

  // ---- per-lane constants: this lane's 32 channels [32u, 32u+32) of head hs
  float qf[4][8];          // q_d·log2e/√D, by (k-step, k-slot)
  float qz[16];            // q_d·log2e/√D for the z-term: channels 32u + 16·part + c
  {
    const bool valid = hs < nh;
    const float* qrow = a.q + (int64_t(b) * a.Hq + hq0 + (valid ? hs : 0)) * kHeadDim + 32 * u;
#pragma unroll
    for (int sl = 0; sl < 4; ++sl)
#pragma unroll
      for (int j = 0; j < 8; ++j)
        qf[sl][j] = valid ? qrow[k_channel(sl, j)] * a.qscale : 0.0f;
#pragma unroll
    for (int c = 0; c < 16; ++c) qz[c] = valid ? qrow[(low ? 16 : 0) + c] * a.qscale : 0.0f;
  }
  const uint32_t selmask = low ? 0xFFFFFFFFu : 0u;
  const uint32_t vsh = (BITS == 2) ? uint32_t(4 * u) : uint32_t(8 * (u % 2));
  const uint32_t vm0 = (BITS == 2) ? 0x00030003u : 0x000F000Fu;
  const uint32_t vm1 = 0x000C000Cu;
  const uint32_t magic = 0x43004300u;

  WaveAcc W;
  W.m_ref = -INFINITY;
  W.l_acc = 0.0f;
  W.pz_acc = 0.0f;
#pragma unroll
  for (int n = 0; n < 8; ++n) W.cv[n] = f32x4{0.f, 0.f, 0.f, 0.f};
  W.cones = f32x4{0.f, 0.f, 0.f, 0.f};

  if (split < a.n_split_main) {
    const int64_t n_groups = a.n_main / kGroup;
    const int64_t g0 = int64_t(split) * a.tiles_per_split;
    const int64_t g1 = min(g0 + int64_t(a.tiles_per_split), n_groups);
    // groups g0 + wave, g0 + wave + 4, ...; the next one is loaded while the
    // current one is processed (index clamped to the range, so the load is
    // always issued and always in bounds)
    int64_t g = g0 + wave;
    if (g < g1) {
      GroupRegs<BITS> A, B;
      float* slot = ksz_slot[wave];
      load_group<BITS>(A, a, bh, g, lane, r, u, low);
      while (true) {
        load_group<BITS>(B, a, bh, min(g + kWaves, g1 - 1), lane, r, u, low);
        process_group<BITS>(A, W, slot, lane, u, qf, qz, selmask, low, vsh, vm0, vm1, magic);
        g += kWaves;
        if (g >= g1) break;
        load_group<BITS>(A, a, bh, min(g + kWaves, g1 - 1), lane, r, u, low);
        process_group<BITS>(B, W, slot, lane, u, qf, qz, selmask, low, vsh, vm0, vm1, magic);
        g += kWaves;
        if (g >= g1) break;
      }
    }
  } else {
    // the FP16 window: q·log2e/√D as fp16 high/low terms, channel 32s + 8u + j
    u32x4 bqw[4];
    {
      const bool valid = hs < nh;
      const float* qrow = a.q + (int64_t(b) * a.Hq + hq0 + (valid ? hs : 0)) * kHeadDim;
#pragma unroll
      for (int sl = 0; sl < 4; ++sl) {
        uint32_t d[4];
#pragma unroll
        for (int p = 0; p < 4; ++p) {
          const float x0 = valid ? qrow[32 * sl + 8 * u + 2 * p] * a.qscale : 0.0f;
          const float x1 = valid ? qrow[32 * sl + 8 * u + 2 * p + 1] * a.qscale : 0.0f;
          const uint32_t hi = mix_pair(x0, 1.0f, x1, 1.0f);
          d[p] = mix_pair_sub(x0, 1.0f, x1, 1.0f, hi & selmask);
        }
        bqw[sl] = u32x4{d[0], d[1], d[2], d[3]};
      }
    }
    const int64_t n_tiles = (a.n_win + kGroup - 1) / kGroup;
    for (int64_t tile = wave; tile < n_tiles; tile += kWaves)
      process_window_tile(a, W, bh, tile, bqw, r, u, low);
  }

  // ---- wave epilogue: head totals, offset removal, high + low columns
  const float l_tot = head_sum(W.l_acc);
  const float pz_tot = head_sum(W.pz_acc);
  const float off = 128.0f * (W.cones[0] + xor8(W.cones[0]));
#pragma unroll
  for (int n = 0; n < 8; ++n) {
    f32x4 o;
#pragma unroll
    for (int i = 0; i < 4; ++i) o[i] = W.cv[n][i] + xor8(W.cv[n][i]) - off + pz_tot;
    if (!low) *reinterpret_cast<f32x4*>(&mo[wave][hs][16 * n + 4 * u]) = o;
  }
  if (lane < 8) {
    ml[wave][hs][0] = W.m_ref;
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
  const dim3 grid(a.n_split, a.B * a.H, a.nq / a.heads_per_chunk);
  if (a.src == kSrcKivi2) {
    kivi_mfma_split_kernel<2><<<grid, kThreads, 0, s>>>(a);
  } else {
    kivi_mfma_split_kernel<4><<<grid, kThreads, 0, s>>>(a);
  }
  return hipGetLastError();
}

}  // namespace kvq
