// kvq_decode_mfma.hip — decode attention over the KIVI grouped region on the
// gfx950 matrix cores (MFMA 16x16x32), fed by asynchronous global→LDS loads.
//
// Attention as in "大模型量化从0到1（十三）：KV Cache 量化", §二 (score = q·k̂/√D,
// softmax, Σ p·v̂), over KIVI groups ("4.4 KV Cache 量化：KIVI 2-bit 与 FP8 KV
// Cache", §3.2: K per channel, V per token, groups of 32 tokens). The
// dequantization is folded so that the codes enter the matrix cores as exact
// small integers:
//   q·k̂_t = Σ_d (q_d·s[g,d])·c[t,d] + Σ_d q_d·z[g,d]          (K per channel)
//   Σ_t p_t·v̂_t[d] = Σ_t (p_t·s_t)·c[t,d] + Σ_t p_t·z_t         (V per token)
//
// Data movement. Each wavefront owns a ring of LDS stages, one 32-token group
// per stage (K codes, V codes, K scale | zero, V scale | zero: 3328 bytes at
// 2 bits, 5376 at 4 bits), filled by global_load_lds (one instruction moves
// 1 KiB, no VGPRs involved) one or two groups ahead of the group in work.
// Work is split over (b, h, head chunk) blocks and, within one, over splits of
// its 32-token tiles; the wavefronts of a split's workgroup take its tiles
// from a shared LDS counter (unit-sized workgroups) or in a fixed order.
//
// One wavefront processes one group at a time; lane l has r = l%16, u = l/16,
// head slot hs = r%8 (up to 8 query heads of one KV head) and part = r/8.
// A lane's channels are the 16 channels 32u + 16·part + (0..15).
//
// Scores, Sᵀ[token][col] = Σ_d code[token][d] · Q'[d][col], as f16 MFMA:
//   A = K codes of token 16·tile + r as exact small fp16 integers, made by the
//       gfx950 scaled conversions (2-bit codes as fp4 E2M1 nibbles c/2 scaled
//       by 2, 4-bit codes as fp8 E4M3 bytes c·2⁻⁹ scaled by 2⁹). The operands
//       are normal fp16 numbers on purpose: the matrix core aligns the 32
//       products of a k-step to the largest product built from the operands'
//       exponent fields, so a subnormal operand (exponent field 0, read as
//       2⁻¹⁴) would cost up to ten bits of the sum's precision.
//   B = Q' for column r: head hs, the fp16 high (part 0) or low (part 1) term
//       of q_d·s[g,d]·log2(e)/√D. Each lane splits the products of its own 16
//       channels into both terms, and a bank-masked DPP swap with lane l ^ 8
//       hands the high terms to part 0 and the low terms to part 1.
//   C starts at the z-term Σ_d q_d·z[g,d] of the lane's half of the channels;
//   adding columns hs and hs+8 (DPP rotate by 8) completes both sums.
// The Sᵀ accumulator layout (lane holds column r, tokens 4u..4u+3 of a tile)
// is exactly the B-operand layout of the value product, so no transpose is
// needed:
//   Oᵀ[d][col] = Σ_t (o_t + code[t][d]) · P'[t][col]   (bf16 MFMA, 8 tiles
//       of 16 channels), with A = codes OR-ed into the mantissa of a bf16
//       power of two o_t whose last mantissa step at the code's bit position
//       is 1 (128.0 for codes in bits 0..1 or 0..3, 32.0 for codes in bits
//       2..3) and B = P' = p_t·s_t as a bf16 high + low split (columns hs,
//       hs+8); Σ_t o_t·P'[t][col] from one more MFMA (A = o_t / 128, then
//       times 128) removes them.
// Online softmax in the log2 domain with a per-head reference maximum that
// is only raised (with rescaling) when a score exceeds it by more than 16;
// after a wavefront's first group the score accumulator starts at −m_ref, so
// the scores come out relative to it.
#include <hip/hip_fp16.h>
#include <hip/hip_runtime.h>

#include <math.h>

#include <atomic>
#include <type_traits>

#include "kvq_fp8.h"
#include "kvq_internal.h"

namespace kvq {
namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / 64;
// ring stages per wavefront (2-bit / 4-bit) and the occupancy the register
// allocation targets (wavefronts per SIMD)
#ifndef KVQ_RING_STAGES_2BIT
#define KVQ_RING_STAGES_2BIT 4
#endif
#ifndef KVQ_RING_STAGES_4BIT
#define KVQ_RING_STAGES_4BIT 3
#endif
#ifndef KVQ_TAKE_AHEAD
#define KVQ_TAKE_AHEAD 1   // take a split's next tile one iteration before it is issued
#endif
#ifndef KVQ_RING_STAGES_UNIT
#define KVQ_RING_STAGES_UNIT 3
#endif
#ifndef KVQ_DECODE_WAVES_PER_SIMD
#define KVQ_DECODE_WAVES_PER_SIMD 3
#endif
constexpr int kPart = kHeadDim + 2;
constexpr float kLazy = 16.0f;                 // log2-domain slack before rescaling

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ f16x8 as_f16x8(u32x4 v) { return __builtin_bit_cast(f16x8, v); }
__device__ __forceinline__ f16x4 as_f16x4(u32x2 v) { return __builtin_bit_cast(f16x4, v); }
__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

// LDS stage of one 32-token tile (byte offsets), K codes at KB bits, V
// codes at VB bits, NVS V scales (and zero-points) per token.
template <int KB, int VB, int NVS = 1>
struct Stage {
  static constexpr int kKBytes = kGroup * kHeadDim * KB / 8;   // K codes
  static constexpr int kVBytes = kGroup * kHeadDim * VB / 8;   // V codes
  static constexpr int kKc = 0;
  static constexpr int kVc = kKBytes;
  static constexpr int kKsz = kKBytes + kVBytes;         // 128 fp32 scales, 128 zero-points
  static constexpr int kVsz = kKsz + 2 * kHeadDim * 4;   // 32·NVS fp32 scales, zero-points
  static constexpr int kBytes = kVsz + 2 * kGroup * 4 * NVS;
  static constexpr int kDepth = (KB == 2 && VB == 2) ? KVQ_RING_STAGES_2BIT : KVQ_RING_STAGES_4BIT;
  static_assert(kDepth >= 3 && kDepth <= 4, "one or two groups in flight ahead");
  static constexpr int kLoads = (kKBytes + kVBytes) / 1024 + 4;   // DMA instructions per tile
  static constexpr int kSecond = kKBytes;   // M0 of the second copy block (V codes on)
  static_assert(kVsz - kSecond < 4096, "copy offsets fit the 12-bit immediate");
};

template <int N>
__device__ __forceinline__ void wait_vmem() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// value of lane l ^ 8 (rotate by 8 inside each row of 16 lanes)
__device__ __forceinline__ float xor8(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x128, 0xF, 0xF, false));
}
// Exchange of high and low terms between partner lanes l and l ^ 8 (part 0:
// lanes with l % 16 < 8): afterwards hi holds {part 0: own hi, part 1:
// partner's lo} and lo holds {part 0: partner's hi, part 1: own lo}. One
// v_cndmask_b32 per register, its first source read from lane l ^ 8 by DPP
// (a masked DPP move pair would need a third instruction to keep a copy).
// The block opens with two wait states (a DPP read of a VGPR that a VALU
// instruction just wrote) and closes with two (a matrix-core operand read of
// a VGPR a VALU instruction just wrote): the compiler pads only around
// instructions it emitted itself. Both masks are set with s_mov, which
// leaves SCC alone: the compiler may hold a branch condition in SCC across
// the block (an SCC-writing s_not here once broke a loop's exit test).
__device__ __forceinline__ void swap_halves2(uint32_t (&hi)[2], uint32_t (&lo)[2]) {
  uint32_t h0, h1, l0, l1;
  asm volatile(
      "s_nop 1\n\t"
      "s_mov_b32 vcc_lo, 0x00ff00ff\n\t"
      "s_mov_b32 vcc_hi, 0x00ff00ff\n\t"
      // vcc = part 0: part 0 keeps its hi (src1), part 1 takes lo of l ^ 8 (src0)
      "v_cndmask_b32_dpp %0, %6, %4, vcc row_ror:8 row_mask:0xf bank_mask:0xf\n\t"
      "v_cndmask_b32_dpp %1, %7, %5, vcc row_ror:8 row_mask:0xf bank_mask:0xf\n\t"
      "s_mov_b32 vcc_lo, 0xff00ff00\n\t"
      "s_mov_b32 vcc_hi, 0xff00ff00\n\t"
      // vcc = part 1: part 1 keeps its lo (src1), part 0 takes hi of l ^ 8 (src0)
      "v_cndmask_b32_dpp %2, %4, %6, vcc row_ror:8 row_mask:0xf bank_mask:0xf\n\t"
      "v_cndmask_b32_dpp %3, %5, %7, vcc row_ror:8 row_mask:0xf bank_mask:0xf\n\t"
      "s_nop 1"
      : "=&v"(h0), "=&v"(h1), "=&v"(l0), "=&v"(l1)
      : "v"(hi[0]), "v"(hi[1]), "v"(lo[0]), "v"(lo[1])
      : "vcc");
  hi[0] = h0; hi[1] = h1; lo[0] = l0; lo[1] = l1;
}
__device__ __forceinline__ void swap_halves4(uint32_t (&hi)[4], uint32_t (&lo)[4]) {
  uint32_t h0, h1, h2, h3, l0, l1, l2, l3;
  asm volatile(
      "s_nop 1\n\t"
      "s_mov_b32 vcc_lo, 0x00ff00ff\n\t"
      "s_mov_b32 vcc_hi, 0x00ff00ff\n\t"
      "v_cndmask_b32_dpp %0, %12, %8, vcc row_ror:8 row_mask:0xf bank_mask:0xf\n\t"
      "v_cndmask_b32_dpp %1, %13, %9, vcc row_ror:8 row_mask:0xf bank_mask:0xf\n\t"
      "v_cndmask_b32_dpp %2, %14, %10, vcc row_ror:8 row_mask:0xf bank_mask:0xf\n\t"
      "v_cndmask_b32_dpp %3, %15, %11, vcc row_ror:8 row_mask:0xf bank_mask:0xf\n\t"
      "s_mov_b32 vcc_lo, 0xff00ff00\n\t"
      "s_mov_b32 vcc_hi, 0xff00ff00\n\t"
      "v_cndmask_b32_dpp %4, %8, %12, vcc row_ror:8 row_mask:0xf bank_mask:0xf\n\t"
      "v_cndmask_b32_dpp %5, %9, %13, vcc row_ror:8 row_mask:0xf bank_mask:0xf\n\t"
      "v_cndmask_b32_dpp %6, %10, %14, vcc row_ror:8 row_mask:0xf bank_mask:0xf\n\t"
      "v_cndmask_b32_dpp %7, %11, %15, vcc row_ror:8 row_mask:0xf bank_mask:0xf\n\t"
      "s_nop 1"
      : "=&v"(h0), "=&v"(h1), "=&v"(h2), "=&v"(h3), "=&v"(l0), "=&v"(l1), "=&v"(l2), "=&v"(l3)
      : "v"(hi[0]), "v"(hi[1]), "v"(hi[2]), "v"(hi[3]), "v"(lo[0]), "v"(lo[1]), "v"(lo[2]),
        "v"(lo[3])
      : "vcc");
  hi[0] = h0; hi[1] = h1; hi[2] = h2; hi[3] = h3;
  lo[0] = l0; lo[1] = l1; lo[2] = l2; lo[3] = l3;
}
// sum over the lanes l ^ 16 and l ^ 32 (gfx950 permlane swaps)
__device__ __forceinline__ float sum_x16_x32(float x) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}
__device__ __forceinline__ float max_x16_x32(float x) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}
// 2^x on the transcendental unit (results below 2^-126 flush to 0)
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
// sum / max over the 8 lanes sharing l % 8 (xor 8, 16, 32)
__device__ __forceinline__ float head_sum(float x) { return sum_x16_x32(x + xor8(x)); }
__device__ __forceinline__ float head_max(float x) { return max_x16_x32(fmaxf(x, xor8(x))); }

// VALU helpers are plain C or compiler builtins, never inline asm: a matrix
// core instruction that reads a VGPR needs two wait states after the VALU
// instruction that wrote it, and the compiler only inserts them for
// instructions it emitted itself (an inline-asm v_bfi_b32 one slot before an
// MFMA reading its result fed that MFMA a stale register).

// {f16(x0), f16(x1)}, round to nearest even, packed
__device__ __forceinline__ uint32_t pack_rn(float x0, float x1) {
  return __builtin_bit_cast(uint32_t, __floats2half2_rn(x0, x1));
}
// {f16(x0 − c.lo), f16(x1 − c.hi)} with c an fp16 pair that is 0 or the
// pack_rn of (x0, x1): the fp32 difference is exact, so each term is rounded
// once
__device__ __forceinline__ uint32_t pack_rn_sub(float x0, float x1, uint32_t c) {
  const __half2 h = __builtin_bit_cast(__half2, c);
  return pack_rn(x0 - __low2float(h), x1 - __high2float(h));
}
// fp16 high and low terms of x0 and x1, packed: high = x rounded toward zero
// to fp16 (in fp16's normal range that is x with its fp32 mantissa cut to 10
// bits), low = the exact remainder rounded toward zero; together 22
// significant bits. Only 4-byte instructions (the mixed-precision FMA form
// costs about three of them on gfx950). Requires |x| < 65504.
__device__ __forceinline__ void split_pair(float x0, float x1, uint32_t& hi, uint32_t& lo) {
  hi = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pkrtz(x0, x1));
  const float r0 = x0 - __uint_as_float(__float_as_uint(x0) & 0xFFFFE000u);
  const float r1 = x1 - __uint_as_float(__float_as_uint(x1) & 0xFFFFE000u);
  lo = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pkrtz(r0, r1));
}
// (mask & x) | (~mask & y): one v_bfi_b32
__device__ __forceinline__ uint32_t bfi(uint32_t mask, uint32_t x, uint32_t y) {
  return (mask & x) | (~mask & y);
}

// ---- K code positions. The conversions turn one byte (two fp4 nibbles) or
// one half-word (two fp8 bytes) into an fp16 pair, so in k-step sl the k-slots
// j = 0..7 of a lane whose 32 channels start at 32·u hold channels
// 8·sl + kslot_channel(j), kslot_channel = {0, 2, 1, 3, 4, 6, 5, 7} (both widths):
//   2-bit: word sl/2; m0 = w & 0x33333333 has code 2n in nibble n, m1 =
//          (w >> 2) & 0x33333333 code 2n+1; byte k of m0 / m1 gives codes
//          {4k, 4k+2} / {4k+1, 4k+3}; k-step sl uses bytes 2·(sl%2) + {0, 1}.
//   4-bit: word sl; m0 = w & 0x0F0F0F0F has code 2n in byte n, m1 =
//          (w >> 4) & 0x0F0F0F0F code 2n+1; half-word 0 / 1 of m0 gives codes
//          {0, 2} / {4, 6}, of m1 {1, 3} / {5, 7}.
__device__ __forceinline__ constexpr int kslot_channel(int j) {
  return 4 * (j / 4) + (j / 2) % 2 + 2 * (j % 2);
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

// Code masks of one token's K words (2-bit: 2 words → 4 masks; 4-bit: 4 words
// → 8 masks) and the A operand of k-step sl from them.
template <int BITS>
__device__ __forceinline__ void k_masks(const uint32_t (&w)[BITS], uint32_t (&m)[2 * BITS]) {
#pragma unroll
  for (int x = 0; x < BITS; ++x) {
    if (BITS == 2) {
      m[2 * x] = w[x] & 0x33333333u;
      m[2 * x + 1] = (w[x] >> 2) & 0x33333333u;
    } else {
      m[2 * x] = w[x] & 0x0F0F0F0Fu;
      m[2 * x + 1] = (w[x] >> 4) & 0x0F0F0F0Fu;
    }
  }
}
template <int BITS>
__device__ __forceinline__ u32x4 k_operand(const uint32_t (&m)[2 * BITS], int sl) {
  if (BITS == 2) {
    const uint32_t m0 = m[2 * (sl / 2)], m1 = m[2 * (sl / 2) + 1];
    const int k = 2 * (sl % 2);
    return u32x4{fp4x2_to_f16x2(m0, k), fp4x2_to_f16x2(m1, k), fp4x2_to_f16x2(m0, k + 1),
                 fp4x2_to_f16x2(m1, k + 1)};
  }
  const uint32_t m0 = m[2 * sl], m1 = m[2 * sl + 1];
  return u32x4{fp8x2_to_f16x2(m0, false), fp8x2_to_f16x2(m1, false), fp8x2_to_f16x2(m0, true),
               fp8x2_to_f16x2(m1, true)};
}

// Per-lane state of one wavefront across its groups; NVS V scales per token
// (runs of 128 / NVS channels) keep one zero-point sum and one offset sum each.
template <int NVS = 1>
struct WaveAccT {
  float m_ref, l_acc, pz_acc[NVS];
  f32x4 cv[8];
  f32x4 cones[NVS];
};
using WaveAcc = WaveAccT<1>;

// Softmax step for four scores, then P'·V for one group or window tile.
template <int NVS>
__device__ __forceinline__ void rescale_if_needed(WaveAccT<NVS>& W, const float (&sc)[4],
                                                  float lazy = kLazy) {
  const float lmax = fmaxf(fmaxf(sc[0], sc[1]), fmaxf(sc[2], sc[3]));
  if (__any(lmax > W.m_ref + lazy)) {            // wave-uniform, rare
    const float m_new = fmaxf(W.m_ref, head_max(lmax));
    const float alpha = fast_exp2(W.m_ref - m_new);
    W.l_acc *= alpha;
#pragma unroll
    for (int n = 0; n < 8; ++n) W.cv[n] *= alpha;
#pragma unroll
    for (int j = 0; j < NVS; ++j) {
      W.pz_acc[j] *= alpha;
      W.cones[j] *= alpha;
    }
    W.m_ref = m_new;
  }
}

// The same step for scores already taken relative to the reference maximum
// (the score accumulator starts at −m_ref): the threshold is the constant
// slack, and a raise by d shifts the reference and the four scores by d.
template <int NVS>
__device__ __forceinline__ void rescale_rel(WaveAccT<NVS>& W, float (&sc)[4]) {
  const float lmax = fmaxf(fmaxf(sc[0], sc[1]), fmaxf(sc[2], sc[3]));
  if (__any(lmax > kLazy)) {                     // wave-uniform, rare
    const float d = fmaxf(0.0f, head_max(lmax));
    const float alpha = fast_exp2(-d);
    W.l_acc *= alpha;
#pragma unroll
    for (int n = 0; n < 8; ++n) W.cv[n] *= alpha;
#pragma unroll
    for (int j = 0; j < NVS; ++j) {
      W.pz_acc[j] *= alpha;
      W.cones[j] *= alpha;
    }
    W.m_ref += d;
#pragma unroll
    for (int i = 0; i < 4; ++i) sc[i] -= d;
  }
}

// bf16 high / low terms of four P' values; part 0 ends with the high terms of
// tile 0 (own) and tile 1 (partner's), part 1 with the low terms of tile 0
// (partner's) and tile 1 (own): the B operand of the value products.
__device__ __forceinline__ u32x4 p_operand(const float (&pp)[4]) {
  uint32_t hp[2], lp[2];
#pragma unroll
  for (int p = 0; p < 2; ++p) {
    const float x0 = pp[2 * p], x1 = pp[2 * p + 1];
    const float l0 = x0 - __uint_as_float(__float_as_uint(x0) & 0xFFFF0000u);
    const float l1 = x1 - __uint_as_float(__float_as_uint(x1) & 0xFFFF0000u);
    hp[p] = __builtin_amdgcn_perm(__float_as_uint(x1), __float_as_uint(x0), 0x07060302u);
    lp[p] = __builtin_amdgcn_perm(__float_as_uint(l1), __float_as_uint(l0), 0x07060302u);
  }
  swap_halves2(hp, lp);
  return u32x4{hp[0], hp[1], lp[0], lp[1]};
}

// A group runs in three phases: scores, probabilities, value products. Each
// iteration of the main loop first issues all of its LDS reads (the V codes
// of group i - 1, the K codes and scales of group i), then computes the
// scores of group i and the value products of group i - 1 (independent
// instruction streams in one basic block), then turns the scores of group i
// into probabilities.

// LDS data of one group for one lane: K codes of tokens r and 16 + r
// (channels 32u..32u+31), K scale and zero-point of the lane's 16 channels,
// V scale and zero-point of the tokens it keeps (16·part + 4u + i): vs[0]
// holds the four tokens' scales (NVS = 1), or vs[i] token i's four run
// scales (NVS = 4).
template <int BITS, int NVS = 1>
struct KLoad {
  uint32_t w0[BITS], w1[BITS];
  float4 ks[4], kz[4];
  float4 vs[NVS], vz[NVS];
};
// V code words of channel 16n + r (n = 0..7) that lane group u needs
struct VLoad {
  uint32_t w[8][2];
};

template <int BITS, int VB, int NVS>
__device__ __forceinline__ void load_k(const uint8_t* st, int r, int u, bool low,
                                       KLoad<BITS, NVS>& K, bool kscale = true) {
  using S = Stage<BITS, VB, NVS>;
  const uint8_t* kc = st + S::kKc;
  constexpr int kRow = kHeadDim * BITS / 8;
  if (BITS == 2) {
    const uint2 x = *reinterpret_cast<const uint2*>(kc + r * kRow + 8 * u);
    const uint2 y = *reinterpret_cast<const uint2*>(kc + (16 + r) * kRow + 8 * u);
    K.w0[0] = x.x; K.w0[1] = x.y; K.w1[0] = y.x; K.w1[1] = y.y;
  } else {
    const uint4 x = *reinterpret_cast<const uint4*>(kc + r * kRow + 16 * u);
    const uint4 y = *reinterpret_cast<const uint4*>(kc + (16 + r) * kRow + 16 * u);
    K.w0[0] = x.x; K.w0[1] = x.y; K.w0[2] = x.z; K.w0[3] = x.w;
    K.w1[0] = y.x; K.w1[1] = y.y; K.w1[2] = y.z; K.w1[3] = y.w;
  }
  // K scales and zero-points (read apart, once per K group, when a group's
  // operands are kept across its tiles)
  if (kscale) {
    const float4* ksz = reinterpret_cast<const float4*>(st + S::kKsz) + 8 * u + (low ? 4 : 0);
#pragma unroll
    for (int c4 = 0; c4 < 4; ++c4) K.kz[c4] = ksz[kHeadDim / 4 + c4];
#pragma unroll
    for (int c4 = 0; c4 < 4; ++c4) K.ks[c4] = ksz[c4];
  }
  if (NVS == 1) {
    const float4* vsz = reinterpret_cast<const float4*>(st + S::kVsz) + (low ? 4 : 0) + u;
    K.vs[0] = vsz[0];
    K.vz[0] = vsz[kGroup / 4];
  } else {
    // token-major [32][NVS]: the lane's four tokens are NVS float4 each
    const float4* vsz = reinterpret_cast<const float4*>(st + S::kVsz) + (low ? 16 : 0) + 4 * u;
#pragma unroll
    for (int i = 0; i < NVS; ++i) {
      K.vs[i] = vsz[i];
      K.vz[i] = vsz[kGroup * NVS / 4 + i];
    }
  }
}

// K scales and zero-points of a stage alone (the kscale part of load_k)
template <int BITS, int VB, int NVS>
__device__ __forceinline__ void load_kscale(const uint8_t* st, int u, bool low,
                                            KLoad<BITS, NVS>& K) {
  using S = Stage<BITS, VB, NVS>;
  const float4* ksz = reinterpret_cast<const float4*>(st + S::kKsz) + 8 * u + (low ? 4 : 0);
#pragma unroll
  for (int c4 = 0; c4 < 4; ++c4) K.kz[c4] = ksz[kHeadDim / 4 + c4];
#pragma unroll
  for (int c4 = 0; c4 < 4; ++c4) K.ks[c4] = ksz[c4];
}

template <int KB, int BITS, int NVS>
__device__ __forceinline__ void load_v(const uint8_t* st, int r, int u, VLoad& V) {
  using S = Stage<KB, BITS, NVS>;
  const uint8_t* vc = st + S::kVc;
#pragma unroll
  for (int n = 0; n < 8; ++n) {
    if (BITS == 2) {
      const uint2 x = *reinterpret_cast<const uint2*>(vc + (16 * n + r) * 8);
      V.w[n][0] = x.x;
      V.w[n][1] = x.y;
    } else {
      const uint32_t* cw = reinterpret_cast<const uint32_t*>(vc + (16 * n + r) * 16);
      V.w[n][0] = cw[u / 2];
      V.w[n][1] = cw[2 + u / 2];
    }
  }
}

__device__ __forceinline__ float f4_at(const float4 (&v)[4], int i) {
  const float4 x = v[i / 4];
  return (i % 4 == 0) ? x.x : (i % 4 == 1) ? x.y : (i % 4 == 2) ? x.z : x.w;
}

// Scores of the four tokens this lane keeps (log2 units).
template <int BITS, int NVS>
__device__ __forceinline__ void group_scores(const KLoad<BITS, NVS>& K, bool low,
                                             const float (&q16)[16], float m_part,
                                             float (&sc)[4]) {
  uint32_t m0[2 * BITS], m1[2 * BITS];
  k_masks<BITS>(K.w0, m0);
  k_masks<BITS>(K.w1, m1);
  // ---- z-term of this lane's 16 channels less its share of the reference
  // maximum, as one chain of fused multiply-adds
  float zacc = -m_part;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const float4 z = K.kz[j];
    zacc = fmaf(q16[4 * j], z.x, zacc);
    zacc = fmaf(q16[4 * j + 1], z.y, zacc);
    zacc = fmaf(q16[4 * j + 2], z.z, zacc);
    zacc = fmaf(q16[4 * j + 3], z.w, zacc);
  }
  // The z-term summed over the four lane groups by the matrix cores (one
  // 16×16×16 product instead of two lane swaps and the accumulator fills):
  // B holds the lane's partial, less −m_ref once per head (lane group 0 of
  // part 0, the m_part the caller passes there), times 2^-8, as an fp16
  // high/low pair in k-slots 0 and 1 (slots 2 and 3 zero); A is 256 in every
  // slot. Each column's sum over the lane groups then lands in every row of
  // that column, the accumulator the scores build on. The 2^-8 (undone
  // exactly by A) keeps partials up to 2^24 inside fp16's range; the pair
  // carries 22 significant bits, and fp16's subnormal step adds at most
  // 2^-16 per partial (2^-13 over the 8 partials of a score, in log2 units).
  const float zs = zacc * 0.00390625f;
  const float zr = zs - __uint_as_float(__float_as_uint(zs) & 0xFFFFE000u);
  const u32x2 bz = u32x2{__builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pkrtz(zs, zr)), 0u};
  const u32x2 a256 = u32x2{0x5C005C00u, 0x5C005C00u};
  f32x4 s0 = __builtin_amdgcn_mfma_f32_16x16x16f16(as_f16x4(a256), as_f16x4(bz),
                                                   f32x4{0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
  f32x4 s1 = s0;
  // ---- scores: local k-step h is global k-step h (part 0) or 2 + h (part 1)
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    uint32_t hi[4], lo[4];
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      const int c0 = 8 * h + kslot_channel(2 * p), c1 = 8 * h + kslot_channel(2 * p + 1);
      split_pair(q16[c0] * f4_at(K.ks, c0), q16[c1] * f4_at(K.ks, c1), hi[p], lo[p]);
    }
    // part 0 takes the partner's high terms (k-step 2 + h), part 1 the
    // partner's low terms (k-step h)
    swap_halves4(hi, lo);
    const u32x4 bh = u32x4{hi[0], hi[1], hi[2], hi[3]};
    const u32x4 bl = u32x4{lo[0], lo[1], lo[2], lo[3]};
    s0 = __builtin_amdgcn_mfma_f32_16x16x32_f16(as_f16x8(k_operand<BITS>(m0, h)), as_f16x8(bh), s0, 0, 0, 0);
    s1 = __builtin_amdgcn_mfma_f32_16x16x32_f16(as_f16x8(k_operand<BITS>(m1, h)), as_f16x8(bh), s1, 0, 0, 0);
    s0 = __builtin_amdgcn_mfma_f32_16x16x32_f16(as_f16x8(k_operand<BITS>(m0, 2 + h)), as_f16x8(bl), s0, 0, 0, 0);
    s1 = __builtin_amdgcn_mfma_f32_16x16x32_f16(as_f16x8(k_operand<BITS>(m1, 2 + h)), as_f16x8(bl), s1, 0, 0, 0);
  }
  // ---- both columns of the head; part 0 keeps tile 0, part 1 tile 1
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float t0 = s0[i] + xor8(s0[i]);
    const float t1 = s1[i] + xor8(s1[i]);
    sc[i] = low ? t1 : t0;
  }
}

// With G > 32 (the K scales and zero-points shared by G / 32 tiles) the
// score-side operands of a K group are built once, on its first tile, and
// kept across the group's tiles: Q' as the B operands of both halves of the
// k-steps (high and low terms already exchanged) and the z-term.
struct GroupQ {
  u32x4 bh[2], bl[2];
  float zt;
};

// The first half of group_scores: Q' and the z-term of a K group.
template <int BITS, int NVS>
__device__ __forceinline__ void group_q(const KLoad<BITS, NVS>& K, const float (&q16)[16],
                                        GroupQ& Q) {
  float zp[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const float4 z = K.kz[j];
    zp[j] = fmaf(q16[4 * j + 3], z.w, fmaf(q16[4 * j + 2], z.z,
                 fmaf(q16[4 * j + 1], z.y, q16[4 * j] * z.x)));
  }
  Q.zt = sum_x16_x32((zp[0] + zp[1]) + (zp[2] + zp[3]));
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    uint32_t hi[4], lo[4];
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      const int c0 = 8 * h + kslot_channel(2 * p), c1 = 8 * h + kslot_channel(2 * p + 1);
      split_pair(q16[c0] * f4_at(K.ks, c0), q16[c1] * f4_at(K.ks, c1), hi[p], lo[p]);
    }
    swap_halves4(hi, lo);
    Q.bh[h] = u32x4{hi[0], hi[1], hi[2], hi[3]};
    Q.bl[h] = u32x4{lo[0], lo[1], lo[2], lo[3]};
  }
}

// The second half of group_scores: the scores of one tile from its K codes
// and its group's operands.
template <int BITS, int NVS>
__device__ __forceinline__ void tile_scores(const KLoad<BITS, NVS>& K, bool low, const GroupQ& Q,
                                            float m_part, float (&sc)[4]) {
  uint32_t m0[2 * BITS], m1[2 * BITS];
  k_masks<BITS>(K.w0, m0);
  k_masks<BITS>(K.w1, m1);
  const float zt = Q.zt - m_part;
  f32x4 s0 = f32x4{zt, zt, zt, zt}, s1 = s0;
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    s0 = __builtin_amdgcn_mfma_f32_16x16x32_f16(as_f16x8(k_operand<BITS>(m0, h)), as_f16x8(Q.bh[h]), s0, 0, 0, 0);
    s1 = __builtin_amdgcn_mfma_f32_16x16x32_f16(as_f16x8(k_operand<BITS>(m1, h)), as_f16x8(Q.bh[h]), s1, 0, 0, 0);
    s0 = __builtin_amdgcn_mfma_f32_16x16x32_f16(as_f16x8(k_operand<BITS>(m0, 2 + h)), as_f16x8(Q.bl[h]), s0, 0, 0, 0);
    s1 = __builtin_amdgcn_mfma_f32_16x16x32_f16(as_f16x8(k_operand<BITS>(m1, 2 + h)), as_f16x8(Q.bl[h]), s1, 0, 0, 0);
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float t0 = s0[i] + xor8(s0[i]);
    const float t1 = s1[i] + xor8(s1[i]);
    sc[i] = low ? t1 : t0;
  }
}

// Online-softmax step for the group's scores; sets the B operands P' of its
// value products (p times the V scale, one per run of V channels with its
// own scale). REL: the scores are relative to the reference maximum already;
// otherwise (the first group of a wavefront) they are absolute.
__device__ __forceinline__ float f4c(float4 x, int c) {
  return c == 0 ? x.x : c == 1 ? x.y : c == 2 ? x.z : x.w;
}
template <int BITS, bool REL, int NVS>
__device__ __forceinline__ void group_probs(WaveAccT<NVS>& W, float (&sc)[4],
                                            const float4 (&vs)[NVS], const float4 (&vz)[NVS],
                                            u32x4 (&bp)[NVS]) {
  if (REL) {
    rescale_rel(W, sc);
  } else {
    rescale_if_needed(W, sc);
#pragma unroll
    for (int i = 0; i < 4; ++i) sc[i] -= W.m_ref;
  }
  if constexpr (NVS == 1) {
    const float vsa[4] = {vs[0].x, vs[0].y, vs[0].z, vs[0].w};
    const float vza[4] = {vz[0].x, vz[0].y, vz[0].z, vz[0].w};
    float pp[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float p = fast_exp2(sc[i]);
      W.l_acc += p;
      W.pz_acc[0] = fmaf(p, vza[i], W.pz_acc[0]);
      pp[i] = p * vsa[i];
    }
    bp[0] = p_operand(pp);
  } else {
    float p[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      p[i] = fast_exp2(sc[i]);
      W.l_acc += p[i];
    }
#pragma unroll
    for (int j = 0; j < NVS; ++j) {
      // token i's scale of run j is component j of vs[i]
      float pp[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        W.pz_acc[j] = fmaf(p[i], f4c(vz[i], j), W.pz_acc[j]);
        pp[i] = p[i] * f4c(vs[i], j);
      }
      bp[j] = p_operand(pp);
    }
  }
}

// P'·V of one group: 8 tiles of 16 channels, codes in the mantissa of 128.0
// or 32.0, plus the offset-weighted column sums of P' that remove the offsets.
template <int BITS, int NVS>
__device__ __forceinline__ void group_values(const VLoad& V, WaveAccT<NVS>& W,
                                             const u32x4 (&bp)[NVS], uint32_t vsh,
                                             uint32_t vm0, uint32_t vm1, uint32_t magic,
                                             uint32_t magic32) {
#pragma unroll
  for (int n = 0; n < 8; ++n) {
    uint32_t d[4];
    // both words shifted at once: the bits of the second word that enter the
    // first (at 20 and above for shifts up to 12) lie outside the masks
    const uint64_t pair = (uint64_t(V.w[n][1]) << 32) | V.w[n][0];
    if (BITS == 2) {
      const uint64_t x = pair >> vsh;
      const uint32_t v0 = uint32_t(x), v1 = uint32_t(x >> 32);
      d[0] = bfi(vm0, v0, magic);
      d[1] = bfi(vm1, v0, magic32);
      d[2] = bfi(vm0, v1, magic);
      d[3] = bfi(vm1, v1, magic32);
    } else {
      const uint64_t x = pair >> vsh, y = pair >> (vsh + 4);
      d[0] = bfi(vm0, uint32_t(x), magic);
      d[1] = bfi(vm0, uint32_t(y), magic);
      d[2] = bfi(vm0, uint32_t(x >> 32), magic);
      d[3] = bfi(vm0, uint32_t(y >> 32), magic);
    }
    // channels 16n..16n+15 lie in run n·NVS/8
    W.cv[n] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(u32x4{d[0], d[1], d[2], d[3]}),
                                                       as_bf16x8(bp[n * NVS / 8]), W.cv[n], 0,
                                                       0, 0);
  }
  // each k-slot's code offset over 128 (1, or 1/4 for the 2-bit codes in
  // bits 2..3, whose offset is 32): 128 times this product is what the codes
  // carry on top of their values
  const uint32_t o1 = BITS == 2 ? 0x3E803E80u : 0x3F803F80u;
  const u32x4 offs = u32x4{0x3F803F80u, o1, 0x3F803F80u, o1};
#pragma unroll
  for (int j = 0; j < NVS; ++j)
    W.cones[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(offs), as_bf16x8(bp[j]),
                                                         W.cones[j], 0, 0, 0);
}

// One 32-token tile of the FP16 window ("4.4 KV Cache 量化：KIVI 2-bit 与 FP8
// KV Cache", §3.2: the newest tokens stay unquantized). Scores: A = K values
// (fp16, exact), B = fp16 high/low terms of q·log2e/√D (channels 32s + 8u + j
// in k-step s). Values: V enters as two exact bf16 terms (fp16 has 11
// significant bits, a bf16 pair holds 16), P' = p as a bf16 high/low pair.
// Tokens past n_win are masked (score −∞, value 0).
template <int NVS>
__device__ __forceinline__ void process_window_tile(const DecodeArgs& a, WaveAccT<NVS>& W, int bh,
                                                    int64_t tile, const u32x4 (&bqw)[4],
                                                    int r, int u, bool low, int n_win) {
  const __half* kw = a.k_win + (int64_t(bh) * a.win_cap + tile * kGroup) * kHeadDim;
  const __half* vwp = a.v_win + (int64_t(bh) * a.win_cap + tile * kGroup) * kHeadDim;
  const int n_in = int(min<int64_t>(kGroup, n_win - tile * kGroup));
  // a folded append: the newest token (slot n_win − 1) comes from the
  // caller's buffer, not from the window it is being stored into
  const bool here = a.k_new != nullptr && n_win - tile * kGroup <= kGroup;
  const int t_new = here ? n_in - 1 : -1;                  // its slot in this tile
  const __half* k_new = here ? a.k_new + int64_t(bh) * kHeadDim : kw;
  const __half* v_new = here ? a.v_new + int64_t(bh) * kHeadDim : vwp;
  const __half* k_row0 = r == t_new ? k_new : kw + r * kHeadDim;
  const __half* k_row1 = 16 + r == t_new ? k_new : kw + (16 + r) * kHeadDim;
  f32x4 s0 = f32x4{0.f, 0.f, 0.f, 0.f}, s1 = s0;
#pragma unroll
  for (int sl = 0; sl < 4; ++sl) {
    const uint4 k0 = *reinterpret_cast<const uint4*>(k_row0 + 32 * sl + 8 * u);
    const uint4 k1 = *reinterpret_cast<const uint4*>(k_row1 + 32 * sl + 8 * u);
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
  rescale_if_needed(W, sc);
  float pp[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    pp[i] = fast_exp2(sc[i] - W.m_ref);      // 0 for masked tokens
    W.l_acc += pp[i];
  }
  const u32x4 bp = p_operand(pp);
  // V^T tiles: lane (r, u) needs channel 16n + r at tokens 4u + j (j < 4) and
  // 16 + 4u + j - 4. Every slot of a window tile lies inside the window buffer
  // (its capacity is a whole number of tiles), so the loads are issued
  // unconditionally, those of two channel tiles at a time in flight together;
  // masked tokens become 0 after the load (a slot past the last token may hold
  // anything, even a NaN).
  __half vh[2][8];
#pragma unroll
  for (int n = 0; n < 8; ++n) {
    if (n % 2 == 0) {
#pragma unroll
      for (int m = 0; m < 2; ++m) {
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const int t = (j < 4) ? 4 * u + j : 16 + 4 * u + (j - 4);
          vh[m][j] = (t == t_new ? v_new : vwp + t * kHeadDim)[16 * (n + m) + r];
        }
      }
    }
    float v[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int t = (j < 4) ? 4 * u + j : 16 + 4 * u + (j - 4);
      const float x = __half2float(vh[n % 2][j]);
      v[j] = t < n_in ? x : 0.0f;
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

// The FP16 window tiles of (b, h): tile t goes to wavefront t % NW.
template <int NVS, int NW = kWaves>
__device__ __forceinline__ void run_window(const DecodeArgs& a, WaveAccT<NVS>& W, int bh, int b,
                                           int hq0, int nh, int hs, int r, int u, bool low,
                                           int wave, int n_win) {
  // the FP16 window: q·log2e/√D as fp16 high/low terms, channel 32s + 8u + j
  u32x4 bqw[4];
  {
    const uint32_t selmask = low ? 0xFFFFFFFFu : 0u;
    const bool valid = hs < nh;
    const float qs = valid ? a.qscale : 0.0f;
    const float* qrow = a.q + (int64_t(b) * a.Hq + hq0 + (valid ? hs : 0)) * kHeadDim;
#pragma unroll
    for (int sl = 0; sl < 4; ++sl) {
      uint32_t d[4];
#pragma unroll
      for (int p = 0; p < 4; ++p) {
        const float x0 = qrow[32 * sl + 8 * u + 2 * p] * qs;
        const float x1 = qrow[32 * sl + 8 * u + 2 * p + 1] * qs;
        const uint32_t hi = pack_rn(x0, x1);
        d[p] = pack_rn_sub(x0, x1, hi & selmask);
      }
      bqw[sl] = u32x4{d[0], d[1], d[2], d[3]};
    }
  }
  const int64_t n_tiles = (n_win + kGroup - 1) / kGroup;
  // a folded append: wavefront 0 of head chunk 0 stores the appended token
  // into its window slot (16 lanes for K, 16 for V, 16 bytes each); no
  // wavefront of this launch reads that slot from the window
  if (a.k_new != nullptr && wave == 0 && hq0 % a.nq == 0 && n_win > 0) {
    const int lane = u * 16 + r;
    if (lane < 32) {
      const int c = lane & 15;
      const __half* src = (lane < 16 ? a.k_new : a.v_new) + int64_t(bh) * kHeadDim + 8 * c;
      __half* dst = (lane < 16 ? a.k_win_store : a.v_win_store) +
                    (int64_t(bh) * a.win_cap + n_win - 1) * kHeadDim + 8 * c;
      *reinterpret_cast<uint4*>(dst) = *reinterpret_cast<const uint4*>(src);
    }
  }
  for (int64_t tile = wave; tile < n_tiles; tile += NW)
    process_window_tile(a, W, bh, tile, bqw, r, u, low, n_win);
}

// Asynchronous global→LDS copies (global_load_lds): lane i's 16 or 4 bytes
// land at M0 + offset + 16·i (or 4·i); the immediate offset moves the global
// address by the same amount, so every global base below is biased by minus
// the stage offset its copy lands at. The copies are issued from inline asm so
// that the compiler does not model them: it cannot tell the ring's stages
// apart and would otherwise wait for every copy in flight (vmcnt(0)) before
// each LDS read. The kernel orders them itself with s_waitcnt vmcnt (copies
// complete in issue order). They are non-temporal (nt): the cache is streamed
// once per decode, and the streaming hint is worth about a fifth of the
// achievable HBM read rate. M0 and EXEC are restored at the end of each block.
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return static_cast<uint32_t>(
      reinterpret_cast<uintptr_t>((__attribute__((address_space(3))) const void*)(p)));
}

// Wave epilogue and workgroup merge, shared by the decode kernels: head
// totals, removal of the offsets of the value codes (zero when unused),
// high + low columns, times oscale; then the four wave states are merged
// through LDS (each wave's results go to the start of its own ring region,
// `wave_stride` bytes apart) into this split's partial (o[D], m, l).
template <int NVS, int NW = kWaves>
__device__ __forceinline__ void wave_epilogue_and_merge(const DecodeArgs& a, const WaveAccT<NVS>& W,
                                                        uint8_t* ring, size_t wave_stride,
                                                        int wave, int lane, int hs, int u,
                                                        bool low, int tid, int b, int hq0,
                                                        int nh, int split, float oscale) {
  float* mo = reinterpret_cast<float*>(ring + wave * wave_stride);     // [8][kHeadDim]
  float* ml = mo + 8 * kHeadDim;                                         // [8][2]
  const float l_tot = head_sum(W.l_acc);
  float pz_tot[NVS], off[NVS];     // zero-point sum and code offsets, per V run
#pragma unroll
  for (int j = 0; j < NVS; ++j) {
    pz_tot[j] = head_sum(W.pz_acc[j]);
    off[j] = 128.0f * (W.cones[j][0] + xor8(W.cones[j][0]));
  }
#pragma unroll
  for (int n = 0; n < 8; ++n) {
    f32x4 o;
    const int j = n * NVS / 8;
#pragma unroll
    for (int i = 0; i < 4; ++i) o[i] = (W.cv[n][i] + xor8(W.cv[n][i]) - off[j] + pz_tot[j]) * oscale;
    if (!low) *reinterpret_cast<f32x4*>(&mo[hs * kHeadDim + 16 * n + 4 * u]) = o;
  }
  if (lane < 8) {
    ml[2 * hs] = W.m_ref;
    ml[2 * hs + 1] = l_tot;
  }
  __syncthreads();
  for (int i = tid; i < nh * kHeadDim; i += 64 * NW) {
    const int h = i / kHeadDim;
    const int d = i % kHeadDim;
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      const float* mlw = reinterpret_cast<const float*>(ring + w * wave_stride) + 8 * kHeadDim;
      M = fmaxf(M, mlw[2 * h]);
    }
    float O = 0.0f, L = 0.0f;
    if (M != -INFINITY) {
#pragma unroll
      for (int w = 0; w < NW; ++w) {
        const float* mow = reinterpret_cast<const float*>(ring + w * wave_stride);
        const float* mlw = mow + 8 * kHeadDim;
        const float mw = mlw[2 * h];
        const float f = mw == -INFINITY ? 0.0f : exp2f(mw - M);
        O = fmaf(f, mow[h * kHeadDim + d], O);
        L = fmaf(f, mlw[2 * h + 1], L);
      }
    }
    if (KVQ_DIRECT_SINGLE_SPLIT && a.n_split == 1) {
      // one split per row: the merge would compute exactly O / L (its one
      // weight is 2^0 = 1), so the output is written here and no merge runs
      a.out[(int64_t(b) * a.Hq + hq0 + h) * kHeadDim + d] = O / L;
      continue;
    }
    float* part = a.ws + ((int64_t(b) * a.Hq + hq0 + h) * a.n_split + split) * kPart;
    part[d] = O;
    if (d == 0) {
      part[kHeadDim] = M;
      part[kHeadDim + 1] = L;
    }
  }
}

// Block order of the split kernels: a 1-D grid, split-major — block id
// covers split id / X of (b, h, head chunk) id % X, X = B·H·chunks. All
// (b, h) of split 0 come first, then split 1, and so on, so the window-only
// split (index n_split_main, when the window has a split of its own) runs
// last, and in a ragged batch the splits past a short sequence's end (empty
// blocks) come after the populated ones instead of holding back the first
// round of resident workgroups.
struct BlockCoord {
  int split, bh, chunk;
};
__device__ __forceinline__ BlockCoord block_coord(const DecodeArgs& a) {
  const int x = a.B * a.H * (a.nq / a.heads_per_chunk);
  const int id = int(blockIdx.x);
  const int rest = id % x;
  BlockCoord c;
  c.split = id / x;
  c.bh = rest % (a.B * a.H);
  c.chunk = rest / (a.B * a.H);
  return c;
}
__host__ inline dim3 split_grid(const DecodeArgs& a) {
  return dim3(unsigned(a.n_split) * unsigned(a.B * a.H) * unsigned(a.nq / a.heads_per_chunk));
}

// Wave-uniform, offset-biased sources of the next group a wavefront loads.
struct GroupSrc {
  const uint8_t* kc;   // K codes
  const uint8_t* vc;   // V codes
  const uint8_t* ks;   // K scales, read by lanes 0..31
  const uint8_t* kz;   // K zero-points, read by lanes 32..63
  const uint8_t* vs;   // V scales, lanes 0..31
  const uint8_t* vz;   // V zero-points, lanes 32..63
};

// Sources of 32-token tile g of (b, h); its K scales and zero-points are
// those of group g >> gshift (G = 32 << gshift tokens share them). A paged
// cache's tile sits in the (page, h) block of the page its sequence's block
// table names (clamped into the pool), as tile g mod (page tiles) of it.
template <int BITS, int VB, int NVS, bool PAGED>
__device__ __forceinline__ GroupSrc group_src(const DecodeArgs& a, int bh, int b, int h,
                                              int64_t g) {
  using S = Stage<BITS, VB, NVS>;
  int64_t blk = bh;
  if constexpr (PAGED) {
    // a scalar load (the table is read-only for the launch): a vector load's
    // wait would also drain the copies in flight, every tile
    typedef __attribute__((address_space(4))) const int32_t ConstI32;
    const ConstI32* table = (const ConstI32*)(a.block_table);
    const int e = table[int64_t(b) * a.max_pages + (g >> a.page_tile_shift)];
    blk = int64_t(min(max(e, 0), a.num_pages - 1)) * a.H + h;
    g &= (int64_t(1) << a.page_tile_shift) - 1;
  }
  const int64_t kg = (blk * a.NG + (g >> a.gshift)) * kHeadDim * 4;   // bytes
  const int64_t vg = (blk * a.main_bh_tokens + g * kGroup) * 4 * NVS;
  GroupSrc P;
  P.kc = static_cast<const uint8_t*>(a.k_main) +
         (blk * a.main_bh_tokens + g * kGroup) * (kHeadDim * BITS / 8) - S::kKc;
  P.vc = static_cast<const uint8_t*>(a.v_main) + (blk * a.NT + g) * S::kVBytes -
         (S::kVc - S::kSecond);
  P.ks = reinterpret_cast<const uint8_t*>(a.k_scale) + kg - (S::kKsz - S::kSecond);
  P.kz = reinterpret_cast<const uint8_t*>(a.k_zero) + kg - (S::kKsz - S::kSecond);
  P.vs = reinterpret_cast<const uint8_t*>(a.v_scale) + vg - (S::kVsz - S::kSecond);
  P.vz = reinterpret_cast<const uint8_t*>(a.v_zero) + vg - (S::kVsz - S::kSecond);
  return P;
}

// Copies of one group into stage st: K codes (block 1, M0 = st), then V
// codes, K scale | zero and V scale | zero (block 2, M0 = st + kSecond).
// v16 = 16·lane, h16 = 16·(lane % 32), h4 = 4·(lane % 32). Stage::kLoads
// instructions per group.
// K and V code copies: one 1 KiB copy per 2 bits of width
#define KVQ_COPY_K1 "global_load_lds_dwordx4 %3, %6 nt\n\t"
#define KVQ_COPY_K2 KVQ_COPY_K1 "global_load_lds_dwordx4 %3, %6 offset:1024 nt\n\t"
#define KVQ_COPY_V1 "global_load_lds_dwordx4 %3, %7 offset:%13 nt\n\t"
#define KVQ_COPY_V2 KVQ_COPY_V1 "global_load_lds_dwordx4 %3, %7 offset:%16 nt\n\t"
// V scales and zero-points of a tile: 128 B each (one dword per lane), or
// 512 B each with four scales per token (16 bytes per lane)
#define KVQ_COPY_VS1 "global_load_lds_dword %5, %10 offset:%15 nt\n\t"
#define KVQ_COPY_VZ1 "global_load_lds_dword %5, %12 offset:%15 nt\n\t"
#define KVQ_COPY_VS4 "global_load_lds_dwordx4 %4, %10 offset:%15 nt\n\t"
#define KVQ_COPY_VZ4 "global_load_lds_dwordx4 %4, %12 offset:%15 nt\n\t"
#define KVQ_ISSUE_TILE(KCOPY, VCOPY, VSCOPY, VZCOPY)                                          \
  asm volatile("s_mov_b32 %0, m0\n\t"                                                         \
               "s_mov_b32 m0, %2\n\t"                                                         \
               "s_nop 0\n\t" KCOPY                                                            \
               "s_mov_b32 m0, %9\n\t"                                                         \
               "s_nop 0\n\t" VCOPY                                                            \
               "s_mov_b64 %1, exec\n\t"                                                       \
               "s_mov_b32 exec_hi, 0\n\t"                                                     \
               "global_load_lds_dwordx4 %4, %8 offset:%14 nt\n\t" VSCOPY                      \
               "s_mov_b64 exec, %1\n\t"                                                       \
               "s_mov_b32 exec_lo, 0\n\t"                                                     \
               "global_load_lds_dwordx4 %4, %11 offset:%14 nt\n\t" VZCOPY                     \
               "s_mov_b64 exec, %1\n\t"                                                       \
               "s_mov_b32 m0, %0"                                                             \
               : "=&s"(m), "=&s"(e)                                                           \
               : "s"(lds_addr(st)), "v"(v16), "v"(h16), "v"(h4), "s"(P.kc), "s"(P.vc),        \
                 "s"(P.ks), "s"(lds_addr(st + S::kSecond)), "s"(P.vs), "s"(P.kz), "s"(P.vz),  \
                 "i"(S::kVc - S::kSecond), "i"(S::kKsz - S::kSecond),                        \
                 "i"(S::kVsz - S::kSecond), "i"(S::kVc - S::kSecond + 1024)                   \
               : "memory")

template <int KB, int VB, int NVS>
__device__ __forceinline__ void issue_group(uint8_t* st, const GroupSrc& P, uint32_t v16,
                                            uint32_t h16, uint32_t h4) {
  using S = Stage<KB, VB, NVS>;
  uint32_t m;
  uint64_t e;
  if constexpr (NVS == 1) {
    if constexpr (KB == 2 && VB == 2) {
      KVQ_ISSUE_TILE(KVQ_COPY_K1, KVQ_COPY_V1, KVQ_COPY_VS1, KVQ_COPY_VZ1);
    } else if constexpr (KB == 4 && VB == 4) {
      KVQ_ISSUE_TILE(KVQ_COPY_K2, KVQ_COPY_V2, KVQ_COPY_VS1, KVQ_COPY_VZ1);
    } else if constexpr (KB == 4) {
      KVQ_ISSUE_TILE(KVQ_COPY_K2, KVQ_COPY_V1, KVQ_COPY_VS1, KVQ_COPY_VZ1);
    } else {
      KVQ_ISSUE_TILE(KVQ_COPY_K1, KVQ_COPY_V2, KVQ_COPY_VS1, KVQ_COPY_VZ1);
    }
  } else {
    static_assert(NVS == 4, "four V scales per token (runs of 32 channels)");
    if constexpr (KB == 2 && VB == 2) {
      KVQ_ISSUE_TILE(KVQ_COPY_K1, KVQ_COPY_V1, KVQ_COPY_VS4, KVQ_COPY_VZ4);
    } else if constexpr (KB == 4 && VB == 4) {
      KVQ_ISSUE_TILE(KVQ_COPY_K2, KVQ_COPY_V2, KVQ_COPY_VS4, KVQ_COPY_VZ4);
    } else if constexpr (KB == 4) {
      KVQ_ISSUE_TILE(KVQ_COPY_K2, KVQ_COPY_V1, KVQ_COPY_VS4, KVQ_COPY_VZ4);
    } else {
      KVQ_ISSUE_TILE(KVQ_COPY_K1, KVQ_COPY_V2, KVQ_COPY_VS4, KVQ_COPY_VZ4);
    }
  }
}

// Wait until at most `ahead` groups' copies are in flight.
template <int BITS, int VB, int NVS>
__device__ __forceinline__ void wait_groups(int ahead) {
  using S = Stage<BITS, VB, NVS>;
  if (ahead >= 2) wait_vmem<2 * S::kLoads>();
  else if (ahead == 1) wait_vmem<S::kLoads>();
  else wait_vmem<0>();
}

// Wavefronts per SIMD each KIVI instance's registers allow, and its
// workgroup size. The wavefronts of a workgroup take the split's 32-token
// tiles from one LDS counter, so however the SIMDs share their issue slots
// between them (older wavefronts go first), they all run out of tiles within
// about one tile of each other; with a fixed share per wavefront, or per
// workgroup among several workgroups on a unit, the favoured ones finish
// early and leave their SIMDs one wavefront deep for the rest of the launch
// (measured: three equal workgroups per unit ended at 46, 67 and 88 µs of a
// 91 µs launch).
// Wavefronts per SIMD: what registers and LDS allow (2-bit K and V, or one of
// them 4-bit: 3 at up to 170 VGPRs; 4-bit K and V, and every instance with V
// scales per 32 channels: 2).
template <int BITS, int VB, int NVS>
constexpr int kivi_waves_per_simd() {
  return (BITS == 2 && VB == 2 && NVS == 1) ? KVQ_DECODE_WAVES_PER_SIMD
         : (NVS == 1 && !(BITS == 4 && VB == 4)) ? 3
                                                 : 2;
}
// Each instance comes in two workgroup shapes: UNIT = the whole compute unit
// in one workgroup (that many wavefronts on each SIMD, tiles shared), for
// launches with at most one (b, h) block per unit; otherwise four-wavefront
// workgroups with a fixed tile order, which keep a unit busy across the many
// rounds of a launch with more blocks than units (a unit-sized workgroup
// leaves the unit idle between rounds: 7 % on the 4-bit B = 64 layer).
template <int BITS, int VB, int NVS, bool UNIT>
constexpr int kivi_waves() {
  return UNIT ? 4 * kivi_waves_per_simd<BITS, VB, NVS>() : 4;
}

// GRP (G > 32, one V scale per token, contiguous cache): a wavefront takes
// whole K groups of G / 32 tiles and keeps the group's score operands across
// them (K scales read, Q' split and z-term summed once per group).
template <int BITS, int VB, int NVS, bool UNIT, bool PAGED, bool GRP = false>
__global__ __launch_bounds__((64 * kivi_waves<BITS, VB, NVS, UNIT>()))
__attribute__((amdgpu_waves_per_eu((kivi_waves_per_simd<BITS, VB, NVS>())))) void kivi_mfma_split_kernel(
    DecodeArgs a) {
  static_assert(!GRP || (NVS == 1 && !PAGED), "group operands kept on the contiguous layout");
  using S = Stage<BITS, VB, NVS>;
  constexpr int NW = kivi_waves<BITS, VB, NVS, UNIT>();
  // ring stages per wavefront: the unit-sized workgroup keeps one group in
  // flight ahead (its wavefronts hold fewer tiles when the split runs out,
  // and it measured faster than two ahead: 32K GQA 92 -> 88 us)
  constexpr int kDepth = UNIT ? KVQ_RING_STAGES_UNIT : S::kDepth;
  static_assert(kDepth >= 3 && kDepth <= 4, "one or two groups in flight ahead");
  __shared__ __attribute__((aligned(16))) uint8_t ring[NW][kDepth][S::kBytes];
  __shared__ uint32_t next_tile;   // tiles of this split handed out so far

  const BlockCoord bc = block_coord(a);
  const int split = bc.split;
  const int bh = bc.bh;
  const int b = bh / a.H;
  const int h_kv = bh % a.H;
  const int hq0 = h_kv * a.nq + bc.chunk * a.heads_per_chunk;
  const int nh = min(a.heads_per_chunk, a.nq - bc.chunk * a.heads_per_chunk);
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int r = lane & 15;
  const int u = lane >> 4;
  const int hs = r & 7;
  const bool low = r >= 8;

  const uint32_t vsh = (VB == 2) ? uint32_t(4 * u) : uint32_t(8 * (u % 2));
  uint32_t vm0 = (VB == 2) ? 0x00030003u : 0x000F000Fu;
  uint32_t vm1 = 0x000C000Cu;
  uint32_t magic = 0x43004300u;           // bf16 128.0: codes in bits 0..3 count 1
  uint32_t magic32 = 0x42004200u;         // bf16 32.0: codes in bits 2..3 count 1
  // registers the compiler cannot fold (an empty asm, no instruction): with
  // the constants known it splits each bit insert into an and plus an or;
  // with them opaque it selects one v_bfi_b32 and still tracks its hazards
  asm("" : "+v"(vm0), "+v"(vm1), "+v"(magic), "+v"(magic32));

  WaveAccT<NVS> W;
  W.m_ref = -INFINITY;
  W.l_acc = 0.0f;
#pragma unroll
  for (int n = 0; n < 8; ++n) W.cv[n] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int j = 0; j < NVS; ++j) {
    W.pz_acc[j] = 0.0f;
    W.cones[j] = f32x4{0.f, 0.f, 0.f, 0.f};
  }

  // grouped tokens, window tokens and the split that runs the window: the
  // launch's, or this sequence's in a ragged batch (its window joins its
  // last main split, or split 0 when it has no grouped tiles)
  int64_t n_main = a.n_main;
  int n_win = a.n_win;
  int win_split = a.win_split;
  if (a.ragged) {
    const int tiles = a.seq.x[b];
    n_main = int64_t(tiles) * kGroup;
    n_win = a.seq.y[b];
    win_split = n_win <= 0 ? -1 : tiles > 0 ? (tiles + a.tiles_per_split - 1) / a.tiles_per_split - 1 : 0;
  }

  if (tid == 0) next_tile = 0;
  __syncthreads();

  if (split < a.n_split_main) {
    // q_d·log2e/√D of this lane's channels 32u + 16·part + c
    float q16[16];
    {
      // head slots past the chunk read head 0 and get weight 0
      const bool valid = hs < nh;
      const float qs = valid ? a.qscale : 0.0f;
      const float4* qrow = reinterpret_cast<const float4*>(
          a.q + (int64_t(b) * a.Hq + hq0 + (valid ? hs : 0)) * kHeadDim + 32 * u + (low ? 16 : 0));
#pragma unroll
      for (int c4 = 0; c4 < 4; ++c4) {
        const float4 x = qrow[c4];
        q16[4 * c4] = x.x * qs;
        q16[4 * c4 + 1] = x.y * qs;
        q16[4 * c4 + 2] = x.z * qs;
        q16[4 * c4 + 3] = x.w * qs;
      }
    }
    const int64_t n_groups = n_main / kGroup;
    const int64_t g0 = int64_t(split) * a.tiles_per_split;
    const int64_t g1 = min(g0 + int64_t(a.tiles_per_split), n_groups);
    const uint32_t n_blk = g1 > g0 ? uint32_t(g1 - g0) : 0u;   // tiles of this split
    // Group i of this wavefront (the i-th tile it takes) sits in stage
    // i % kDepth. Loads run kAhead groups ahead; group i + kAhead refills the
    // stage of group i - 2, whose value products ran in the previous
    // iteration. n_mine, the wavefront's group count, is known once a take
    // comes back empty (-1 until then).
    constexpr int kAhead = kDepth - 2;
    const uint32_t v16 = 16u * lane, h16 = 16u * (lane & 31), h4 = 4u * (lane & 31);
    uint8_t* ring_w = &ring[wave][0][0];
    // the next tile of the split, or n_blk and above when none is left:
    // from the shared counter (unit-sized workgroups; four-wavefront ones
    // share a unit with others, so balancing inside them gains little), or
    // wave, wave + NW, ... in fixed order
    constexpr bool kShare = UNIT;
    uint32_t taken = 0;
    // GRP: the counter and the fixed order hand out K groups, whose tiles the
    // wavefront then takes one by one (a split holds whole groups)
    auto take_unit = [&]() -> uint32_t {
      if (!kShare || a.fixed_order) return uint32_t(wave) + uint32_t(NW) * taken++;
      uint32_t t = 0;
      if (lane == 0) t = atomicAdd(&next_tile, 1u);
      return __builtin_amdgcn_readfirstlane(t);
    };
    const uint32_t gs_mask = GRP ? (1u << a.gshift) - 1u : 0u;   // tiles per K group - 1
    uint32_t grp_next = 0;                                        // GRP: next tile to hand out
    auto take = [&]() -> uint32_t {
      if constexpr (GRP) {
        if ((grp_next & gs_mask) == 0) grp_next = take_unit() << a.gshift;
        return grp_next++;
      }
      return take_unit();
    };
    // The wavefront's i-th tile is the first of its K group when i is a
    // multiple of G / 32 (it takes whole groups, in order). Its operands are
    // built from the stage before the iteration's other LDS reads, while the
    // previous tile's V codes are not yet in registers.
    GroupQ Qg;
    auto group_ops = [&](const uint8_t* st, int idx) {
      if constexpr (GRP) {
        if ((uint32_t(idx) & gs_mask) == 0) {
          KLoad<BITS, NVS> KS;
          load_kscale<BITS, VB, NVS>(st, u, low, KS);
          group_q<BITS, NVS>(KS, q16, Qg);
        }
      }
    };
    // −m_ref enters each head's scores once: from every lane of part 0 when
    // the z-term is broadcast from one lane-group sum (G > 32), from lane
    // group 0 of part 0 when the matrix cores add the lane groups' partials
    const bool m_lane = GRP ? !low : (!low && u == 0);
    auto m_part_of = [&](float m_ref) -> float { return m_lane ? m_ref : 0.0f; };
    auto scores = [&](const KLoad<BITS, NVS>& K, float m_part, float (&sc_out)[4]) {
      if constexpr (GRP) tile_scores<BITS, NVS>(K, low, Qg, m_part, sc_out);
      else group_scores<BITS, NVS>(K, low, q16, m_part, sc_out);
    };
    int n_mine = -1;
#pragma unroll
    for (int j = 0; j < kAhead; ++j) {
      if (n_mine < 0) {
        const uint32_t t = take();
        if (t < n_blk) {
          issue_group<BITS, VB, NVS>(ring_w + j * S::kBytes, group_src<BITS, VB, NVS, PAGED>(a, bh, b, h_kv, g0 + t),
                                     v16, h16, h4);
        } else {
          n_mine = j;
        }
      }
    }
    // the last main split of (b, h) also takes the window, while the first
    // copies are in flight (its loads are ordinary ones, older than every
    // copy waited on below, so the counted waits still hold)
    if (split == win_split) run_window<NVS, NW>(a, W, bh, b, hq0, nh, hs, r, u, low, wave, n_win);
    if (n_mine != 0) {
      float sc[4];
      if (n_mine < 0) {
        const uint32_t t = take();
        if (t < n_blk) {
          issue_group<BITS, VB, NVS>(ring_w + kAhead * S::kBytes,
                                     group_src<BITS, VB, NVS, PAGED>(a, bh, b, h_kv, g0 + t), v16, h16, h4);
          wait_vmem<kAhead * S::kLoads>();
        } else {
          n_mine = kAhead;
        }
      }
      if (n_mine >= 0) wait_groups<BITS, VB, NVS>(n_mine - 1);
      KLoad<BITS, NVS> K;
      VLoad V;
      group_ops(ring_w, 0);
      load_k<BITS, VB, NVS>(ring_w, r, u, low, K, !GRP);
      scores(K, 0.0f, sc);
      u32x4 bp_prev[NVS];
      group_probs<BITS, false, NVS>(W, sc, K.vs, K.vz, bp_prev);
      int i = 1;
      // steady state: a group is loaded every iteration, one fixed wait,
      // until the split runs out of tiles; each iteration takes the tile of
      // the next one, so the counter's round trip overlaps the arithmetic
      uint32_t t_next = (KVQ_TAKE_AHEAD && n_mine < 0) ? take() : n_blk;
      // One steady-state iteration for group i, whose stage i % kDepth is the
      // compile-time PH: every LDS address of the ring is then a constant
      // offset from the wavefront's ring base. Returns false once the split
      // has no tile left (n_mine is then known).
      auto step = [&](auto ph) -> bool {
        constexpr int PH = decltype(ph)::value;
        // the refilled stage was last read two groups ago; its reads are done
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
        if (!KVQ_TAKE_AHEAD) t_next = take();
        if (t_next >= n_blk) {
          n_mine = i + kAhead;
          return false;
        }
        issue_group<BITS, VB, NVS>(ring_w + ((PH + kAhead) % kDepth) * S::kBytes,
                                   group_src<BITS, VB, NVS, PAGED>(a, bh, b, h_kv, g0 + t_next),
                                   v16, h16, h4);
        wait_vmem<kAhead * S::kLoads>();
        group_ops(ring_w + PH * S::kBytes, i);
        load_v<BITS, VB, NVS>(ring_w + ((PH + kDepth - 1) % kDepth) * S::kBytes, r, u, V);
        load_k<BITS, VB, NVS>(ring_w + PH * S::kBytes, r, u, low, K, !GRP);
        if (KVQ_TAKE_AHEAD) t_next = take();
        // keep every LDS read of the iteration ahead of the arithmetic
        __builtin_amdgcn_sched_barrier(0);
        scores(K, m_part_of(W.m_ref), sc);
        group_values<VB, NVS>(V, W, bp_prev, vsh, vm0, vm1, magic, magic32);
        group_probs<BITS, true, NVS>(W, sc, K.vs, K.vz, bp_prev);
        ++i;
        return true;
      };
      // group 1 is in stage 1: the stages then follow 2, .., kDepth - 1, 0, 1, ..
      if (n_mine < 0) {
        using std::integral_constant;
        if constexpr (kDepth == 3) {
          while (step(integral_constant<int, 1>{}) && step(integral_constant<int, 2>{}) &&
                 step(integral_constant<int, 0>{})) {
          }
        } else {
          while (step(integral_constant<int, 1>{}) && step(integral_constant<int, 2>{}) &&
                 step(integral_constant<int, 3>{}) && step(integral_constant<int, 0>{})) {
          }
        }
      }
      // the last kAhead groups (fewer for a wavefront with fewer groups):
      // nothing left to load
      for (; i < n_mine; ++i) {
        wait_groups<BITS, VB, NVS>(n_mine - 1 - i);
        group_ops(ring_w + (i % kDepth) * S::kBytes, i);
        load_v<BITS, VB, NVS>(ring_w + ((i - 1) % kDepth) * S::kBytes, r, u, V);
        load_k<BITS, VB, NVS>(ring_w + (i % kDepth) * S::kBytes, r, u, low, K, !GRP);
        // keep every LDS read of the iteration ahead of the arithmetic
        __builtin_amdgcn_sched_barrier(0);
        scores(K, m_part_of(W.m_ref), sc);
        group_values<VB, NVS>(V, W, bp_prev, vsh, vm0, vm1, magic, magic32);
        group_probs<BITS, true, NVS>(W, sc, K.vs, K.vz, bp_prev);
      }
      load_v<BITS, VB, NVS>(ring_w + ((n_mine - 1) % kDepth) * S::kBytes, r, u, V);
      group_values<VB, NVS>(V, W, bp_prev, vsh, vm0, vm1, magic, magic32);
    }
  } else {
    run_window<NVS, NW>(a, W, bh, b, hq0, nh, hs, r, u, low, wave, n_win);
  }

  wave_epilogue_and_merge<NVS, NW>(a, W, &ring[0][0][0], sizeof(ring[0]), wave, lane, hs, u,
                                   low, tid, b, hq0, nh, split, 1.0f);
}

// ===================================================================== FP8 / FP16
// Decode over the FP8 and FP16 caches ("大模型量化从0到1（十三）：KV Cache 量化", §二
// and §十 FP8 formula: x̂ = fp8_value(code) · s, s per tensor or per KV head
// as in §十八.6), same split-K structure and online softmax as the KIVI
// kernel, 32-token tiles streamed through an LDS ring. K rows [CT][D] and V
// tiles [D][32] enter the f16 matrix cores directly (E4M3 codes through the
// exact E4M3 → fp16 scaled conversion; an E5M2 code is the high byte of the
// fp16 of the same value, placed there by a byte permute): scores A = K rows,
// B = q·log2(e)/√D (·s_K) as a constant fp16 high/low pair; values A = V tile
// rows, B = p as an fp16 high/low pair, so p must stay below fp16's maximum:
// the reference maximum is raised when a score exceeds it by 14 (p ≤ 2^14).
// s_V scales the output at the end.
// In the FP8 domain (§十八.7) the query is quantized to E4M3 per head inside
// the launch (the encoder of kvq_quantize_query_fp8) and B = the query codes'
// values, exact in fp16 (no high/low split: both B columns of a head carry the
// same values, so each lane's own column is the whole score); s_q·s_K·log2e/√D
// scales the fp32 result. The fp8 × fp8 products go to the f16 matrix cores,
// where they are exact and their fp32 sums keep full precision: the FP8
// matrix cores sum each run of 8 products aligned to the largest and drop
// bits about 12 binary places below it (measured), and the decode is
// memory-bound, so they would cost accuracy for no time.

constexpr float kLazyDense = 14.0f;

template <int SRC>
struct DenseStage {
  static constexpr int kElem = SRC == kSrcFp16 ? 2 : 1;
  static constexpr int kRows = kGroup * kHeadDim * kElem;   // K rows (= V tile) of a tile
  static constexpr int kBytes = 2 * kRows;
  static constexpr int kDepth = 2;                          // stages per wavefront
  static constexpr int kLoads = kBytes / 1024;              // copies per tile
};

// one 16-byte-per-lane copy (1 KiB per wavefront), M0 saved and restored
__device__ __forceinline__ void dma_kib(void* lds, const void* base, uint32_t voff) {
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\ts_mov_b32 m0, %1\n\ts_nop 0\n\t"
      "global_load_lds_dwordx4 %2, %3 nt\n\ts_mov_b32 m0, %0"
      : "=&s"(saved) : "s"(lds_addr(lds)), "v"(voff), "s"(base) : "memory");
}

template <int SRC>
__device__ __forceinline__ void issue_tile(uint8_t* st, const DecodeArgs& a, int bh, int64_t tile,
                                           uint32_t v16) {
  using S = DenseStage<SRC>;
  const uint8_t* kr = static_cast<const uint8_t*>(a.k_main) +
                      (int64_t(bh) * a.main_bh_tokens + tile * kGroup) * kHeadDim * S::kElem;
  const uint8_t* vt = static_cast<const uint8_t*>(a.v_main) +
                      (int64_t(bh) * a.NT + tile) * int64_t(S::kRows);
#pragma unroll
  for (int c = 0; c < S::kRows / 1024; ++c) {
    dma_kib(st + 1024 * c, kr + 1024 * c, v16);
    dma_kib(st + S::kRows + 1024 * c, vt + 1024 * c, v16);
  }
}

// fp16 pair from two E4M3 bytes (half-word `high` of w), exact
__device__ __forceinline__ uint32_t e4m3x2_to_f16x2(uint32_t w, bool high) {
  typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
  const f16x2 r = high ? __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 1.0f, true)
                       : __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 1.0f, false);
  return __builtin_bit_cast(uint32_t, r);
}

// fp16 pair from two E5M2 bytes (half-word `high` of w), exact: each byte
// becomes the high byte of its fp16 (selector 0x0C gives a zero byte)
__device__ __forceinline__ uint32_t e5m2x2_to_f16x2(uint32_t w, bool high) {
  return __builtin_amdgcn_perm(0u, w, high ? 0x030C020Cu : 0x010C000Cu);
}

template <int SRC>
__device__ __forceinline__ uint32_t fp8x2_to_f16x2(uint32_t w, bool high) {
  return SRC == kSrcE5M2 ? e5m2x2_to_f16x2(w, high) : e4m3x2_to_f16x2(w, high);
}

// fp16 high / low terms of four p values; part 0 ends with the high terms of
// tile 0 (own) and tile 1 (partner's), part 1 with the low terms of tile 0
// (partner's) and tile 1 (own).
__device__ __forceinline__ u32x4 p_operand_f16(const float (&pp)[4]) {
  uint32_t hp[2], lp[2];
  split_pair(pp[0], pp[1], hp[0], lp[0]);
  split_pair(pp[2], pp[3], hp[1], lp[1]);
  swap_halves2(hp, lp);
  return u32x4{hp[0], hp[1], lp[0], lp[1]};
}

template <int SRC, bool QF8>
__device__ __forceinline__ void process_dense_tile(const uint8_t* st, WaveAcc& W, int n_in,
                                                   const u32x4 (&bq)[4], float smul, int r,
                                                   int u, bool low) {
  using S = DenseStage<SRC>;
  // ---- scores
  f32x4 s0 = f32x4{0.f, 0.f, 0.f, 0.f}, s1 = s0;
#pragma unroll
  for (int sl = 0; sl < 4; ++sl) {
    u32x4 a0, a1;
    if (SRC == kSrcFp16) {
      const uint4 x = *reinterpret_cast<const uint4*>(st + (r * kHeadDim + 32 * sl + 8 * u) * 2);
      const uint4 y =
          *reinterpret_cast<const uint4*>(st + ((16 + r) * kHeadDim + 32 * sl + 8 * u) * 2);
      a0 = u32x4{x.x, x.y, x.z, x.w};
      a1 = u32x4{y.x, y.y, y.z, y.w};
    } else {
      const uint2 x = *reinterpret_cast<const uint2*>(st + r * kHeadDim + 32 * sl + 8 * u);
      const uint2 y = *reinterpret_cast<const uint2*>(st + (16 + r) * kHeadDim + 32 * sl + 8 * u);
      a0 = u32x4{fp8x2_to_f16x2<SRC>(x.x, false), fp8x2_to_f16x2<SRC>(x.x, true),
                 fp8x2_to_f16x2<SRC>(x.y, false), fp8x2_to_f16x2<SRC>(x.y, true)};
      a1 = u32x4{fp8x2_to_f16x2<SRC>(y.x, false), fp8x2_to_f16x2<SRC>(y.x, true),
                 fp8x2_to_f16x2<SRC>(y.y, false), fp8x2_to_f16x2<SRC>(y.y, true)};
    }
    s0 = __builtin_amdgcn_mfma_f32_16x16x32_f16(as_f16x8(a0), as_f16x8(bq[sl]), s0, 0, 0, 0);
    s1 = __builtin_amdgcn_mfma_f32_16x16x32_f16(as_f16x8(a1), as_f16x8(bq[sl]), s1, 0, 0, 0);
  }
  float sc[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    // the cross-lane add runs in every lane; tokens past n_in are masked after;
    // smul undoes the normalisation of the score operand (a power of two), or
    // applies s_q·s_K·log2e/√D in the FP8 domain, where columns r and r + 8
    // both hold head hs: lane r (part 0) has tile 0's scores, lane r + 8 tile 1's
    const float t0 = (QF8 ? s0[i] : s0[i] + xor8(s0[i])) * smul;
    const float t1 = (QF8 ? s1[i] : s1[i] + xor8(s1[i])) * smul;
    const int t = (low ? 16 : 0) + 4 * u + i;
    sc[i] = t < n_in ? (low ? t1 : t0) : -INFINITY;
  }
  rescale_if_needed(W, sc, kLazyDense);
  float pp[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    pp[i] = fast_exp2(sc[i] - W.m_ref);       // 0 for masked tokens
    W.l_acc += pp[i];
  }
  const u32x4 bp = p_operand_f16(pp);
  // ---- values: row 16n + r of the V tile, tokens 4u..4u+3 and 16+4u..16+4u+3
  const uint8_t* vt = st + S::kRows;
#pragma unroll
  for (int n = 0; n < 8; ++n) {
    u32x4 av;
    if (SRC == kSrcFp16) {
      const uint8_t* row = vt + (16 * n + r) * kGroup * 2;
      const uint2 x = *reinterpret_cast<const uint2*>(row + 8 * u);
      const uint2 y = *reinterpret_cast<const uint2*>(row + 32 + 8 * u);
      av = u32x4{x.x, x.y, y.x, y.y};
    } else {
      const uint8_t* row = vt + (16 * n + r) * kGroup;
      const uint32_t x = *reinterpret_cast<const uint32_t*>(row + 4 * u);
      const uint32_t y = *reinterpret_cast<const uint32_t*>(row + 16 + 4 * u);
      av = u32x4{fp8x2_to_f16x2<SRC>(x, false), fp8x2_to_f16x2<SRC>(x, true),
                 fp8x2_to_f16x2<SRC>(y, false), fp8x2_to_f16x2<SRC>(y, true)};
    }
    W.cv[n] = __builtin_amdgcn_mfma_f32_16x16x32_f16(as_f16x8(av), as_f16x8(bp), W.cv[n], 0, 0, 0);
  }
}

// Wavefronts of a dense decode workgroup. UNIT (FP8 caches, tiles shared,
// chosen only when the cache is not deterministic): the whole compute unit in
// one workgroup, two wavefronts per SIMD on two 8 KiB stages each; otherwise
// four wavefronts with a fixed tile order (the FP16 caches' 16 KiB stages fit
// no more). Same-box A/B of the 128K FP8 decode: the unit shape with shared
// tiles 2-4 % faster, with a fixed order 7-8 % slower.
template <int SRC, bool UNIT>
constexpr int dense_waves() { return (UNIT && SRC != kSrcFp16) ? 8 : 4; }

template <int SRC, bool QF8, bool UNIT>
__global__ __launch_bounds__((64 * dense_waves<SRC, UNIT>())) void dense_mfma_split_kernel(DecodeArgs a) {
  using S = DenseStage<SRC>;
  constexpr int NW = dense_waves<SRC, UNIT>();
  __shared__ __attribute__((aligned(16))) uint8_t ring[NW][S::kDepth][S::kBytes];
  __shared__ uint32_t next_tile;   // tiles of this split handed out so far

  const BlockCoord bc = block_coord(a);
  const int split = bc.split;
  const int bh = bc.bh;
  const int b = bh / a.H;
  const int h_kv = bh % a.H;
  const int hq0 = h_kv * a.nq + bc.chunk * a.heads_per_chunk;
  const int nh = min(a.heads_per_chunk, a.nq - bc.chunk * a.heads_per_chunk);
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int r = lane & 15;
  const int u = lane >> 4;
  const int hs = r & 7;
  const bool low = r >= 8;

  // FP8: the scale row of the tensor, or of this KV head
  const float sk = SRC != kSrcFp16 ? a.tensor_scale[a.scale_stride * h_kv] : 1.0f;
  const float sv = SRC != kSrcFp16 ? a.tensor_scale[a.scale_stride * h_kv + 1] : 1.0f;
  // B of the scores: q·log2e/√D (·s_K) as fp16 high (part 0) / low (part 1)
  // terms, channel 32s + 8u + j in k-step s. An FP8 scale can be small enough
  // (amax / 57344 for E5M2, or a narrow head's scale) to push these terms
  // into fp16's subnormal range, so for FP8 the factor log2e/√D·s_K = m·2^e
  // enters B as its mantissa m ∈ [0.5, 1) and the scores are multiplied by
  // 2^e afterwards (both steps exact).
  float smul = 1.0f, qfac = a.qscale;
  if (SRC != kSrcFp16) {
    int e;
    qfac = frexpf(a.qscale * sk, &e);
    smul = ldexpf(1.0f, e);
  }
  u32x4 bq[4];
  if constexpr (QF8) {
    // the query row of head hs as E4M3 codes, channel 32s + 8u + j in k-step s
    // (byte j); lanes r and r + 8 build the same operand
    const bool valid = hs < nh;
    const float* qrow = a.q + (int64_t(b) * a.Hq + hq0 + (valid ? hs : 0)) * kHeadDim;
    float x[32];
    float amax = 0.0f;
#pragma unroll
    for (int sl = 0; sl < 4; ++sl) {
      const float4 x0 = *reinterpret_cast<const float4*>(qrow + 32 * sl + 8 * u);
      const float4 x1 = *reinterpret_cast<const float4*>(qrow + 32 * sl + 8 * u + 4);
      const float xs[8] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w};
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        x[8 * sl + j] = valid ? xs[j] : 0.0f;
        amax = fmaxf(amax, fabsf(x[8 * sl + j]));
      }
    }
    amax = max_x16_x32(amax);                    // the row's four lane groups u
    const float sq = amax / kFp8Max<kE4M3>;
    const float rs = sq != 0.0f ? 1.0f / sq : 0.0f;
    const bool tiny = sq < kTinyQueryScale;
#pragma unroll
    for (int sl = 0; sl < 4; ++sl) {
      uint32_t w[2] = {0u, 0u};
      if (sq != 0.0f) {
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const float* xx = x + 8 * sl + 4 * h;
          w[h] = fp8_pack2<kE4M3>(query_quotient(xx[0], sq, rs, tiny),
                                  query_quotient(xx[1], sq, rs, tiny), 0u, false);
          w[h] = fp8_pack2<kE4M3>(query_quotient(xx[2], sq, rs, tiny),
                                  query_quotient(xx[3], sq, rs, tiny), w[h], true);
        }
      }
      bq[sl] = u32x4{e4m3x2_to_f16x2(w[0], false), e4m3x2_to_f16x2(w[0], true),
                     e4m3x2_to_f16x2(w[1], false), e4m3x2_to_f16x2(w[1], true)};
    }
    smul = sq * sk * a.qscale;
  } else {
    const bool valid = hs < nh;
    const float qs = valid ? qfac : 0.0f;
    const float* qrow = a.q + (int64_t(b) * a.Hq + hq0 + (valid ? hs : 0)) * kHeadDim;
#pragma unroll
    for (int sl = 0; sl < 4; ++sl) {
      uint32_t d[4];
#pragma unroll
      for (int p = 0; p < 4; ++p) {
        uint32_t hi, lo;
        split_pair(qrow[32 * sl + 8 * u + 2 * p] * qs, qrow[32 * sl + 8 * u + 2 * p + 1] * qs,
                   hi, lo);
        d[p] = low ? lo : hi;
      }
      bq[sl] = u32x4{d[0], d[1], d[2], d[3]};
    }
  }

  WaveAcc W;
  W.m_ref = -INFINITY;
  W.l_acc = 0.0f;
  W.pz_acc[0] = 0.0f;
#pragma unroll
  for (int n = 0; n < 8; ++n) W.cv[n] = f32x4{0.f, 0.f, 0.f, 0.f};
  W.cones[0] = f32x4{0.f, 0.f, 0.f, 0.f};

  if (tid == 0) next_tile = 0;
  __syncthreads();
  const int64_t n_tiles = (a.n_main + kGroup - 1) / kGroup;
  const int64_t g0 = int64_t(split) * a.tiles_per_split;
  const int64_t g1 = min(g0 + int64_t(a.tiles_per_split), n_tiles);
  const uint32_t n_blk = g1 > g0 ? uint32_t(g1 - g0) : 0u;   // tiles of this split
  static_assert(S::kDepth == 2, "one tile in flight ahead of the one in work");
  const uint32_t v16 = 16u * lane;
  uint8_t* ring_w = &ring[wave][0][0];
  // the next tile of the split (n_blk and above: none left), from the shared
  // counter (UNIT) or in fixed order wave, wave + NW, ...
  uint32_t taken = 0;
  auto take = [&]() -> uint32_t {
    if (!UNIT) return uint32_t(wave) + uint32_t(NW) * taken++;
    uint32_t t = 0;
    if (lane == 0) t = atomicAdd(&next_tile, 1u);
    return __builtin_amdgcn_readfirstlane(t);
  };
  // tile i of this wavefront sits in stage i % 2; cur: the tile in work,
  // t_next: the one after it (taken a tile ahead)
  const uint32_t t0 = take();
  bool have = t0 < n_blk;
  int64_t cur = g0 + t0;
  if (have) issue_tile<SRC>(ring_w, a, bh, cur, v16);
  uint32_t t_next = have ? take() : n_blk;
  for (int i = 0; have; ++i) {
    const bool more = t_next < n_blk;
    const int64_t nxt = g0 + t_next;
    if (more) {
      // the refilled stage was read by the previous tile; its reads are done
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
      issue_tile<SRC>(ring_w + ((i + 1) % S::kDepth) * S::kBytes, a, bh, nxt, v16);
      wait_vmem<S::kLoads>();
      t_next = take();
    } else {
      wait_vmem<0>();
    }
    const int n_in = int(min<int64_t>(kGroup, a.n_main - cur * kGroup));
    process_dense_tile<SRC, QF8>(ring_w + (i % S::kDepth) * S::kBytes, W, n_in, bq, smul, r,
                                 u, low);
    have = more;
    cur = nxt;
  }

  wave_epilogue_and_merge<1, NW>(a, W, &ring[0][0][0], sizeof(ring[0]), wave, lane, hs, u, low,
                                 tid, b, hq0, nh, split, sv);
}

}  // namespace

template <int SRC, bool QF8>
static void launch_dense_shape(const DecodeArgs& a, dim3 grid, hipStream_t s) {
  if (a.unit)
    dense_mfma_split_kernel<SRC, QF8, true><<<grid, 64 * dense_waves<SRC, true>(), 0, s>>>(a);
  else
    dense_mfma_split_kernel<SRC, QF8, false><<<grid, 64 * dense_waves<SRC, false>(), 0, s>>>(a);
}

hipError_t launch_dense_mfma(const DecodeArgs& a, hipStream_t s) {
  const dim3 grid = split_grid(a);
  if (a.src == kSrcFp16) {
    dense_mfma_split_kernel<kSrcFp16, false, false><<<grid, 64 * dense_waves<kSrcFp16, false>(), 0, s>>>(a);
  } else if (a.src == kSrcE5M2) {
    if (a.qfp8) launch_dense_shape<kSrcE5M2, true>(a, grid, s);
    else launch_dense_shape<kSrcE5M2, false>(a, grid, s);
  } else {
    if (a.qfp8) launch_dense_shape<kSrcFp8, true>(a, grid, s);
    else launch_dense_shape<kSrcFp8, false>(a, grid, s);
  }
  return hipGetLastError();
}

// launches the (K bits, V bits) instance with NVS V scales per token, in the
// workgroup shape a.unit selects
template <int KB, int VB, int NVS, bool PAGED, bool GRP>
static void launch_kivi_paging(const DecodeArgs& a, dim3 grid, hipStream_t s) {
  if (a.unit)
    kivi_mfma_split_kernel<KB, VB, NVS, true, PAGED, GRP>
        <<<grid, 64 * kivi_waves<KB, VB, NVS, true>(), 0, s>>>(a);
  else
    kivi_mfma_split_kernel<KB, VB, NVS, false, PAGED, GRP>
        <<<grid, 64 * kivi_waves<KB, VB, NVS, false>(), 0, s>>>(a);
}
// Contiguous caches with G > 32 and one V scale per token keep each K
// group's score operands across its tiles (the split plan holds whole groups).
template <int KB, int VB, int NVS>
static void launch_kivi_shape(const DecodeArgs& a, dim3 grid, hipStream_t s) {
  if (a.paged) {
    launch_kivi_paging<KB, VB, NVS, true, false>(a, grid, s);
    return;
  }
  if constexpr (NVS == 1) {
    if (a.gshift > 0) {
      launch_kivi_paging<KB, VB, NVS, false, true>(a, grid, s);
      return;
    }
  }
  launch_kivi_paging<KB, VB, NVS, false, false>(a, grid, s);
}
template <int NVS>
static hipError_t launch_kivi_nvs(const DecodeArgs& a, dim3 grid, hipStream_t s) {
  if (a.kbits == 2 && a.vbits == 2) launch_kivi_shape<2, 2, NVS>(a, grid, s);
  else if (a.kbits == 4 && a.vbits == 4) launch_kivi_shape<4, 4, NVS>(a, grid, s);
  else if (a.kbits == 4 && a.vbits == 2) launch_kivi_shape<4, 2, NVS>(a, grid, s);
  else if (a.kbits == 2 && a.vbits == 4) launch_kivi_shape<2, 4, NVS>(a, grid, s);
  else return hipErrorInvalidValue;
  return hipGetLastError();
}

// Resident workgroups per compute unit of each split-kernel instance, found
// once per process (all instances are fixed at build time; 0 = not yet known).
template <typename Kernel>
static int blocks_per_cu(Kernel kernel, std::atomic<int>& slot, int threads = kThreads) {
  int n = slot.load(std::memory_order_relaxed);
  if (n > 0) return n;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, kernel, threads, 0) != hipSuccess || n <= 0)
    return 0;
  slot.store(n, std::memory_order_relaxed);
  return n;
}

// (the paged instances have the same occupancy: both are built for the same
// wavefronts per SIMD, and a kernel that would spill fails the build)
template <int KB, int VB, int NVS>
static int kivi_blocks_per_cu(bool unit, std::atomic<int>* slot) {
  return unit ? blocks_per_cu(kivi_mfma_split_kernel<KB, VB, NVS, true, false>, slot[1],
                              64 * kivi_waves<KB, VB, NVS, true>())
              : blocks_per_cu(kivi_mfma_split_kernel<KB, VB, NVS, false, false>, slot[0],
                              64 * kivi_waves<KB, VB, NVS, false>());
}

template <int SRC, bool QF8>
static int dense_blocks_per_cu(bool unit, std::atomic<int>* slot) {
  return unit ? blocks_per_cu(dense_mfma_split_kernel<SRC, QF8, true>, slot[1],
                              64 * dense_waves<SRC, true>())
              : blocks_per_cu(dense_mfma_split_kernel<SRC, QF8, false>, slot[0],
                              64 * dense_waves<SRC, false>());
}

int device_compute_units() {
  // per device, queried once (a fixed property of the device)
  static std::atomic<int> known[64];
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 0;
  if (dev >= 0 && dev < 64 && (cus = known[dev].load(std::memory_order_relaxed)) > 0) return cus;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
    return 0;
  if (dev >= 0 && dev < 64 && cus > 0) known[dev].store(cus, std::memory_order_relaxed);
  return cus;
}

int decode_resident_workgroups(const DecodeArgs& a) {
  static std::atomic<int> slots[32];
  int per_cu = 0;
  switch (a.src) {
    case kSrcKivi2:
    case kSrcKivi4: {
      if (a.nvs != 1 && a.nvs != 4) return 0;
      const int k = (a.kbits == 4 ? 1 : 0) + (a.vbits == 4 ? 2 : 0) + (a.nvs == 4 ? 4 : 0);
      std::atomic<int>* slot = &slots[16 + 2 * k];
      const bool u = a.unit != 0;
      switch (k) {
        case 0: per_cu = kivi_blocks_per_cu<2, 2, 1>(u, slot); break;
        case 1: per_cu = kivi_blocks_per_cu<4, 2, 1>(u, slot); break;
        case 2: per_cu = kivi_blocks_per_cu<2, 4, 1>(u, slot); break;
        case 3: per_cu = kivi_blocks_per_cu<4, 4, 1>(u, slot); break;
        case 4: per_cu = kivi_blocks_per_cu<2, 2, 4>(u, slot); break;
        case 5: per_cu = kivi_blocks_per_cu<4, 2, 4>(u, slot); break;
        case 6: per_cu = kivi_blocks_per_cu<2, 4, 4>(u, slot); break;
        default: per_cu = kivi_blocks_per_cu<4, 4, 4>(u, slot); break;
      }
      break;
    }
    case kSrcFp16:
      per_cu = blocks_per_cu(dense_mfma_split_kernel<kSrcFp16, false, false>, slots[8],
                             64 * dense_waves<kSrcFp16, false>());
      break;
    case kSrcFp8:
      per_cu = a.qfp8 ? dense_blocks_per_cu<kSrcFp8, true>(a.unit != 0, &slots[0])
                      : dense_blocks_per_cu<kSrcFp8, false>(a.unit != 0, &slots[2]);
      break;
    case kSrcE5M2:
      per_cu = a.qfp8 ? dense_blocks_per_cu<kSrcE5M2, true>(a.unit != 0, &slots[4])
                      : dense_blocks_per_cu<kSrcE5M2, false>(a.unit != 0, &slots[6]);
      break;
    default:
      return 0;
  }
  if (per_cu <= 0) return 0;
  const int cus = device_compute_units();
  return cus > 0 ? cus * per_cu : 0;
}

hipError_t launch_kivi_mfma(const DecodeArgs& a, hipStream_t s) {
  const dim3 grid = split_grid(a);
  if (a.nvs == 1) return launch_kivi_nvs<1>(a, grid, s);
  if (a.nvs == 4) return launch_kivi_nvs<4>(a, grid, s);
  return hipErrorInvalidValue;
}

}  // namespace kvq
