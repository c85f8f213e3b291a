// kvq_quant_kivi.hip — KIVI group quantization for gfx950 (prefill and window
// flush).
//
// KIVI ("4.4 KV Cache 量化：KIVI 2-bit 与 FP8 KV Cache", §2 and §3.2;
// "大模型量化从0到1（十三）：KV Cache 量化", §九 and the affine formula of §十):
// K gets one (scale, zero) per (group of G tokens, channel), V one per token.
// Quantizer, each op in fp32 and correctly rounded (no contraction; the
// library is built with -ffp-contract=off):
//   s = (max − min) / (2^b − 1), z = min,
//   code = clamp(rint((x − min) / s), 0, 2^b − 1), code = 0 when s == 0.
//
// Built with the IEEE mode bit off (-mno-amdgpu-ieee, which needs
// -fno-honor-nans): fp16 min / max then take their operands as they are,
// where IEEE mode makes the compiler quiet each loaded or lane-moved value
// first (one extra packed max per value). Results on finite inputs are the
// same; NaN inputs give unspecified codes. Work-group and work-item ids come
// from the builtins: the device library's id functions carry the IEEE mode
// attribute and would no longer inline.
#include <hip/hip_fp16.h>
#include <hip/hip_runtime.h>

#include "kvq_internal.h"
#include "kvq_quant_common.h"

namespace kvq {
namespace {

constexpr int kThreads = 256;

__device__ __forceinline__ uint32_t affine_code(float x, float mn, float s, float qmax) {
  if (s == 0.0f) return 0u;
  float r = rintf((x - mn) / s);
  r = fminf(fmaxf(r, 0.0f), qmax);
  return static_cast<uint32_t>(r);
}

__device__ __forceinline__ float f4c(float4 v, int c) {
  return c == 0 ? v.x : c == 1 ? v.y : c == 2 ? v.z : v.w;
}

// ---- fast exact quotient. The code is rint(q), q = RN(RN(x − min) / s), with
// x and min fp16 values. The kernel takes p = RN(x·r + n) in one fma, with r
// within about an ulp of 1/s and n = RN(−min·r), per channel (K) or token (V).
// Against the real quotient Q = RN(x − min) / s ≤ 2^b − 1 < 16, the errors are
// r's (2⁻²³·Q), the rounding of x − min that the fma does not make (2⁻²⁴·Q),
// the fma's own rounding (2⁻²⁴·Q) and n's rounding (2⁻²⁴·|min·r|); with q's
// own 2⁻²⁴·Q, |p − q| < 1.25·2⁻²²·Q + 2⁻²⁴·|min·r| < 2⁻¹⁶ + 2⁻²³·|n|. Unless
// p lies that close to a half-integer (a possible rounding tie), rint(p) is
// the code; the rare lanes with such a value redo those values' codes with
// the correctly rounded division. The edge below is the threshold on
// |p − rint(p)| for n = 0, less 2⁻²³·|n| per channel block (K) or token (V).
// When min·r is large against the codes (a group far from zero with a tiny
// range) every value takes the division, which is still exact.
constexpr float kTieEdge = 0.5f - 1.0f / 65536.0f;
__device__ __forceinline__ float tie_edge(float n_abs) { return kTieEdge - n_abs * 0x1p-23f; }

// 1/s to within about an ulp (one Newton step on the hardware estimate);
// 0 when s == 0, which makes every code 0 as the quantizer requires.
__device__ __forceinline__ float quant_recip(float s) {
  if (s == 0.0f) return 0.0f;
  const float r = __builtin_amdgcn_rcpf(s);
  return fmaf(r, fmaf(-s, r, 1.0f), r);
}

// rint(x·r + n) as a float (0 ≤ code ≤ 2^b − 1); `dev` keeps the largest
// |p − rint(p)| seen, so that dev above the edge flags a possible rounding tie.
__device__ __forceinline__ float fast_code(float x, float r, float n, float& dev) {
  const float p = fmaf(x, r, n);
  const float c = rintf(p);
  dev = fmaxf(dev, fabsf(p - c));
  return c;
}

// x / d correctly rounded, for d = 3 or 15 (2^b − 1 at b = 2, 4): q = RN(x·y)
// with y = RN(1/d) is within an ulp of the quotient, the remainder x − q·d is
// exact in one fma, and one more fma of it with y gives RN(x / d). Equal bit
// for bit to the IEEE division for every finite fp32 x of either sign, for
// both d (a host check runs every pattern of the binades where the steps do
// not scale by powers of two and of one middle binade); the one exception,
// x = −0 (where the correction gives +0), and non-finite x take q itself.
template <int D>
__device__ __forceinline__ float div_code_range(float x) {
  static_assert(D == 3 || D == 15, "code ranges of 2- and 4-bit codes");
  constexpr float y = 1.0f / float(D);
  const float q = x * y;
  const float r = fmaf(-q, float(D), x);
  const float c = fmaf(r, y, q);
  // class mask: NaN (bits 0, 1), ±inf (2, 9), ±0 (5, 6)
  return __builtin_amdgcn_classf(x, 0x267) ? q : c;
}

// pack 16 codes (floats 0..2^b−1) of consecutive channels into 32-bit words,
// channel i of a word at bits [b·i, b·i + b): 2 bits → 1 word, 4 bits → 2.
template <int BITS>
__device__ __forceinline__ void pack16(const float (&c)[16], uint32_t (&w)[BITS / 2]) {
  constexpr int PER = 32 / BITS;
#pragma unroll
  for (int k = 0; k < BITS / 2; ++k) {
    // two exact float sums of 8 codes each (< 2^16), then one integer merge
    float lo = c[k * PER], hi = c[k * PER + PER / 2];
#pragma unroll
    for (int i = 1; i < PER / 2; ++i) {
      lo = fmaf(c[k * PER + i], float(1 << (BITS * i)), lo);
      hi = fmaf(c[k * PER + PER / 2 + i], float(1 << (BITS * i)), hi);
    }
    w[k] = static_cast<uint32_t>(lo) | (static_cast<uint32_t>(hi) << 16);
  }
}

// The appended token of (b, h) block bh into window slot `slot`: 16 threads
// copy K, 16 copy V (16 bytes each).
__device__ __forceinline__ void write_new_token(const KiviQuantArgs& a, int bh, int64_t slot,
                                                int tid) {
  if (tid >= 32) return;
  const int c = tid & 15;
  const __half* src = (tid < 16 ? a.k_new : a.v_new) + int64_t(bh) * kHeadDim + 8 * c;
  __half* dst = (tid < 16 ? a.k_win : a.v_win) + bh * a.win_bh_stride + slot * kHeadDim + 8 * c;
  *reinterpret_cast<uint4*>(dst) = *reinterpret_cast<const uint4*>(src);
}

// One workgroup quantizes one group of G = 32·NS tokens (NS sub-tiles of 32
// tokens × 128 channels) of K and of V for one (b, h). The group's K and V
// rows are copied into LDS first; thread (t = tid / 8, j = tid % 8) then takes
// channels [16j, 16j + 16) of token t of each sub-tile.
//   V (per token): min / max over the 8 threads of a token, or over the 2
//      threads of each run of 32 channels (packed fp16 max of (x, −x), DPP
//      exchanges), codes in registers, one word (two at 4
//      bits) of 16 channel codes per thread into an LDS transpose, from which
//      each thread assembles the sub-tile's V words along tokens.
//   K (per channel over the G tokens): wavefront w takes channels [32w, 32w + 32), lane (pair c = l % 16, quarter
//      u = l / 16) reduces rows [u·G/4, (u+1)·G/4) of channels 32w + 2c, +1
//      into LDS; wavefront 0 then combines the four quarters of every channel
//      pair and derives the per-channel scale and zero, from which the codes
//      of each thread's 16 channels follow.
template <int KB, int VB, int NS>
__global__ __launch_bounds__(kThreads) void kivi_quantize_kernel(KiviQuantArgs a) {
  constexpr int G = NS * kGroup;           // tokens per group
  constexpr int KPER = 32 / KB;            // K codes per 32-bit word
  constexpr int KW = kHeadDim / KPER;      // K words per token
  constexpr int KTW = KB / 2;              // words of one thread's 16 K codes
  constexpr float KQMAX = float((1 << KB) - 1);
  constexpr int VPER = 32 / VB;            // V codes per 32-bit word
  constexpr int VTR = kHeadDim / VPER;     // V transpose rows (words of a token's codes)
  constexpr int VW = kGroup / VPER;        // V words per (32-token tile, channel)
  constexpr int VTW = VB / 2;              // words of one thread's 16 V codes
  constexpr float VQMAX = float((1 << VB) - 1);
  constexpr int kRow = kGroup + 8;         // padded transpose row (words)

  __shared__ __attribute__((aligned(16))) __half tile_k[G][kHeadDim];
  // V rows in LDS too, up to G = 64 (at G = 128 the two tiles would halve
  // the workgroups a compute unit holds; V is then loaded per sub-tile)
  constexpr bool kVlds = NS <= 2;
  __shared__ __attribute__((aligned(16))) __half tile_v[kVlds ? G : 1][kHeadDim];
  __shared__ __attribute__((aligned(16))) float s_k[kHeadDim];
  __shared__ __attribute__((aligned(16))) float z_k[kHeadDim];
  __shared__ __attribute__((aligned(16))) float r_k[kHeadDim];
  __shared__ __attribute__((aligned(16))) float n_k[kHeadDim];       // RN(−min·r) per channel
  __shared__ float edge_k[kHeadDim / 16];                            // tie edge per 16 channels
  __shared__ __attribute__((aligned(16))) uint2 k_part[4][kHeadDim / 2];  // [quarter][pair] (max, min)
  __shared__ __attribute__((aligned(16))) uint32_t vt[NS][VTR][kRow];  // [sub][channel word][token]

  const int g = int(__builtin_amdgcn_workgroup_id_x());
  const int bh = int(__builtin_amdgcn_workgroup_id_y());
  const int tid = int(__builtin_amdgcn_workitem_id_x());
  const int t = tid >> 3;
  const int j = tid & 7;
  int64_t gg = a.g0 + g;                   // cache group
  int64_t new_slot = 0;                    // window slot of the appended token
  if (a.ragged) {                          // block-uniform: the whole block leaves
    const int b = bh / a.H;
    new_slot = a.seq.z[b];
    if (g >= a.seq.x[b]) {
      // a sequence that does not flush only takes the appended token
      if (g == 0 && a.k_new != nullptr) write_new_token(a, bh, new_slot, tid);
      return;
    }
    gg = int64_t(a.seq.y[b]) + g;
  }
  // destination (b, h) block of the cache arrays, and the group within it: a
  // paged cache's group lives in the (page, h) block of the page its
  // sequence's block table names for it (clamped into the pool)
  int64_t blk = bh;
  if (a.paged) {
    const int b = bh / a.H;
    const int h = bh - b * a.H;
    typedef __attribute__((address_space(4))) const int32_t ConstI32;   // scalar load
    const ConstI32* table = (const ConstI32*)(a.block_table);
    const int e = table[int64_t(b) * a.max_pages + (gg >> a.page_group_shift)];
    blk = int64_t(min(max(e, 0), a.num_pages - 1)) * a.H + h;
    gg &= (int64_t(1) << a.page_group_shift) - 1;
  }
  const int64_t CT = a.NG * G;             // token slots of one block

  // ---- the group's K rows (G·256 contiguous bytes), and its V rows up to
  // G = 64, straight into LDS: one copy instruction moves 1 KiB per
  // wavefront (16 bytes per lane), non-temporal since the inputs are read
  // once. This moves the kernel's bytes about 9 % faster than loads through
  // registers.
  uint4 vreg[kVlds ? 1 : NS][2];
  {
    const int wave = tid >> 6, lane = tid & 63;
    const int64_t base = bh * a.src_bh_stride + int64_t(g) * G * kHeadDim;
    const uint8_t* kg = reinterpret_cast<const uint8_t*>(a.k_src + base) + 16 * lane;
    const uint8_t* vg = reinterpret_cast<const uint8_t*>(a.v_src + base) + 16 * lane;
    uint8_t* lk = reinterpret_cast<uint8_t*>(&tile_k[0][0]);
    uint8_t* lv = reinterpret_cast<uint8_t*>(&tile_v[0][0]);
    constexpr int kKiB = G * kHeadDim * 2 / 1024;   // KiB of each tensor
    constexpr int kNonTemporal = 2;
#pragma unroll
    for (int c = 0; c < kKiB / 4; ++c) {
      const int kib = 4 * c + wave;
      __builtin_amdgcn_global_load_lds(kg + 1024 * kib, lk + 1024 * kib, 16, 0, kNonTemporal);
      if (kVlds) __builtin_amdgcn_global_load_lds(vg + 1024 * kib, lv + 1024 * kib, 16, 0, kNonTemporal);
    }
    // without the V tile in LDS, each thread's V values of every sub-tile go
    // to registers, in flight together with the K copies
    if constexpr (!kVlds) {
#pragma unroll
      for (int sub = 0; sub < NS; ++sub) {
        const __half* vsrc = a.v_src + bh * a.src_bh_stride +
                             (int64_t(g) * G + sub * kGroup + t) * kHeadDim + j * 16;
        vreg[sub][0] = *reinterpret_cast<const uint4*>(vsrc);
        vreg[sub][1] = *reinterpret_cast<const uint4*>(vsrc + 8);
      }
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  }
  __syncthreads();

#pragma unroll
  for (int sub = 0; sub < NS; ++sub) {
    const int tr = sub * kGroup + t;       // token row within the group
    uint4 v0, v1;
    if constexpr (kVlds) {
      v0 = *reinterpret_cast<const uint4*>(&tile_v[tr][j * 16]);
      v1 = *reinterpret_cast<const uint4*>(&tile_v[tr][j * 16 + 8]);
    } else {
      v0 = vreg[sub][0];
      v1 = vreg[sub][1];
    }

    // ---- V statistics: (max, max of −x) of the 16 values, then over the 8
    // threads of the token (xor 1, xor 2 inside a quad, then the half-row
    // mirror), or over the 2 threads of a run of 32 channels (xor 1) when V
    // has a scale per run (nvs = 4).
    const uint32_t vw[8] = {v0.x, v0.y, v0.z, v0.w, v1.x, v1.y, v1.z, v1.w};
    h2v mx2 = as_h2(vw[0]), mn2 = mx2;
#pragma unroll
    for (int i = 1; i < 8; ++i) {
      mx2 = h2max(mx2, as_h2(vw[i]));
      mn2 = h2min(mn2, as_h2(vw[i]));
    }
    // (max, −min) of the thread's 16 values in one fp16 pair
    h2v mm = h2max(h2v{mx2[0], -mn2[0]}, h2v{mx2[1], -mn2[1]});
    mm = h2max(mm, as_h2(uint32_t(__builtin_amdgcn_mov_dpp(int(as_u(mm)), 0xB1, 0xF, 0xF, false))));
    if (a.nvs == 1) {
      mm = h2max(mm, as_h2(uint32_t(__builtin_amdgcn_mov_dpp(int(as_u(mm)), 0x4E, 0xF, 0xF, false))));
      mm = h2max(mm, as_h2(uint32_t(__builtin_amdgcn_mov_dpp(int(as_u(mm)), 0x141, 0xF, 0xF, false))));
    }
    const float vmx = float(mm[0]);
    const float vmn = -float(mm[1]);
    const float vs = div_code_range<(1 << VB) - 1>(vmx - vmn);
    // one thread per token (nvs = 1) or per run of 32 channels (nvs = 4)
    if (a.nvs == 1 ? j == 0 : (j & 1) == 0) {
      const int64_t o = (blk * CT + gg * G + tr) * a.nvs + (a.nvs == 1 ? 0 : j / 2);
      store_nt(a.v_scale + o, vs);
      store_nt(a.v_zero + o, vmn);
    }

    // ---- V codes of the thread's 16 channels → the LDS transpose
    float vx[16], c[16];
    halves_to_float(v0, vx);
    halves_to_float(v1, vx + 8);
    const float vr = quant_recip(vs);
    const float vn = -(vmn * vr);
    const float vedge = tie_edge(fabsf(vn));
    float dev = 0.0f;
#pragma unroll
    for (int i = 0; i < 16; ++i) c[i] = fast_code(vx[i], vr, vn, dev);
    if (dev > vedge) {
      // a lane with a possible tie recomputes only the values that may sit on
      // one (the fast codes of the others are exact): a wavefront then runs
      // the division for the value slots where some lane has one
#pragma unroll
      for (int i = 0; i < 16; ++i)
        if (fabsf(fmaf(vx[i], vr, vn) - c[i]) > vedge)
          c[i] = float(affine_code(vx[i], vmn, vs, VQMAX));
    }
    uint32_t w[VTW];
    pack16<VB>(c, w);
#pragma unroll
    for (int k = 0; k < VTW; ++k) vt[sub][VTW * j + k][t] = w[k];
  }
  // ---- K statistics over the G rows, first half: lane (pair c = l % 16,
  // quarter u = l / 16) of wavefront w takes the minimum and maximum of rows
  // [u·G/4, (u+1)·G/4) of channels 32w + 2c and 32w + 2c + 1
  {
    const int wv = tid >> 6;
    const int c = tid & 15;
    const int u = (tid >> 4) & 3;
    const int d0 = 32 * wv + 2 * c;
    constexpr int kRowsPerQuarter = G / 4;
    h2v kmx = as_h2(*reinterpret_cast<const uint32_t*>(&tile_k[u * kRowsPerQuarter][d0])),
        kmn = kmx;
#pragma unroll
    for (int tt = 1; tt < kRowsPerQuarter; ++tt) {
      const h2v x = as_h2(*reinterpret_cast<const uint32_t*>(&tile_k[u * kRowsPerQuarter + tt][d0]));
      kmx = h2max(kmx, x);
      kmn = h2min(kmn, x);
    }
    k_part[u][16 * wv + c] = make_uint2(as_u(kmx), as_u(kmn));
  }
  __syncthreads();
  // every load of the group has been consumed: slot 0 may take the new token
  if (g == 0 && a.k_new != nullptr) write_new_token(a, bh, new_slot, tid);

  // ---- K statistics, second half, in wavefront 0 alone (the other three
  // would repeat the same scalar work): lane p combines the four quarters of
  // channels 2p and 2p + 1 and derives their scale, zero, reciprocal, −min·r
  // and the tie edge of their block of 16 channels
  if (tid < 64) {
    const int p = tid;
    const int d0 = 2 * p;
    const uint2 q0 = k_part[0][p], q1 = k_part[1][p], q2 = k_part[2][p], q3 = k_part[3][p];
    const h2v kmx = h2max(h2max(as_h2(q0.x), as_h2(q1.x)), h2max(as_h2(q2.x), as_h2(q3.x)));
    const h2v kmn = h2min(h2min(as_h2(q0.y), as_h2(q1.y)), h2min(as_h2(q2.y), as_h2(q3.y)));
    const float mn0 = float(kmn[0]), mn1 = float(kmn[1]);
    const float s0 = div_code_range<(1 << KB) - 1>(float(kmx[0]) - mn0);
    const float s1 = div_code_range<(1 << KB) - 1>(float(kmx[1]) - mn1);
    const float r0 = quant_recip(s0), r1 = quant_recip(s1);
    const float n0 = -(mn0 * r0), n1 = -(mn1 * r1);
    // the largest |n| of each block of 16 channels (8 lanes: xor 1, xor 2,
    // then the half-row mirror)
    float nm = fmaxf(fabsf(n0), fabsf(n1));
    nm = fmaxf(nm, __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(nm), 0xB1, 0xF, 0xF, false)));
    nm = fmaxf(nm, __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(nm), 0x4E, 0xF, 0xF, false)));
    nm = fmaxf(nm, __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(nm), 0x141, 0xF, 0xF, false)));
    const int64_t o = (blk * a.NG + gg) * kHeadDim + d0;
    store_nt2(a.k_scale + o, __float_as_uint(s0), __float_as_uint(s1));
    store_nt2(a.k_zero + o, __float_as_uint(mn0), __float_as_uint(mn1));
    *reinterpret_cast<float2*>(&s_k[d0]) = make_float2(s0, s1);
    *reinterpret_cast<float2*>(&z_k[d0]) = make_float2(mn0, mn1);
    *reinterpret_cast<float2*>(&r_k[d0]) = make_float2(r0, r1);
    *reinterpret_cast<float2*>(&n_k[d0]) = make_float2(n0, n1);
    if ((p & 7) == 0) edge_k[p >> 3] = tie_edge(nm);
  }

  // ---- V words: per (tile, channel), the tile's 32 token codes packed along
  // tokens; within a word, even tokens fill the low half-word and odd tokens
  // the high.
#pragma unroll
  for (int sub = 0; sub < NS; ++sub) {
    uint32_t* vdst = a.v_codes + (blk * a.NT + gg * NS + sub) * kHeadDim * VW;
#pragma unroll
    for (int rep = 0; rep < (kHeadDim * VW) / kThreads; ++rep) {
      const int idx = rep * kThreads + tid;
      const int d = idx / VW;
      const int w = idx % VW;
      const uint32_t* row = &vt[sub][d / VPER][w * VPER];
      const int sh = VB * (d % VPER);
      uint32_t word = 0;
#pragma unroll
      for (int q4 = 0; q4 < VPER / 4; ++q4) {
        const uint4 x = *reinterpret_cast<const uint4*>(row + 4 * q4);
        const uint32_t xs[4] = {x.x, x.y, x.z, x.w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int i = 4 * q4 + e;
          word |= __builtin_amdgcn_ubfe(xs[e], sh, VB) << (VB * (i / 2) + 16 * (i % 2));
        }
      }
      store_nt(vdst + idx, word);
    }
  }
  __syncthreads();

  // ---- K codes: token 32·sub + t, channels [16j, 16j + 16), packed along channels.
  float4 nq[4], rq[4];
#pragma unroll
  for (int q4 = 0; q4 < 4; ++q4) {
    nq[q4] = *reinterpret_cast<const float4*>(&n_k[16 * j + 4 * q4]);
    rq[q4] = *reinterpret_cast<const float4*>(&r_k[16 * j + 4 * q4]);
  }
  const float kedge = edge_k[j];
#pragma unroll
  for (int sub = 0; sub < NS; ++sub) {
    float kx[16], c[16];
    halves_to_float(*reinterpret_cast<const uint4*>(&tile_k[sub * kGroup + t][j * 16]), kx);
    halves_to_float(*reinterpret_cast<const uint4*>(&tile_k[sub * kGroup + t][j * 16 + 8]), kx + 8);
    float dev = 0.0f;
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) {
      c[4 * q4 + 0] = fast_code(kx[4 * q4 + 0], rq[q4].x, nq[q4].x, dev);
      c[4 * q4 + 1] = fast_code(kx[4 * q4 + 1], rq[q4].y, nq[q4].y, dev);
      c[4 * q4 + 2] = fast_code(kx[4 * q4 + 2], rq[q4].z, nq[q4].z, dev);
      c[4 * q4 + 3] = fast_code(kx[4 * q4 + 3], rq[q4].w, nq[q4].w, dev);
    }
    if (dev > kedge) {
      // as for V: only the values that may sit on a tie
#pragma unroll
      for (int i = 0; i < 16; ++i)
        if (fabsf(fmaf(kx[i], f4c(rq[i / 4], i % 4), f4c(nq[i / 4], i % 4)) - c[i]) > kedge)
          c[i] = float(affine_code(kx[i], z_k[16 * j + i], s_k[16 * j + i], KQMAX));
    }
    uint32_t w[KTW];
    pack16<KB>(c, w);
    uint32_t* kdst = a.k_codes + (blk * CT + gg * G + sub * kGroup + t) * KW;
    if (KB == 2) {
      store_nt(kdst + j, w[0]);
    } else {
      store_nt2(kdst + 2 * j, w[0], w[KTW - 1]);
    }
  }
}

}  // namespace

// launches the (K bits, V bits, NS) instance of the quantize kernel when
// ns == NS (e becomes hipSuccess)
template <int NS>
static void launch_quantize_bits(const KiviQuantArgs& a, dim3 grid, hipStream_t s, int ns,
                          hipError_t& e) {
  if (ns != NS) return;
  e = hipSuccess;
  if (a.bits == 2 && a.vbits == 2) kivi_quantize_kernel<2, 2, NS><<<grid, kThreads, 0, s>>>(a);
  else if (a.bits == 4 && a.vbits == 4) kivi_quantize_kernel<4, 4, NS><<<grid, kThreads, 0, s>>>(a);
  else if (a.bits == 4 && a.vbits == 2) kivi_quantize_kernel<4, 2, NS><<<grid, kThreads, 0, s>>>(a);
  else if (a.bits == 2 && a.vbits == 4) kivi_quantize_kernel<2, 4, NS><<<grid, kThreads, 0, s>>>(a);
  else e = hipErrorInvalidValue;
}

hipError_t launch_kivi_quantize(const KiviQuantArgs& a, hipStream_t s) {
  if (a.n_groups <= 0) return hipSuccess;
  dim3 grid(a.n_groups, a.bh_count);
  const int ns = a.group / kGroup;
  hipError_t e = hipErrorInvalidValue;
  launch_quantize_bits<1>(a, grid, s, ns, e);
  launch_quantize_bits<2>(a, grid, s, ns, e);
  launch_quantize_bits<4>(a, grid, s, ns, e);
  if (e != hipSuccess) return e;
  return hipGetLastError();
}

}  // namespace kvq
