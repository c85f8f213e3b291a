// kvq_quant.hip — cache-write kernels for gfx950: KIVI group quantization
// (prefill and window flush), token copies into the FP16 window / FP16 cache,
// and FP8 (E4M3 or E5M2) quantization with per-tensor or per-KV-head scales.
//
// KIVI ("4.4 KV Cache 量化：KIVI 2-bit 与 FP8 KV Cache", §2 and §3.2;
// "大模型量化从0到1（十三）：KV Cache 量化", §九 and the affine formula of §十):
// K gets one (scale, zero) per (group of G tokens, channel), V one per token.
// Quantizer, each op in fp32 and correctly rounded (no contraction; the
// library is built with -ffp-contract=off):
//   s = (max − min) / (2^b − 1), z = min,
//   code = clamp(rint((x − min) / s), 0, 2^b − 1), code = 0 when s == 0.
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

__device__ __forceinline__ void halves_to_float(const uint4& raw, float* f) {
  const __half2* h = reinterpret_cast<const __half2*>(&raw);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    float2 v = __half22float2(h[i]);
    f[2 * i] = v.x;
    f[2 * i + 1] = v.y;
  }
}

// ---- fast exact quotient. The code is rint(RN((x − min) / s)). With r within
// about one ulp of 1/s, p = RN((x − min)·r) lies within 1.5·2⁻²³·Q of the exact
// quotient Q ≤ 2^b − 1 < 16, so |p − RN(Q)| < 2⁻¹⁸. Unless p is within 2⁻¹⁶ of
// a half-integer (a possible rounding tie), rint(p) is the code; the rare lanes
// with such a value redo their codes with the correctly rounded division.
constexpr float kTieEdge = 0.5f - 1.0f / 65536.0f;

// 1/s to within about an ulp (one Newton step on the hardware estimate);
// 0 when s == 0, which makes every code 0 as the quantizer requires.
__device__ __forceinline__ float quant_recip(float s) {
  if (s == 0.0f) return 0.0f;
  const float r = __builtin_amdgcn_rcpf(s);
  return fmaf(r, fmaf(-s, r, 1.0f), r);
}

// rint((x − mn)·r) as a float (0 ≤ code ≤ 2^b − 1); `dev` keeps the largest
// |p − rint(p)| seen, so that dev > kTieEdge flags a possible rounding tie.
__device__ __forceinline__ float fast_code(float x, float mn, float r, float& dev) {
  const float p = (x - mn) * r;
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
  return __builtin_amdgcn_class(x, 0x267) ? q : c;
}

typedef _Float16 h2v __attribute__((ext_vector_type(2)));

__device__ __forceinline__ h2v as_h2(uint32_t u) { return __builtin_bit_cast(h2v, u); }
__device__ __forceinline__ uint32_t as_u(h2v h) { return __builtin_bit_cast(uint32_t, h); }
__device__ __forceinline__ h2v h2max(h2v a, h2v b) { return __builtin_elementwise_max(a, b); }
__device__ __forceinline__ h2v h2min(h2v a, h2v b) { return __builtin_elementwise_min(a, b); }

// pack 16 codes (floats 0..2^b−1) of consecutive channels into 32-bit words,
// channel i of a word at bits [b·i, b·i + b): 2 bits → 1 word, 4 bits → 2.
template <int BITS>
__device__ __forceinline__ void pack16(const float (&c)[16], uint32_t (&w)[BITS / 2]) {
  constexpr int PER = 32 / BITS;
#pragma unroll
  for (int k = 0; k < BITS / 2; ++k) {
    // two exact float sums of 8 codes each (< 2^16), then one integer merge
    float lo = 0.0f, hi = 0.0f;
#pragma unroll
    for (int i = 0; i < PER / 2; ++i) {
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
// tokens × 128 channels) of K and of V for one (b, h). Loads: thread
// (t = tid / 8, j = tid % 8) holds channels [16j, 16j + 16) of token t of each
// sub-tile (256 contiguous bytes per token).
//   V (per token): min / max over the 8 threads of a token, or over the 2
//      threads of each run of 32 channels (packed fp16 max of (x, −x), DPP
//      exchanges), codes in registers, one word (two at 4
//      bits) of 16 channel codes per thread into an LDS transpose, from which
//      each thread assembles the sub-tile's V words along tokens.
//   K (per channel over the G tokens): the group goes through LDS; wavefront
//      w takes channels [32w, 32w + 32), lane (pair c = l % 16, quarter
//      u = l / 16) reduces rows [u·G/4, (u+1)·G/4) of channels 32w + 2c, +1,
//      then the four quarters are combined; codes of the thread's 16 channels
//      follow from the per-channel scale and zero.
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
  __shared__ __attribute__((aligned(16))) float s_k[kHeadDim];
  __shared__ __attribute__((aligned(16))) float z_k[kHeadDim];
  __shared__ __attribute__((aligned(16))) float r_k[kHeadDim];
  __shared__ __attribute__((aligned(16))) uint32_t vt[NS][VTR][kRow];  // [sub][channel word][token]

  const int g = blockIdx.x;
  const int bh = blockIdx.y;
  const int tid = threadIdx.x;
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
    const int e = a.block_table[int64_t(b) * a.max_pages + (gg >> a.page_group_shift)];
    blk = int64_t(min(max(e, 0), a.num_pages - 1)) * a.H + h;
    gg &= (int64_t(1) << a.page_group_shift) - 1;
  }
  const int64_t CT = a.NG * G;             // token slots of one block

  uint4 kr[NS][2];                         // the thread's K values of each sub-tile
#pragma unroll
  for (int sub = 0; sub < NS; ++sub) {
    const int tr = sub * kGroup + t;       // token row within the group
    const int64_t src = bh * a.src_bh_stride + (int64_t(g) * G + tr) * kHeadDim + j * 16;
    kr[sub][0] = *reinterpret_cast<const uint4*>(a.k_src + src);
    kr[sub][1] = *reinterpret_cast<const uint4*>(a.k_src + src + 8);
    const uint4 v0 = *reinterpret_cast<const uint4*>(a.v_src + src);
    const uint4 v1 = *reinterpret_cast<const uint4*>(a.v_src + src + 8);
    *reinterpret_cast<uint4*>(&tile_k[tr][j * 16]) = kr[sub][0];
    *reinterpret_cast<uint4*>(&tile_k[tr][j * 16 + 8]) = kr[sub][1];

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
      a.v_scale[o] = vs;
      a.v_zero[o] = vmn;
    }

    // ---- V codes of the thread's 16 channels → the LDS transpose
    float vx[16], c[16];
    halves_to_float(v0, vx);
    halves_to_float(v1, vx + 8);
    const float vr = quant_recip(vs);
    float dev = 0.0f;
#pragma unroll
    for (int i = 0; i < 16; ++i) c[i] = fast_code(vx[i], vmn, vr, dev);
    if (dev > kTieEdge) {
      // a lane with a possible tie recomputes only the values that may sit on
      // one (the fast codes of the others are exact): a wavefront then runs
      // the division for the value slots where some lane has one
#pragma unroll
      for (int i = 0; i < 16; ++i)
        if (fabsf((vx[i] - vmn) * vr - c[i]) > kTieEdge)
          c[i] = float(affine_code(vx[i], vmn, vs, VQMAX));
    }
    uint32_t w[VTW];
    pack16<VB>(c, w);
#pragma unroll
    for (int k = 0; k < VTW; ++k) vt[sub][VTW * j + k][t] = w[k];
  }
  __syncthreads();
  // every load of the group has been consumed: slot 0 may take the new token
  if (g == 0 && a.k_new != nullptr) write_new_token(a, bh, new_slot, tid);

  // ---- K statistics over the G rows: wavefront w, channels 32w + 2c, +1
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
    // combine the four quarters (lanes l ^ 16, l ^ 32)
#pragma unroll
    for (int step = 0; step < 2; ++step) {
      const auto px = step == 0
          ? __builtin_amdgcn_permlane16_swap(as_u(kmx), as_u(kmx), false, false)
          : __builtin_amdgcn_permlane32_swap(as_u(kmx), as_u(kmx), false, false);
      const auto pn = step == 0
          ? __builtin_amdgcn_permlane16_swap(as_u(kmn), as_u(kmn), false, false)
          : __builtin_amdgcn_permlane32_swap(as_u(kmn), as_u(kmn), false, false);
      kmx = h2max(as_h2(px[0]), as_h2(px[1]));
      kmn = h2min(as_h2(pn[0]), as_h2(pn[1]));
    }
    const float mn0 = float(kmn[0]), mn1 = float(kmn[1]);
    const float s0 = div_code_range<(1 << KB) - 1>(float(kmx[0]) - mn0);
    const float s1 = div_code_range<(1 << KB) - 1>(float(kmx[1]) - mn1);
    if (u == 0) {
      const int64_t o = (blk * a.NG + gg) * kHeadDim + d0;
      *reinterpret_cast<float2*>(a.k_scale + o) = make_float2(s0, s1);
      *reinterpret_cast<float2*>(a.k_zero + o) = make_float2(mn0, mn1);
      *reinterpret_cast<float2*>(&s_k[d0]) = make_float2(s0, s1);
      *reinterpret_cast<float2*>(&z_k[d0]) = make_float2(mn0, mn1);
      *reinterpret_cast<float2*>(&r_k[d0]) = make_float2(quant_recip(s0), quant_recip(s1));
    }
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
          word |= ((xs[e] >> sh) & ((1u << VB) - 1)) << (VB * (i / 2) + 16 * (i % 2));
        }
      }
      vdst[idx] = word;
    }
  }
  __syncthreads();

  // ---- K codes: token 32·sub + t, channels [16j, 16j + 16), packed along channels.
  float4 zq[4], rq[4];
#pragma unroll
  for (int q4 = 0; q4 < 4; ++q4) {
    zq[q4] = *reinterpret_cast<const float4*>(&z_k[16 * j + 4 * q4]);
    rq[q4] = *reinterpret_cast<const float4*>(&r_k[16 * j + 4 * q4]);
  }
#pragma unroll
  for (int sub = 0; sub < NS; ++sub) {
    float kx[16], c[16];
    halves_to_float(kr[sub][0], kx);
    halves_to_float(kr[sub][1], kx + 8);
    float dev = 0.0f;
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) {
      c[4 * q4 + 0] = fast_code(kx[4 * q4 + 0], zq[q4].x, rq[q4].x, dev);
      c[4 * q4 + 1] = fast_code(kx[4 * q4 + 1], zq[q4].y, rq[q4].y, dev);
      c[4 * q4 + 2] = fast_code(kx[4 * q4 + 2], zq[q4].z, rq[q4].z, dev);
      c[4 * q4 + 3] = fast_code(kx[4 * q4 + 3], zq[q4].w, rq[q4].w, dev);
    }
    if (dev > kTieEdge) {
      // as for V: only the values that may sit on a tie
#pragma unroll
      for (int i = 0; i < 16; ++i)
        if (fabsf((kx[i] - f4c(zq[i / 4], i % 4)) * f4c(rq[i / 4], i % 4) - c[i]) > kTieEdge)
          c[i] = float(affine_code(kx[i], z_k[16 * j + i], s_k[16 * j + i], KQMAX));
    }
    uint32_t w[KTW];
    pack16<KB>(c, w);
    uint32_t* kdst = a.k_codes + (blk * CT + gg * G + sub * kGroup + t) * KW;
    if (KB == 2) {
      kdst[j] = w[0];
    } else {
      *reinterpret_cast<uint2*>(kdst + 2 * j) = make_uint2(w[0], w[KTW - 1]);
    }
  }
}

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
  // about 4096 workgroups in all, at most one per 256 chunks of a (b, h)
  const int64_t per_bh_chunks = a.n_tokens * (kHeadDim / 8);
  int64_t per_bh = (4096 + a.bh_count - 1) / a.bh_count;
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
