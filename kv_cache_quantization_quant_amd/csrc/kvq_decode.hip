// kvq_decode.hip — split-K single-query decode attention over a KIVI, FP8 or
// FP16 cache, for gfx950.
//
// Attention ("大模型量化从0到1（十三）：KV Cache 量化", §二 and §八.1–八.2):
//   score_t = q·k̂_t / √D,  p = softmax(score),  out = Σ_t p_t v̂_t,
// over every cached token (grouped region, then the FP16 window). Query head
// hq reads KV head hq / (Hq / H) (§五.3, consecutive query heads share).
// Dequantization happens inside the kernel, in registers:
//   KIVI  k̂ = code · s[g, d] + z[g, d],  v̂ = code · s[t] + z[t]
//   FP8   x̂ = e4m3_value(code) · s_tensor
//
// Work decomposition: a workgroup (4 wavefronts) owns one (b, KV head, chunk
// of query heads) and a contiguous range of 32-token tiles (one KIVI group per
// tile). Each wavefront streams every 4th tile of the range with its own
// online-softmax state (log2 domain: q is pre-scaled by log2(e)/√D and exp2 is
// used); the four states are merged through LDS into one partial
// (m, l, o[D]) per (b, hq, split). A second kernel merges the splits.
#include <hip/hip_fp16.h>
#include <hip/hip_runtime.h>

#include <math.h>

#include "kvq_internal.h"

namespace kvq {
namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / 64;
constexpr int kPart = kHeadDim + 2;   // partial record: o[D], m, l

__device__ __forceinline__ void wave_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

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

template <int NQ>
struct WaveState {
  float m[NQ];
  float l[NQ];
  float o[NQ][2];   // channels 2·lane, 2·lane + 1
};

template <int NQ>
struct Smem {
  float q[NQ][kHeadDim];
  float ksz[kWaves][2][kHeadDim];      // KIVI: K scale / zero of the tile's group
  float vsz[kWaves][2][kGroup];        // KIVI: V scale / zero of the tile's tokens
  float p[kWaves][NQ][kGroup];         // probabilities of the tile
  float mo[kWaves][NQ][kHeadDim];      // wave states for the merge
  float ml[kWaves][NQ][2];
};

__device__ __forceinline__ void halves8(const uint4& raw, float* f) {
  const __half2* h = reinterpret_cast<const __half2*>(&raw);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    float2 v = __half22float2(h[i]);
    f[2 * i] = v.x;
    f[2 * i + 1] = v.y;
  }
}

__device__ __forceinline__ float e4m3_to_float(uint32_t word, int byte) {
  switch (byte) {
    case 0: return __builtin_amdgcn_cvt_f32_fp8(word, 0);
    case 1: return __builtin_amdgcn_cvt_f32_fp8(word, 1);
    case 2: return __builtin_amdgcn_cvt_f32_fp8(word, 2);
    default: return __builtin_amdgcn_cvt_f32_fp8(word, 3);
  }
}

// One 32-token tile: scores, online-softmax update, P·V.
// Lane (t = lane % 32, hf = lane / 32) scores token t over channels
// [64·hf, 64·hf + 64); in P·V the lane owns channels 2·lane, 2·lane + 1.
template <int SRC, int NQ, int OUTER = (NQ <= 2 ? 8 : 1)>
__device__ __forceinline__ void process_tile(const DecodeArgs& a, Smem<NQ>& sm,
                                             WaveState<NQ>& st, int wave, int lane,
                                             int bh, int64_t tile, int64_t n_tok,
                                             const void* kbase, const void* vbase,
                                             int64_t bh_tokens, int nh) {
  const int t = lane & 31;
  const int hf = lane >> 5;
  const int64_t tok = tile * kGroup + t;
  const bool valid = tok < n_tok;
  const int n_in_tile = int(min<int64_t>(kGroup, n_tok - tile * kGroup));

  float acc[NQ];
#pragma unroll
  for (int h = 0; h < NQ; ++h) acc[h] = 0.0f;

  if constexpr (SRC == kSrcKivi2 || SRC == kSrcKivi4) {
    constexpr int BITS = SRC == kSrcKivi2 ? 2 : 4;
    constexpr int PER = 32 / BITS;
    constexpr int KW = kHeadDim / PER;
    constexpr uint32_t MASK = (1u << BITS) - 1u;
    // stage this group's per-channel scale and zero-point
    const int64_t meta = (int64_t(bh) * a.NG + tile) * kHeadDim;
    const float2 s2 = *reinterpret_cast<const float2*>(a.k_scale + meta + 2 * lane);
    const float2 z2 = *reinterpret_cast<const float2*>(a.k_zero + meta + 2 * lane);
    *reinterpret_cast<float2*>(&sm.ksz[wave][0][2 * lane]) = s2;
    *reinterpret_cast<float2*>(&sm.ksz[wave][1][2 * lane]) = z2;
    wave_sync();
    const uint32_t* row = static_cast<const uint32_t*>(kbase) +
                          (int64_t(bh) * bh_tokens + tok) * KW + hf * (KW / 2);
#pragma unroll OUTER
    for (int c = 0; c < 8; ++c) {            // 8 blocks of 8 channels
      const uint32_t word = row[(c * 8) / PER];
      const int sh0 = BITS * ((c * 8) % PER);
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int d = hf * 64 + c * 8 + i;
        const float code = float((word >> (sh0 + BITS * i)) & MASK);
        const float kv = code * sm.ksz[wave][0][d] + sm.ksz[wave][1][d];
#pragma unroll
        for (int h = 0; h < NQ; ++h) acc[h] = fmaf(sm.q[h][d], kv, acc[h]);
      }
    }
  } else if constexpr (SRC == kSrcFp8) {
    const float s = a.tensor_scale[0];
    if (valid) {
      const uint8_t* row = static_cast<const uint8_t*>(kbase) +
                           (int64_t(bh) * bh_tokens + tok) * kHeadDim + hf * 64;
#pragma unroll OUTER
      for (int c = 0; c < 8; ++c) {          // 8 blocks of 8 channels
        const uint2 u = *reinterpret_cast<const uint2*>(row + c * 8);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int d = hf * 64 + c * 8 + e;
          const float kv = e4m3_to_float(e < 4 ? u.x : u.y, e & 3) * s;
#pragma unroll
          for (int h = 0; h < NQ; ++h) acc[h] = fmaf(sm.q[h][d], kv, acc[h]);
        }
      }
    }
  } else {  // FP16
    if (valid) {
      const __half* row = static_cast<const __half*>(kbase) +
                          (int64_t(bh) * bh_tokens + tok) * kHeadDim + hf * 64;
#pragma unroll OUTER
      for (int c8 = 0; c8 < 8; ++c8) {
        float kv[8];
        halves8(*reinterpret_cast<const uint4*>(row + c8 * 8), kv);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int d = hf * 64 + c8 * 8 + e;
#pragma unroll
          for (int h = 0; h < NQ; ++h) acc[h] = fmaf(sm.q[h][d], kv[e], acc[h]);
        }
      }
    }
  }

  // ---- online softmax (both halves of the wave hold the same scores)
#pragma unroll
  for (int h = 0; h < NQ; ++h) {
    float sc = acc[h] + __shfl_xor(acc[h], 32);
    sc = valid ? sc : -INFINITY;
    const float m_new = fmaxf(st.m[h], wave_max(sc));
    const float alpha = exp2f(st.m[h] - m_new);
    const float p = valid ? exp2f(sc - m_new) : 0.0f;
    const float psum = wave_sum(hf == 0 ? p : 0.0f);
    st.l[h] = st.l[h] * alpha + psum;
    st.o[h][0] *= alpha;
    st.o[h][1] *= alpha;
    st.m[h] = m_new;
    if (hf == 0) sm.p[wave][h][t] = (h < nh) ? p : 0.0f;
  }

  // ---- P·V over the tile's tokens
  const int d0 = 2 * lane;
  if constexpr (SRC == kSrcKivi2 || SRC == kSrcKivi4) {
    constexpr int BITS = SRC == kSrcKivi2 ? 2 : 4;
    constexpr int PER = 32 / BITS;
    constexpr int VW = kGroup / PER;
    constexpr uint32_t MASK = (1u << BITS) - 1u;
    const int64_t tok0 = int64_t(bh) * bh_tokens + tile * kGroup;
    sm.vsz[wave][hf][t] = hf == 0 ? a.v_scale[tok0 + t] : a.v_zero[tok0 + t];
    wave_sync();
    const uint32_t* cw = static_cast<const uint32_t*>(vbase) +
                         ((int64_t(bh) * a.NG + tile) * kHeadDim + d0) * VW;
    uint32_t w0[VW], w1[VW];
#pragma unroll
    for (int w = 0; w < VW; ++w) {
      w0[w] = cw[w];
      w1[w] = cw[VW + w];
    }
#pragma unroll OUTER
    for (int tb = 0; tb < kGroup; tb += 8) {   // 4 blocks of 8 tokens
#pragma unroll
      for (int tt = tb; tt < tb + 8; ++tt) {
        const float s = sm.vsz[wave][0][tt];
        const float z = sm.vsz[wave][1][tt];
        const int sh = BITS * ((tt % PER) / 2) + 16 * ((tt % PER) % 2);
        const float v0 = float((w0[tt / PER] >> sh) & MASK) * s + z;
        const float v1 = float((w1[tt / PER] >> sh) & MASK) * s + z;
#pragma unroll
        for (int h = 0; h < NQ; ++h) {
          const float p = sm.p[wave][h][tt];
          st.o[h][0] = fmaf(p, v0, st.o[h][0]);
          st.o[h][1] = fmaf(p, v1, st.o[h][1]);
        }
      }
    }
  } else {
    wave_sync();
    const int64_t tok0 = int64_t(bh) * bh_tokens + tile * kGroup;
    for (int tt = 0; tt < n_in_tile; ++tt) {
      float v0, v1;
      if constexpr (SRC == kSrcFp8) {
        const uint8_t* r = static_cast<const uint8_t*>(vbase) + (tok0 + tt) * kHeadDim + d0;
        const uint32_t two = *reinterpret_cast<const uint16_t*>(r);
        const float s = a.tensor_scale[1];
        v0 = e4m3_to_float(two, 0) * s;
        v1 = e4m3_to_float(two, 1) * s;
      } else {
        const __half2 hv = *reinterpret_cast<const __half2*>(
            static_cast<const __half*>(vbase) + (tok0 + tt) * kHeadDim + d0);
        const float2 f = __half22float2(hv);
        v0 = f.x;
        v1 = f.y;
      }
#pragma unroll
      for (int h = 0; h < NQ; ++h) {
        const float p = sm.p[wave][h][tt];
        st.o[h][0] = fmaf(p, v0, st.o[h][0]);
        st.o[h][1] = fmaf(p, v1, st.o[h][1]);
      }
    }
  }
  wave_sync();
}

template <int SRC, int NQ>
__global__ __launch_bounds__(kThreads) void decode_split_kernel(DecodeArgs a) {
  __shared__ Smem<NQ> sm;
  const int split = int(blockIdx.x) + a.split_offset;
  const int bh = blockIdx.y;
  const int b = bh / a.H;
  const int h_kv = bh % a.H;
  const int hq0 = h_kv * a.nq + blockIdx.z * NQ;
  const int nh = min(NQ, a.nq - int(blockIdx.z) * NQ);
  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;

  for (int i = tid; i < NQ * kHeadDim; i += kThreads) {
    const int h = i / kHeadDim;
    const int d = i % kHeadDim;
    sm.q[h][d] = h < nh ? a.q[(int64_t(b) * a.Hq + hq0 + h) * kHeadDim + d] * a.qscale : 0.0f;
  }
  __syncthreads();

  WaveState<NQ> st;
#pragma unroll
  for (int h = 0; h < NQ; ++h) {
    st.m[h] = -INFINITY;
    st.l[h] = 0.0f;
    st.o[h][0] = 0.0f;
    st.o[h][1] = 0.0f;
  }

  if (split < a.n_split_main) {
    const int64_t n_tiles = (a.n_main + kGroup - 1) / kGroup;
    const int64_t t0 = int64_t(split) * a.tiles_per_split;
    const int64_t t1 = min<int64_t>(t0 + a.tiles_per_split, n_tiles);
    for (int64_t tile = t0 + wave; tile < t1; tile += kWaves)
      process_tile<SRC, NQ>(a, sm, st, wave, lane, bh, tile, a.n_main, a.k_main, a.v_main,
                            a.main_bh_tokens, nh);
  } else {
    const int64_t n_tiles = (a.n_win + kGroup - 1) / kGroup;
    for (int64_t tile = wave; tile < n_tiles; tile += kWaves)
      process_tile<kSrcFp16, NQ>(a, sm, st, wave, lane, bh, tile, a.n_win, a.k_win, a.v_win,
                                 a.win_cap, nh);
  }

  // ---- merge the four wave states of this workgroup
#pragma unroll
  for (int h = 0; h < NQ; ++h) {
    sm.mo[wave][h][2 * lane] = st.o[h][0];
    sm.mo[wave][h][2 * lane + 1] = st.o[h][1];
    if (lane == 0) {
      sm.ml[wave][h][0] = st.m[h];
      sm.ml[wave][h][1] = st.l[h];
    }
  }
  __syncthreads();
  for (int i = tid; i < nh * kHeadDim; i += kThreads) {
    const int h = i / kHeadDim;
    const int d = i % kHeadDim;
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) M = fmaxf(M, sm.ml[w][h][0]);
    float O = 0.0f, L = 0.0f;
    if (M != -INFINITY) {
#pragma unroll
      for (int w = 0; w < kWaves; ++w) {
        const float mw = sm.ml[w][h][0];
        const float f = mw == -INFINITY ? 0.0f : exp2f(mw - M);
        O = fmaf(f, sm.mo[w][h][d], O);
        L = fmaf(f, sm.ml[w][h][1], L);
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

template <int SRC>
hipError_t launch_src(const DecodeArgs& a, int n_splits, hipStream_t s) {
  const dim3 grid(n_splits, a.B * a.H, a.nq / a.heads_per_chunk);
  switch (a.heads_per_chunk) {
    case 1: decode_split_kernel<SRC, 1><<<grid, kThreads, 0, s>>>(a); break;
    case 2: decode_split_kernel<SRC, 2><<<grid, kThreads, 0, s>>>(a); break;
    case 4: decode_split_kernel<SRC, 4><<<grid, kThreads, 0, s>>>(a); break;
    case 8: decode_split_kernel<SRC, 8><<<grid, kThreads, 0, s>>>(a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace

// KIVI: the grouped region and the FP16 window (one extra split) on the
// matrix cores; FP8 / FP16: every split on the vector path. Then the merge.
hipError_t launch_decode(const DecodeArgs& a_in, hipStream_t s) {
  DecodeArgs a = a_in;
  hipError_t e = hipSuccess;
  switch (a.src) {
    case kSrcKivi2:
    case kSrcKivi4:
      a.split_offset = 0;
      e = launch_kivi_mfma(a, s);
      break;
    case kSrcFp16:
      a.split_offset = 0;
      e = launch_src<kSrcFp16>(a, a.n_split, s);
      break;
    case kSrcFp8:
      a.split_offset = 0;
      e = launch_src<kSrcFp8>(a, a.n_split, s);
      break;
    default:
      return hipErrorInvalidValue;
  }
  if (e != hipSuccess) return e;
  decode_merge_kernel<<<a.B * a.Hq, 64, 0, s>>>(a);
  return hipGetLastError();
}

}  // namespace kvq
