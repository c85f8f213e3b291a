// kvq_internal.h — launch parameter blocks shared by the C ABI host code
// (kvq_api.cpp) and the HIP kernels (kvq_quant.hip, kvq_decode.hip).
// Not part of the public interface.
#pragma once

#include <hip/hip_fp16.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kvq {

constexpr int kHeadDim = 128;   // D
constexpr int kGroup = 32;      // tokens per decode tile and per KIVI V code tile (the KIVI group when G = 32)

// Per-sequence counts of a ragged batch, passed by value with the launch
// (sequence b = bh / H); the meaning of x, y, z is stated by each user.
constexpr int kMaxRagged = 128;
struct RaggedTable {
  int32_t x[kMaxRagged];
  int32_t y[kMaxRagged];
  int32_t z[kMaxRagged];
};

// KIVI quantization of whole groups. Source tokens [0, n_groups·G) of each
// (b, h) block of an fp16 [B·H][src_tokens][D] tensor are quantized into the
// cache groups [g0, g0 + n_groups).
struct KiviQuantArgs {
  const __half* k_src;
  const __half* v_src;
  int64_t src_bh_stride;  // elements between consecutive (b, h) blocks
  int n_groups;
  int64_t g0;
  int bh_count;           // B·H
  int bits;               // K bit width
  int vbits;              // V bit width
  int64_t NG;             // group slots per (b, h)
  int64_t NT;             // 32-token V tiles per (b, h) (NG·G/32)
  int group;              // G: 32, 64 or 128 tokens per K scale group
  int nvs;                // V scales per token: 1, or 4 (runs of 32 channels)
  uint32_t* k_codes;      // [B·H][NG·G][D·b/32]
  uint32_t* v_codes;      // [B·H][NT][D][32·b_V/32]
  float* k_scale;         // [B·H][NG][D]
  float* k_zero;
  float* v_scale;         // [B·H][NG·G][nvs]
  float* v_zero;
  // ragged batch: sequence b quantizes groups [0, seq.x[b]) of its source
  // into cache groups [seq.y[b], seq.y[b] + seq.x[b]) (n_groups, g0 unused)
  int ragged;
  int H;
  // paged cache: group gg of sequence b goes to page
  // block_table[b·max_pages + (gg >> page_group_shift)] (clamped to the pool),
  // group gg mod 2^page_group_shift of that page's (page, h) block; NG, NT
  // are then a page's groups and tiles
  int paged;
  const int32_t* block_table;
  int max_pages;
  int page_group_shift;
  int num_pages;
  // a window flush folds in the append that triggered it: the new token
  // (fp16 [B·H][D]) goes to window slot 0 of each (b, h) block (a ragged
  // batch: slot seq.z[b], and sequences that do not flush only take the new
  // token), written by the block's group-0 workgroup once it holds its loads
  // of that slot (null k_new: no token)
  const __half* k_new;
  const __half* v_new;
  __half* k_win;
  __half* v_win;
  int64_t win_bh_stride;  // elements between window blocks
  RaggedTable seq;
};

// Strided copy of `n_tokens` tokens of K and V (fp16, D channels each) from
// [B·H][src_tokens][D] into [B·H][dst_tokens][D] at token offset dst_t0.
struct CopyTokensArgs {
  const __half* k_src;
  const __half* v_src;
  int64_t src_bh_stride;  // elements
  __half* k_dst;
  __half* v_dst;
  int64_t dst_bh_stride;  // elements
  int64_t dst_t0;
  int64_t n_tokens;
  int bh_count;
  // ragged batch: sequence b copies seq.y[b] tokens from source token
  // seq.x[b] to cache token seq.z[b] (n_tokens: the largest count)
  int ragged;
  int H;
  RaggedTable seq;
};

// FP8 code formats (the cache's V tiles and K rows).
enum Fp8Format : int { kE4M3 = 0, kE5M2 = 1 };

// V of the FP8 / FP16 caches in tiles of kGroup tokens: tile g of (b, h) is
// [D][kGroup] (one row of the tile's tokens per channel). Writes source tokens
// [0, n_tokens) of each (b, h) block of an fp16 [B·H][src_tokens][D] tensor
// to cache tokens [dst_t0, dst_t0 + n_tokens), as fp16 or as FP8 codes with
// the stored V scale of the block's KV head (tensor_scale[scale_stride·h + 1]).
// zero_tail: also zero the slots after the last written token up to the end
// of its tile.
struct VTileArgs {
  const __half* v_src;
  int64_t src_bh_stride;  // elements
  int64_t n_tokens;
  int64_t dst_t0;
  void* v_dst;            // fp16 or uint8 [B·H][NT][D][kGroup]
  int64_t NT;             // tiles per (b, h)
  int bh_count;
  int H;                  // KV heads (h = bh % H)
  int fp8;                // 0: fp16 copy, 1: FP8 encode
  int fmt;                // Fp8Format
  int scale_stride;       // floats between KV heads' scale rows (0: per tensor)
  int zero_tail;
  const float* tensor_scale;
};

// FP8 quantization, one scale pair per tensor or per KV head.
struct Fp8QuantArgs {
  const __half* k_src;
  const __half* v_src;
  int64_t src_bh_stride;  // elements
  int64_t n_tokens;       // tokens per (b, h) to encode
  uint8_t* k_codes;       // [B·H][CT][D]
  uint8_t* v_codes;       // row-major V codes, or null (V written in tiles)
  int64_t dst_bh_stride;  // elements (C·D)
  int64_t dst_t0;
  int bh_count;
  int H;                  // KV heads (h = bh % H)
  int fmt;                // Fp8Format
  int per_head;           // 1: row h of tensor_scale belongs to KV head h
  float* tensor_scale;    // [per_head ? H : 1][4] {s_K, s_V, amax_K, amax_V}
};

enum SrcFormat : int { kSrcFp16 = 0, kSrcFp8 = 1, kSrcKivi2 = 2, kSrcKivi4 = 3, kSrcE5M2 = 4 };

// Split-K decode attention. Grid: n_split · B·H · head_chunks blocks in one
// dimension, main-region splits first and window splits last.
// 1: a decode with one split per row writes its output from the split
// kernel, without the merge launch.
#ifndef KVQ_DIRECT_SINGLE_SPLIT
#define KVQ_DIRECT_SINGLE_SPLIT 1
#endif

struct DecodeArgs {
  int src;                // SrcFormat of the main region
  int kbits, vbits;       // KIVI K and V bit widths
  int nvs;                // KIVI V scales per token (1, or 4: runs of 32 channels)
  int B, H, Hq;
  int nq;                 // query heads per KV head (Hq / H)
  int heads_per_chunk;    // query heads one workgroup handles
  // main region: KIVI grouped region, or the whole FP8 / FP16 cache
  const void* k_main;
  const void* v_main;
  const float* k_scale;
  const float* k_zero;
  const float* v_scale;
  const float* v_zero;
  const float* tensor_scale;
  int scale_stride;       // FP8: floats between KV heads' scale rows (0: per tensor)
  int qfp8;               // FP8: scores in the FP8 domain (query quantized to E4M3)
  int64_t NG;             // KIVI group slots per (b, h)
  int64_t NT;             // 32-token tiles per (b, h) (KIVI V codes; FP8 / FP16 V tiles)
  int gshift;             // log2(G / 32): tile t uses the K scales of group t >> gshift
  int64_t main_bh_tokens; // token slots per (b, h) of the main region
  int64_t n_main;         // tokens in the main region
  // KIVI FP16 window
  const __half* k_win;
  const __half* v_win;
  int win_cap;            // token slots per (b, h)
  int n_win;              // tokens in the window
  // split plan
  int tiles_per_split;
  int n_split_main;       // splits over the main region
  int n_split;            // n_split_main, +1 if the window has a split of its own
  int win_split;          // split that runs the window tiles (-1: empty window)
  int fixed_order;        // KIVI: 1 = wavefront w takes tiles w, w + NW, ... of its
                          // split (deterministic); 0 = tiles from a shared counter
  int unit;               // KIVI: 1 = one workgroup per compute unit (tiles shared
                          // unless fixed_order), 0 = four-wavefront workgroups
  // an append folded into the decode (KIVI, no flush due): the appended token
  // (fp16 [B·H][D]) is window slot n_win − 1 (ragged: seq.y[b] − 1); the
  // workgroups that run the window read it from here, and those of head
  // chunk 0 store it into the window buffers (null k_new: no append)
  const __half* k_new;
  const __half* v_new;
  __half* k_win_store;
  __half* v_win_store;
  const float* q;         // [B][Hq][D]
  float* out;             // [B][Hq][D]
  float* ws;              // [B][Hq][n_split][D + 2]
  float qscale;           // log2(e) / sqrt(D)
  // ragged KIVI batch: sequence b has seq.x[b] 32-token tiles in its grouped
  // region and seq.y[b] window tokens (n_main, n_win, win_split unused)
  int ragged;
  // paged KIVI cache: tile g of sequence b is tile g mod 2^page_tile_shift of
  // the (page, h) block of page block_table[b·max_pages + (g >> page_tile_shift)]
  // (clamped to the pool); NG, NT and main_bh_tokens are then a page's
  int paged;
  const int32_t* block_table;
  int max_pages;
  int page_tile_shift;
  int num_pages;
  RaggedTable seq;
};

hipError_t launch_kivi_quantize(const KiviQuantArgs& a, hipStream_t s);
hipError_t launch_copy_tokens(const CopyTokensArgs& a, hipStream_t s);
hipError_t launch_v_tiles(const VTileArgs& a, hipStream_t s);
hipError_t launch_fp8_prefill(const Fp8QuantArgs& a, hipStream_t s);
hipError_t launch_fp8_append(const Fp8QuantArgs& a, hipStream_t s);
// Per-row E4M3 quantization of fp32 query rows of D = 128 values.
struct QueryQuantArgs {
  const float* q;         // [rows][D]
  uint8_t* codes;         // [rows][D]
  float* scales;          // [rows]
  int64_t rows;
};

hipError_t launch_query_fp8(const QueryQuantArgs& a, hipStream_t s);
hipError_t launch_decode(const DecodeArgs& a, hipStream_t s);
// Device address of the current GPU's split-partial array of
// kvq_decode_attention_static (KVQ_STATIC_WORKSPACE_BYTES), looked up once per
// device with that device current.
hipError_t static_workspace(void** ptr);
// Workgroups of the split kernel that a.src, a.kbits, a.vbits, a.nvs and a.qfp8
// select that the current device holds at once (compute units × resident
// workgroups per unit, from the kernel's register and LDS use); 0 if the
// runtime cannot tell.
int decode_resident_workgroups(const DecodeArgs& a);
// Compute units of the current device (0 if the runtime cannot tell).
int device_compute_units();
hipError_t launch_kivi_mfma(const DecodeArgs& a, hipStream_t s);
hipError_t launch_dense_mfma(const DecodeArgs& a, hipStream_t s);

}  // namespace kvq
