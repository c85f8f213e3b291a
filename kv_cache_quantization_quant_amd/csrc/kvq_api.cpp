// kvq_api.cpp — the C ABI declared in include/kvq.h: argument and state
// validation, the KIVI fill-state machine, split planning and kernel dispatch.
//
// State machine ("4.4 KV Cache 量化：KIVI 2-bit 与 FP8 KV Cache", §3.1–3.2):
// prefill fills whole groups and leaves the newest tokens (≤ R) in the FP16
// window; an append that finds the window full first quantizes all of it into
// new groups (lazy flush), then stores the token. With R = 0 the window holds
// the incomplete group (capacity G), because per-channel K needs a whole group
// before it has a scale (§3.1).
//
// Every check runs before any launch; a failing call changes nothing.
#include <hip/hip_runtime.h>

#include <math.h>

#include <algorithm>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#include "../../include/kvq.h"
#include "kvq_internal.h"

namespace {

using kvq::kGroup;
using kvq::kHeadDim;

// Workgroups one decode launch aims for: KVQ_SPLIT_ROUNDS full rounds of the
// split kernel's resident workgroups on the device (one round: every block
// starts at once, and none waits for a slot behind a long one), at most
// kMaxTargetWorkgroups (which bounds the workspace independently of the
// device); kFallbackWorkgroups when the runtime cannot report residency.
#ifndef KVQ_SPLIT_ROUNDS
#define KVQ_SPLIT_ROUNDS 1
#endif
constexpr int64_t kMaxTargetWorkgroups = 4096;
// Time of one FP16 window tile in grouped-region tiles: the last main split
// of each (b, h) runs the window too and gets that much less of the grouped
// region (the wavefronts of a split share its tiles as they go, so the
// window's cost spreads over all of them). A window tile's wavefront waits on
// several dependent memory round trips while the others stream: in a traced
// 32K decode the last split still ended about 2.4 µs after the first at 4,
// and 8 measured faster than 4, 12 and 16.
#ifndef KVQ_WINDOW_TILE_COST
#define KVQ_WINDOW_TILE_COST 8
#endif
constexpr int64_t kFallbackWorkgroups = 2048;
constexpr int64_t kMinTilesPerSplit = 4;   // one tile per wavefront at least

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

bool is_fp8(int32_t format) { return format == KVQ_FMT_FP8_E4M3 || format == KVQ_FMT_FP8_E5M2; }

// KV heads with their own FP8 scale row (1: one row for the tensor)
int64_t fp8_scale_rows(const kvq_config& c) { return c.scale_per_head ? c.num_kv_heads : 1; }

kvq_status validate_config(const kvq_config* c) {
  if (c == nullptr) return KVQ_ERR_INVALID_ARG;
  if (c->format != KVQ_FMT_FP16 && c->format != KVQ_FMT_KIVI && !is_fp8(c->format))
    return KVQ_ERR_INVALID_ARG;
  if (c->batch <= 0 || c->num_kv_heads <= 0 || c->head_dim <= 0 || c->capacity <= 0)
    return KVQ_ERR_INVALID_ARG;
  if (c->head_dim != kHeadDim) return KVQ_ERR_UNSUPPORTED;
  if (c->deterministic != 0 && c->deterministic != 1) return KVQ_ERR_UNSUPPORTED;
  switch (c->format) {
    case KVQ_FMT_KIVI:
      if (c->group_size <= 0 || c->residual_length < 0) return KVQ_ERR_INVALID_ARG;
      if (c->group_size != 32 && c->group_size != 64 && c->group_size != 128)
        return KVQ_ERR_UNSUPPORTED;
      if (c->bits != 2 && c->bits != 4) return KVQ_ERR_UNSUPPORTED;
      if (c->v_bits != 0 && c->v_bits != 2 && c->v_bits != 4) return KVQ_ERR_UNSUPPORTED;
      if (c->v_group_channels != 0 && c->v_group_channels != 32) return KVQ_ERR_UNSUPPORTED;
      if (c->residual_length % c->group_size != 0) return KVQ_ERR_UNSUPPORTED;
      break;
    case KVQ_FMT_FP8_E4M3:
    case KVQ_FMT_FP8_E5M2:
      if (c->bits != 8) return KVQ_ERR_UNSUPPORTED;
      if (c->scale_per_head != 0 && c->scale_per_head != 1) return KVQ_ERR_UNSUPPORTED;
      if (c->fp8_attention != 0 && c->fp8_attention != 1) return KVQ_ERR_UNSUPPORTED;
      break;
    default:
      if (c->bits != 16) return KVQ_ERR_UNSUPPORTED;
  }
  // paged grouped region (KIVI): P a power of two ≥ 32, whole groups per page
  if (c->page_tokens < 0) return KVQ_ERR_INVALID_ARG;
  if (c->page_tokens > 0) {
    const int32_t P = c->page_tokens;
    if (c->format != KVQ_FMT_KIVI) return KVQ_ERR_UNSUPPORTED;
    if (P < kGroup || P > (1 << 24) || (P & (P - 1)) != 0 || P % c->group_size != 0)
      return KVQ_ERR_UNSUPPORTED;
    if (c->num_pages <= 0) return KVQ_ERR_INVALID_ARG;
    if (double(c->num_pages) * c->num_kv_heads * P * c->head_dim > 9.0e15)
      return KVQ_ERR_UNSUPPORTED;
  }
  // grid dimension y carries B·H
  if (int64_t(c->batch) * c->num_kv_heads > 65535) return KVQ_ERR_UNSUPPORTED;
  // keep every element index well inside int64
  const double elems = double(c->batch) * c->num_kv_heads * (double(c->capacity) + 128) *
                       c->head_dim;
  if (elems > 9.0e15) return KVQ_ERR_UNSUPPORTED;
  return KVQ_OK;
}

// G: tokens per K scale group (KIVI), or the 32-token tile (FP8 / FP16);
// NG = ⌈C/G⌉ group slots, CT = NG·G token slots, NT = CT/32 tiles of 32 tokens.
struct Dims {
  int64_t B, H, D, C, G, NG, CT, NT, Rcap, bits, vbits, nvs;
  // paged KIVI: P tokens per page, NP pages, max_pages table entries per sequence
  int64_t P, NP, max_pages;
};

int ilog2(int64_t x) {
  int n = 0;
  while ((int64_t(1) << (n + 1)) <= x) ++n;
  return n;
}

Dims dims_of(const kvq_config& c) {
  Dims d;
  d.B = c.batch;
  d.H = c.num_kv_heads;
  d.D = c.head_dim;
  d.C = c.capacity;
  d.G = c.format == KVQ_FMT_KIVI ? c.group_size : kGroup;
  d.NG = ceil_div(c.capacity, d.G);
  d.CT = d.NG * d.G;
  d.NT = d.CT / kGroup;
  d.Rcap = c.residual_length > 0 ? c.residual_length : d.G;
  d.bits = c.bits;
  d.vbits = (c.format == KVQ_FMT_KIVI && c.v_bits > 0) ? c.v_bits : c.bits;
  d.nvs = (c.format == KVQ_FMT_KIVI && c.v_group_channels > 0) ? c.head_dim / c.v_group_channels
                                                              : 1;
  d.P = c.format == KVQ_FMT_KIVI ? c.page_tokens : 0;
  d.NP = d.P > 0 ? c.num_pages : 0;
  d.max_pages = d.P > 0 ? ceil_div(c.capacity, d.P) : 0;
  return d;
}

kvq_status device_status(hipError_t e) { return e == hipSuccess ? KVQ_OK : KVQ_ERR_DEVICE; }

// Kernels use 16-byte vector loads and stores.
bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

bool is_paged(const kvq_cache* c) {
  return c->cfg.format == KVQ_FMT_KIVI && c->cfg.page_tokens > 0;
}

bool buffers_set(const kvq_cache* c) {
  if (c->k_codes == nullptr || c->v_codes == nullptr) return false;
  if (!aligned16(c->k_codes) || !aligned16(c->v_codes)) return false;
  if (c->cfg.format == KVQ_FMT_KIVI) {
    const void* p[6] = {c->k_scale, c->k_zero, c->v_scale, c->v_zero, c->k_resid, c->v_resid};
    for (const void* x : p)
      if (x == nullptr || !aligned16(x)) return false;
    // a paged cache has its block table, and per-sequence fill levels
    if (is_paged(c))
      return c->block_table != nullptr && (reinterpret_cast<uintptr_t>(c->block_table) & 3u) == 0 &&
             c->seq_n_quant != nullptr && c->seq_n_resid != nullptr;
    return true;
  }
  if (is_fp8(c->cfg.format)) return c->tensor_scale != nullptr && aligned16(c->tensor_scale);
  return true;
}

bool is_ragged(const kvq_cache* c) {
  return c->seq_n_quant != nullptr && c->seq_n_resid != nullptr;
}

// One sequence's KIVI fill levels are reachable ones.
bool kivi_levels_ok(int64_t nq, int64_t nr, const Dims& d) {
  return nq >= 0 && nr >= 0 && nq + nr <= d.C && nq % d.G == 0 && nr <= d.Rcap;
}

// The host-side fill state must be one the state machine can reach; a
// corrupted struct is rejected before it can steer a kernel out of bounds.
// A ragged cache is KIVI with at most kMaxRagged sequences, zero scalar
// levels and reachable levels per sequence (only one of the two arrays set
// is not a state at all).
bool state_ok(const kvq_cache* c, const Dims& d) {
  if ((c->seq_n_quant == nullptr) != (c->seq_n_resid == nullptr)) return false;
  if (is_ragged(c)) {
    if (c->cfg.format != KVQ_FMT_KIVI || d.B > kvq::kMaxRagged) return false;
    if (c->n_quant != 0 || c->n_resid != 0) return false;
    for (int64_t b = 0; b < d.B; ++b)
      if (!kivi_levels_ok(c->seq_n_quant[b], c->seq_n_resid[b], d)) return false;
    return true;
  }
  if (c->n_quant < 0 || c->n_resid < 0 || c->n_quant + c->n_resid > d.C) return false;
  if (c->cfg.format == KVQ_FMT_KIVI) return c->n_quant % d.G == 0 && c->n_resid <= d.Rcap;
  return c->n_resid == 0;
}

// n_quant of a prefill of S tokens: G·max(0, min(⌊S/G⌋, ⌈(S−R)/G⌉)).
int64_t prefill_quant_tokens(int64_t S, int64_t R, int64_t G) {
  int64_t need = S > R ? ceil_div(S - R, G) : 0;
  const int64_t full = S / G;
  if (need > full) need = full;
  return need * G;
}

// The quantize launch block of a KIVI cache (source and group range unset).
kvq::KiviQuantArgs kivi_quant_args(const kvq_cache* c, const Dims& d) {
  kvq::KiviQuantArgs qa{};
  qa.bh_count = int(d.B * d.H);
  qa.bits = int(d.bits);
  qa.vbits = int(d.vbits);
  qa.NG = d.NG;
  qa.NT = d.NT;
  if (d.P > 0) {            // a block is one (page, h): a page's groups and tiles
    qa.paged = 1;
    qa.NG = d.P / d.G;
    qa.NT = d.P / kGroup;
    qa.block_table = c->block_table;
    qa.max_pages = int(d.max_pages);
    qa.page_group_shift = ilog2(d.P / d.G);
    qa.num_pages = int(d.NP);
  }
  qa.group = int(d.G);
  qa.nvs = int(d.nvs);
  qa.H = int(d.H);
  qa.k_codes = static_cast<uint32_t*>(c->k_codes);
  qa.v_codes = static_cast<uint32_t*>(c->v_codes);
  qa.k_scale = c->k_scale;
  qa.k_zero = c->k_zero;
  qa.v_scale = c->v_scale;
  qa.v_zero = c->v_zero;
  return qa;
}

// V of an FP8 / FP16 cache: source tokens [0, n) of an fp16 [B·H][..][D]
// tensor (bh stride in elements) into cache tokens [t0, t0 + n).
kvq::VTileArgs v_tile_args(const kvq_cache* c, const Dims& d, const __half* v,
                           int64_t src_bh_stride, int64_t n, int64_t t0, bool zero_tail) {
  kvq::VTileArgs a{};
  a.v_src = v;
  a.src_bh_stride = src_bh_stride;
  a.n_tokens = n;
  a.dst_t0 = t0;
  a.v_dst = c->v_codes;
  a.NT = d.NT;
  a.bh_count = int(d.B * d.H);
  a.H = int(d.H);
  a.fp8 = is_fp8(c->cfg.format) ? 1 : 0;
  a.fmt = c->cfg.format == KVQ_FMT_FP8_E5M2 ? kvq::kE5M2 : kvq::kE4M3;
  a.scale_stride = c->cfg.scale_per_head ? 4 : 0;
  a.zero_tail = zero_tail ? 1 : 0;
  a.tensor_scale = c->tensor_scale;
  return a;
}

// Query heads one decode workgroup handles: the largest power of two ≤ 8
// dividing Hq / H.
int heads_per_chunk(int nq) {
  for (int c = 8; c > 1; c >>= 1)
    if (nq % c == 0) return c;
  return 1;
}

struct Plan {
  int tiles_per_split, n_split_main, n_split, win_split, hpc, nchunk;
};

Plan make_plan(const Dims& d, int nq, int64_t n_main, int n_win, int64_t target) {
  Plan p;
  p.hpc = heads_per_chunk(nq);
  p.nchunk = nq / p.hpc;
  const int64_t tiles = ceil_div(n_main, kGroup);
  const int64_t x = d.B * d.H * p.nchunk;
  if (target <= 0) target = kFallbackWorkgroups;
  if (target > kMaxTargetWorkgroups) target = kMaxTargetWorkgroups;
  // a non-empty window joins the last main split of (b, h) when there is one
  const bool fold = n_win > 0 && tiles > 0;
  const int64_t win_cost =
      fold ? KVQ_WINDOW_TILE_COST * ceil_div(n_win, kGroup) : 0;
  int64_t tps = ceil_div((tiles + win_cost) * x, target);
  // no more splits per (b, h) than whole rounds of the target allow
  if (x <= target && tiles > 0) tps = std::max(tps, ceil_div(tiles, target / x));
  if (tps < kMinTilesPerSplit) tps = kMinTilesPerSplit;
  // whole K groups per split (G > 32: the decode keeps a group's score
  // operands across its tiles)
  tps = ceil_div(tps, d.G / kGroup) * (d.G / kGroup);
  p.tiles_per_split = int(tps);
  p.n_split_main = int(ceil_div(tiles, tps));
  if (fold) {
    p.n_split = p.n_split_main;
    p.win_split = p.n_split_main - 1;
  } else {
    p.n_split = p.n_split_main + (n_win > 0 ? 1 : 0);
    p.win_split = n_win > 0 ? p.n_split_main : -1;
  }
  return p;
}

// Upper bound of Plan::n_split over every fill state of this configuration:
// n_split_main ≤ ⌊target / x⌋ + 1 and ≤ ⌈max tiles / 4⌉, plus the window split.
int64_t max_splits(const Dims& d, int nq) {
  const int hpc = heads_per_chunk(nq);
  const int64_t x = d.B * d.H * (nq / hpc);
  const int64_t max_tiles = d.CT / kGroup;
  int64_t a = kMaxTargetWorkgroups / x + 1;
  const int64_t b = ceil_div(max_tiles, kMinTilesPerSplit);
  if (b < a) a = b;
  return a + 1;
}

// Split plan of a ragged KIVI batch: one tile count per split over all
// sequences, sized like make_plan from the total work (tiles plus window
// cost) of the batch, but never more splits than the workspace bound allows
// for the longest sequence. Sequence b uses splits [0, ⌈tiles_b / tps⌉); its
// window joins its last one (split 0 when it has no tiles).
Plan make_plan_ragged(const Dims& d, int nq, const kvq_cache* c, int64_t target) {
  Plan p;
  p.hpc = heads_per_chunk(nq);
  p.nchunk = nq / p.hpc;
  if (target <= 0) target = kFallbackWorkgroups;
  if (target > kMaxTargetWorkgroups) target = kMaxTargetWorkgroups;
  int64_t total = 0, max_tiles = 0;
  for (int64_t b = 0; b < d.B; ++b) {
    const int64_t tiles = c->seq_n_quant[b] / kGroup;
    const int64_t n_win = c->seq_n_resid[b];
    total += tiles;
    if (n_win > 0 && tiles > 0)
      total += KVQ_WINDOW_TILE_COST * ceil_div(n_win, kGroup);
    max_tiles = std::max(max_tiles, tiles);
  }
  int64_t tps = ceil_div(total * d.H * p.nchunk, target);
  tps = std::max(tps, ceil_div(max_tiles, max_splits(d, nq) - 1));
  if (tps < kMinTilesPerSplit) tps = kMinTilesPerSplit;
  // Each sequence's last split is a partial one, so the populated blocks can
  // outnumber the resident slots at this size: take the smallest size (binary
  // search; the count only falls as the size grows) whose populated blocks
  // fit in one round, when one exists.
  auto populated = [&](int64_t t) {
    int64_t n = 0;
    for (int64_t b = 0; b < d.B; ++b) {
      const int64_t tiles = c->seq_n_quant[b] / kGroup;
      n += tiles > 0 ? ceil_div(tiles, t) : 1;
    }
    return n * d.H * p.nchunk;
  };
  if (max_tiles > tps && populated(tps) > target && populated(max_tiles) <= target) {
    int64_t lo = tps, hi = max_tiles;          // populated(lo) > target >= populated(hi)
    while (hi - lo > 1) {
      const int64_t mid = lo + (hi - lo) / 2;
      if (populated(mid) <= target) hi = mid;
      else lo = mid;
    }
    tps = hi;
  }
  tps = ceil_div(tps, d.G / kGroup) * (d.G / kGroup);   // whole K groups per split
  p.tiles_per_split = int(tps);
  p.n_split_main = int(ceil_div(max_tiles, tps));
  p.n_split = std::max(p.n_split_main, 1);
  p.win_split = -1;
  return p;
}

}  // namespace

extern "C" {

int32_t kvq_abi_version(void) { return KVQ_ABI_VERSION; }

const char* kvq_status_str(kvq_status s) {
  switch (s) {
    case KVQ_OK: return "ok";
    case KVQ_ERR_INVALID_ARG: return "invalid argument";
    case KVQ_ERR_UNSUPPORTED: return "unsupported configuration";
    case KVQ_ERR_CAPACITY: return "cache capacity exceeded";
    case KVQ_ERR_STATE: return "invalid cache state for this call";
    case KVQ_ERR_DEVICE: return "HIP launch failed";
    case KVQ_ERR_WORKSPACE: return "decode workspace missing or too small";
  }
  return "unknown status";
}

kvq_status kvq_layout_query(const kvq_config* cfg, kvq_layout* out) {
  if (out == nullptr) return KVQ_ERR_INVALID_ARG;
  const kvq_status v = validate_config(cfg);
  if (v != KVQ_OK) return v;
  memset(out, 0, sizeof(*out));
  const Dims d = dims_of(*cfg);
  const size_t bh = size_t(d.B * d.H);
  switch (cfg->format) {
    case KVQ_FMT_KIVI: {
      // blocks of token slots: one per (b, h) of CT slots, or one per
      // (page, h) of P slots in a paged pool
      const size_t blocks = d.P > 0 ? size_t(d.NP * d.H) : bh;
      const size_t CT = d.P > 0 ? size_t(d.P) : size_t(d.CT);
      out->k_codes = blocks * CT * (d.D * d.bits / 32) * 4;
      out->v_codes = blocks * (CT / kGroup) * d.D * (kGroup * d.vbits / 32) * 4;
      out->k_scale = out->k_zero = blocks * (CT / d.G) * d.D * 4;
      out->v_scale = out->v_zero = blocks * CT * d.nvs * 4;
      out->k_resid = out->v_resid = bh * d.Rcap * d.D * 2;
      break;
    }
    case KVQ_FMT_FP8_E4M3:
    case KVQ_FMT_FP8_E5M2:
      out->k_codes = out->v_codes = bh * d.CT * d.D;
      out->tensor_scale = size_t(fp8_scale_rows(*cfg)) * 4 * sizeof(float);
      break;
    default:
      out->k_codes = out->v_codes = bh * d.CT * d.D * 2;
  }
  return KVQ_OK;
}

kvq_status kvq_cache_init(kvq_cache* cache, const kvq_config* cfg) {
  if (cache == nullptr) return KVQ_ERR_INVALID_ARG;
  const kvq_status v = validate_config(cfg);
  if (v != KVQ_OK) return v;
  memset(cache, 0, sizeof(*cache));
  cache->cfg = *cfg;
  return KVQ_OK;
}

kvq_status kvq_cache_reset(kvq_cache* cache) {
  if (cache == nullptr) return KVQ_ERR_INVALID_ARG;
  const kvq_status v = validate_config(&cache->cfg);
  if (v != KVQ_OK) return v;
  cache->n_quant = 0;
  cache->n_resid = 0;
  if (is_ragged(cache)) {
    if (cache->cfg.batch > kvq::kMaxRagged) return KVQ_ERR_UNSUPPORTED;
    for (int32_t b = 0; b < cache->cfg.batch; ++b) {
      cache->seq_n_quant[b] = 0;
      cache->seq_n_resid[b] = 0;
    }
  }
  return KVQ_OK;
}

kvq_status kvq_prefill_quantize(kvq_cache* cache, const void* k, const void* v,
                                int64_t seq_len, void* stream) {
  if (cache == nullptr || k == nullptr || v == nullptr) return KVQ_ERR_INVALID_ARG;
  if (!aligned16(k) || !aligned16(v)) return KVQ_ERR_INVALID_ARG;
  const kvq_status vs = validate_config(&cache->cfg);
  if (vs != KVQ_OK) return vs;
  if (!buffers_set(cache)) return KVQ_ERR_INVALID_ARG;
  if (seq_len <= 0) return KVQ_ERR_INVALID_ARG;
  if (is_ragged(cache)) return KVQ_ERR_INVALID_ARG;   // kvq_prefill_quantize_ragged
  const Dims d = dims_of(cache->cfg);
  if (!state_ok(cache, d)) return KVQ_ERR_STATE;
  if (seq_len > d.C) return KVQ_ERR_CAPACITY;
  if (cache->n_quant != 0 || cache->n_resid != 0) return KVQ_ERR_STATE;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int bh = int(d.B * d.H);
  const __half* kh = static_cast<const __half*>(k);
  const __half* vh = static_cast<const __half*>(v);

  if (cache->cfg.format == KVQ_FMT_KIVI) {
    // n_quant = G·max(0, min(⌊S/G⌋, ⌈(S−R)/G⌉)); the rest stays FP16.
    const int64_t R = cache->cfg.residual_length;
    int64_t need = seq_len > R ? ceil_div(seq_len - R, d.G) : 0;
    const int64_t full = seq_len / d.G;
    if (need > full) need = full;
    const int64_t nq = need * d.G;
    const int64_t nr = seq_len - nq;
    kvq::KiviQuantArgs qa{};
    qa.k_src = kh;
    qa.v_src = vh;
    qa.src_bh_stride = seq_len * d.D;
    qa.n_groups = int(nq / d.G);
    qa.g0 = 0;
    qa.bh_count = bh;
    qa.bits = int(d.bits);
    qa.vbits = int(d.vbits);
    qa.NG = d.NG;
    qa.NT = d.NT;
    qa.group = int(d.G);
    qa.nvs = int(d.nvs);
    qa.k_codes = static_cast<uint32_t*>(cache->k_codes);
    qa.v_codes = static_cast<uint32_t*>(cache->v_codes);
    qa.k_scale = cache->k_scale;
    qa.k_zero = cache->k_zero;
    qa.v_scale = cache->v_scale;
    qa.v_zero = cache->v_zero;
    hipError_t e = kvq::launch_kivi_quantize(qa, s);
    if (e != hipSuccess) return KVQ_ERR_DEVICE;
    kvq::CopyTokensArgs ca{};
    ca.k_src = kh + nq * d.D;
    ca.v_src = vh + nq * d.D;
    ca.src_bh_stride = seq_len * d.D;
    ca.k_dst = static_cast<__half*>(cache->k_resid);
    ca.v_dst = static_cast<__half*>(cache->v_resid);
    ca.dst_bh_stride = d.Rcap * d.D;
    ca.dst_t0 = 0;
    ca.n_tokens = nr;
    ca.bh_count = bh;
    e = kvq::launch_copy_tokens(ca, s);
    if (e != hipSuccess) return KVQ_ERR_DEVICE;
    cache->n_quant = nq;
    cache->n_resid = int32_t(nr);
    return KVQ_OK;
  }
  if (is_fp8(cache->cfg.format)) {
    kvq::Fp8QuantArgs fa{};
    fa.k_src = kh;
    fa.v_src = vh;
    fa.src_bh_stride = seq_len * d.D;
    fa.n_tokens = seq_len;
    fa.k_codes = static_cast<uint8_t*>(cache->k_codes);
    fa.v_codes = nullptr;                       // V goes to tiles below
    fa.dst_bh_stride = d.CT * d.D;
    fa.dst_t0 = 0;
    fa.bh_count = bh;
    fa.H = int(d.H);
    fa.fmt = cache->cfg.format == KVQ_FMT_FP8_E5M2 ? kvq::kE5M2 : kvq::kE4M3;
    fa.per_head = cache->cfg.scale_per_head;
    fa.tensor_scale = cache->tensor_scale;
    if (kvq::launch_fp8_prefill(fa, s) != hipSuccess) return KVQ_ERR_DEVICE;
    if (kvq::launch_v_tiles(v_tile_args(cache, d, vh, seq_len * d.D, seq_len, 0, true), s) !=
        hipSuccess)
      return KVQ_ERR_DEVICE;
    cache->n_quant = seq_len;
    return KVQ_OK;
  }
  kvq::CopyTokensArgs ca{};
  ca.k_src = kh;
  ca.v_src = vh;
  ca.src_bh_stride = seq_len * d.D;
  ca.k_dst = static_cast<__half*>(cache->k_codes);
  ca.v_dst = nullptr;                           // V goes to tiles below
  ca.dst_bh_stride = d.CT * d.D;
  ca.dst_t0 = 0;
  ca.n_tokens = seq_len;
  ca.bh_count = bh;
  if (kvq::launch_copy_tokens(ca, s) != hipSuccess) return KVQ_ERR_DEVICE;
  if (kvq::launch_v_tiles(v_tile_args(cache, d, vh, seq_len * d.D, seq_len, 0, true), s) !=
      hipSuccess)
    return KVQ_ERR_DEVICE;
  cache->n_quant = seq_len;
  return KVQ_OK;
}

kvq_status kvq_prefill_quantize_ragged(kvq_cache* cache, const void* k, const void* v,
                                       int64_t max_len, const int64_t* seq_lens,
                                       void* stream) {
  if (cache == nullptr || k == nullptr || v == nullptr || seq_lens == nullptr)
    return KVQ_ERR_INVALID_ARG;
  if (!aligned16(k) || !aligned16(v)) return KVQ_ERR_INVALID_ARG;
  const kvq_status vs = validate_config(&cache->cfg);
  if (vs != KVQ_OK) return vs;
  if (cache->cfg.format != KVQ_FMT_KIVI) return KVQ_ERR_UNSUPPORTED;
  if (cache->cfg.batch > kvq::kMaxRagged) return KVQ_ERR_UNSUPPORTED;
  if (!is_ragged(cache)) return KVQ_ERR_INVALID_ARG;
  if (!buffers_set(cache)) return KVQ_ERR_INVALID_ARG;
  if (max_len <= 0) return KVQ_ERR_INVALID_ARG;
  const Dims d = dims_of(cache->cfg);
  if (!state_ok(cache, d)) return KVQ_ERR_STATE;
  for (int64_t b = 0; b < d.B; ++b) {
    if (seq_lens[b] <= 0 || seq_lens[b] > max_len) return KVQ_ERR_INVALID_ARG;
  }
  for (int64_t b = 0; b < d.B; ++b) {
    if (seq_lens[b] > d.C) return KVQ_ERR_CAPACITY;
    if (cache->seq_n_quant[b] != 0 || cache->seq_n_resid[b] != 0) return KVQ_ERR_STATE;
  }
  hipStream_t s = static_cast<hipStream_t>(stream);
  const __half* kh = static_cast<const __half*>(k);
  const __half* vh = static_cast<const __half*>(v);
  kvq::KiviQuantArgs qa = kivi_quant_args(cache, d);
  qa.k_src = kh;
  qa.v_src = vh;
  qa.src_bh_stride = max_len * d.D;
  qa.ragged = 1;
  kvq::CopyTokensArgs ca{};
  ca.k_src = kh;
  ca.v_src = vh;
  ca.src_bh_stride = max_len * d.D;
  ca.k_dst = static_cast<__half*>(cache->k_resid);
  ca.v_dst = static_cast<__half*>(cache->v_resid);
  ca.dst_bh_stride = d.Rcap * d.D;
  ca.bh_count = int(d.B * d.H);
  ca.ragged = 1;
  ca.H = int(d.H);
  int64_t max_groups = 0, max_resid = 0;
  for (int64_t b = 0; b < d.B; ++b) {
    const int64_t nq = prefill_quant_tokens(seq_lens[b], cache->cfg.residual_length, d.G);
    qa.seq.x[b] = int32_t(nq / d.G);
    qa.seq.y[b] = 0;
    ca.seq.x[b] = int32_t(nq);
    ca.seq.y[b] = int32_t(seq_lens[b] - nq);
    ca.seq.z[b] = 0;
    max_groups = std::max(max_groups, nq / d.G);
    max_resid = std::max(max_resid, seq_lens[b] - nq);
  }
  qa.n_groups = int(max_groups);
  ca.n_tokens = max_resid;
  if (kvq::launch_kivi_quantize(qa, s) != hipSuccess) return KVQ_ERR_DEVICE;
  if (kvq::launch_copy_tokens(ca, s) != hipSuccess) return KVQ_ERR_DEVICE;
  for (int64_t b = 0; b < d.B; ++b) {
    cache->seq_n_quant[b] = int64_t(ca.seq.x[b]);
    cache->seq_n_resid[b] = ca.seq.y[b];
  }
  return KVQ_OK;
}

namespace {

// One token per sequence of a ragged KIVI cache; sequences with a full
// window flush it into their own next groups first.
kvq_status append_ragged(kvq_cache* cache, const Dims& d, const __half* kh, const __half* vh,
                         hipStream_t s) {
  for (int64_t b = 0; b < d.B; ++b)
    if (cache->seq_n_quant[b] + cache->seq_n_resid[b] >= d.C) return KVQ_ERR_CAPACITY;
  kvq::KiviQuantArgs qa = kivi_quant_args(cache, d);
  qa.k_src = static_cast<const __half*>(cache->k_resid);
  qa.v_src = static_cast<const __half*>(cache->v_resid);
  qa.src_bh_stride = d.Rcap * d.D;
  qa.ragged = 1;
  bool any_flush = false;
  for (int64_t b = 0; b < d.B; ++b) {
    const bool full = cache->seq_n_resid[b] == d.Rcap;
    qa.seq.x[b] = full ? int32_t(d.Rcap / d.G) : 0;
    qa.seq.y[b] = int32_t(cache->seq_n_quant[b] / d.G);
    any_flush = any_flush || full;
  }
  if (any_flush) {
    // one launch: the flushing sequences' groups, and every sequence's new
    // token (slot 0 after a flush, else after its window's last token)
    qa.n_groups = int(d.Rcap / d.G);
    qa.k_new = kh;
    qa.v_new = vh;
    qa.k_win = static_cast<__half*>(cache->k_resid);
    qa.v_win = static_cast<__half*>(cache->v_resid);
    qa.win_bh_stride = d.Rcap * d.D;
    for (int64_t b = 0; b < d.B; ++b) qa.seq.z[b] = qa.seq.x[b] > 0 ? 0 : cache->seq_n_resid[b];
    if (kvq::launch_kivi_quantize(qa, s) != hipSuccess) return KVQ_ERR_DEVICE;
    for (int64_t b = 0; b < d.B; ++b) {
      if (qa.seq.x[b] > 0) {
        cache->seq_n_quant[b] += d.Rcap;
        cache->seq_n_resid[b] = 0;
      }
      cache->seq_n_resid[b] += 1;
    }
    return KVQ_OK;
  }
  kvq::CopyTokensArgs ca{};
  ca.k_src = kh;
  ca.v_src = vh;
  ca.src_bh_stride = d.D;
  ca.k_dst = static_cast<__half*>(cache->k_resid);
  ca.v_dst = static_cast<__half*>(cache->v_resid);
  ca.dst_bh_stride = d.Rcap * d.D;
  ca.n_tokens = 1;
  ca.bh_count = int(d.B * d.H);
  ca.ragged = 1;
  ca.H = int(d.H);
  for (int64_t b = 0; b < d.B; ++b) {
    ca.seq.x[b] = 0;
    ca.seq.y[b] = 1;
    ca.seq.z[b] = cache->seq_n_resid[b];
  }
  if (kvq::launch_copy_tokens(ca, s) != hipSuccess) return KVQ_ERR_DEVICE;
  for (int64_t b = 0; b < d.B; ++b) cache->seq_n_resid[b] += 1;
  return KVQ_OK;
}

}  // namespace

// Every check of kvq_append_token, before anything is enqueued.
static kvq_status append_check(const kvq_cache* cache, const void* k_new, const void* v_new) {
  if (cache == nullptr || k_new == nullptr || v_new == nullptr) return KVQ_ERR_INVALID_ARG;
  if (!aligned16(k_new) || !aligned16(v_new)) return KVQ_ERR_INVALID_ARG;
  const kvq_status vs = validate_config(&cache->cfg);
  if (vs != KVQ_OK) return vs;
  if (!buffers_set(cache)) return KVQ_ERR_INVALID_ARG;
  const Dims d = dims_of(cache->cfg);
  if (!state_ok(cache, d)) return KVQ_ERR_STATE;
  if (is_ragged(cache)) {
    for (int64_t b = 0; b < d.B; ++b)
      if (cache->seq_n_quant[b] + cache->seq_n_resid[b] >= d.C) return KVQ_ERR_CAPACITY;
    return KVQ_OK;
  }
  if (cache->n_quant + cache->n_resid >= d.C) return KVQ_ERR_CAPACITY;
  if (is_fp8(cache->cfg.format) && cache->n_quant == 0) return KVQ_ERR_STATE;
  return KVQ_OK;
}

kvq_status kvq_append_token(kvq_cache* cache, const void* k_new, const void* v_new,
                            void* stream) {
  const kvq_status st = append_check(cache, k_new, v_new);
  if (st != KVQ_OK) return st;
  const Dims d = dims_of(cache->cfg);
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int bh = int(d.B * d.H);
  const __half* kh = static_cast<const __half*>(k_new);
  const __half* vh = static_cast<const __half*>(v_new);
  if (is_ragged(cache)) return append_ragged(cache, d, kh, vh, s);
  if (cache->n_quant + cache->n_resid >= d.C) return KVQ_ERR_CAPACITY;
  if (is_fp8(cache->cfg.format) && cache->n_quant == 0) return KVQ_ERR_STATE;

  if (cache->cfg.format == KVQ_FMT_KIVI) {
    if (cache->n_resid == d.Rcap) {   // lazy flush of the full window
      kvq::KiviQuantArgs qa{};
      qa.k_src = static_cast<const __half*>(cache->k_resid);
      qa.v_src = static_cast<const __half*>(cache->v_resid);
      qa.src_bh_stride = d.Rcap * d.D;
      qa.n_groups = int(d.Rcap / d.G);
      qa.g0 = cache->n_quant / d.G;
      qa.bh_count = bh;
      qa.bits = int(d.bits);
      qa.vbits = int(d.vbits);
      qa.NG = d.NG;
      qa.NT = d.NT;
      qa.group = int(d.G);
      qa.nvs = int(d.nvs);
      qa.k_codes = static_cast<uint32_t*>(cache->k_codes);
      qa.v_codes = static_cast<uint32_t*>(cache->v_codes);
      qa.k_scale = cache->k_scale;
      qa.k_zero = cache->k_zero;
      qa.v_scale = cache->v_scale;
      qa.v_zero = cache->v_zero;
      // the new token goes to window slot 0 in the same launch
      qa.k_new = kh;
      qa.v_new = vh;
      qa.k_win = static_cast<__half*>(cache->k_resid);
      qa.v_win = static_cast<__half*>(cache->v_resid);
      qa.win_bh_stride = d.Rcap * d.D;
      if (kvq::launch_kivi_quantize(qa, s) != hipSuccess) return KVQ_ERR_DEVICE;
      cache->n_quant += d.Rcap;
      cache->n_resid = 1;
      return KVQ_OK;
    }
    kvq::CopyTokensArgs ca{};
    ca.k_src = kh;
    ca.v_src = vh;
    ca.src_bh_stride = d.D;
    ca.k_dst = static_cast<__half*>(cache->k_resid);
    ca.v_dst = static_cast<__half*>(cache->v_resid);
    ca.dst_bh_stride = d.Rcap * d.D;
    ca.dst_t0 = cache->n_resid;
    ca.n_tokens = 1;
    ca.bh_count = bh;
    if (kvq::launch_copy_tokens(ca, s) != hipSuccess) return KVQ_ERR_DEVICE;
    cache->n_resid += 1;
    return KVQ_OK;
  }
  if (is_fp8(cache->cfg.format)) {
    kvq::Fp8QuantArgs fa{};
    fa.k_src = kh;
    fa.v_src = vh;
    fa.src_bh_stride = d.D;
    fa.n_tokens = 1;
    fa.k_codes = static_cast<uint8_t*>(cache->k_codes);
    fa.v_codes = nullptr;
    fa.dst_bh_stride = d.CT * d.D;
    fa.dst_t0 = cache->n_quant;
    fa.bh_count = bh;
    fa.H = int(d.H);
    fa.fmt = cache->cfg.format == KVQ_FMT_FP8_E5M2 ? kvq::kE5M2 : kvq::kE4M3;
    fa.per_head = cache->cfg.scale_per_head;
    fa.tensor_scale = cache->tensor_scale;
    if (kvq::launch_fp8_append(fa, s) != hipSuccess) return KVQ_ERR_DEVICE;
    if (kvq::launch_v_tiles(v_tile_args(cache, d, vh, d.D, 1, cache->n_quant, false), s) !=
        hipSuccess)
      return KVQ_ERR_DEVICE;
    cache->n_quant += 1;
    return KVQ_OK;
  }
  kvq::CopyTokensArgs ca{};
  ca.k_src = kh;
  ca.v_src = vh;
  ca.src_bh_stride = d.D;
  ca.k_dst = static_cast<__half*>(cache->k_codes);
  ca.v_dst = nullptr;
  ca.dst_bh_stride = d.CT * d.D;
  ca.dst_t0 = cache->n_quant;
  ca.n_tokens = 1;
  ca.bh_count = bh;
  if (kvq::launch_copy_tokens(ca, s) != hipSuccess) return KVQ_ERR_DEVICE;
  if (kvq::launch_v_tiles(v_tile_args(cache, d, vh, d.D, 1, cache->n_quant, false), s) !=
      hipSuccess)
    return KVQ_ERR_DEVICE;
  cache->n_quant += 1;
  return KVQ_OK;
}

size_t kvq_decode_workspace_bytes(const kvq_config* cfg, int32_t num_q_heads) {
  if (validate_config(cfg) != KVQ_OK) return 0;
  if (num_q_heads <= 0 || num_q_heads % cfg->num_kv_heads != 0) return 0;
  const Dims d = dims_of(*cfg);
  const int nq = num_q_heads / cfg->num_kv_heads;
  return size_t(d.B) * num_q_heads * max_splits(d, nq) * (kHeadDim + 2) * sizeof(float);
}

}  // extern "C"

// Every check of one decode call but the workspace's, before anything is
// enqueued.
static kvq_status decode_check_args(const kvq_cache* cache, const float* q, int32_t num_q_heads,
                                    float* out) {
  if (cache == nullptr || q == nullptr || out == nullptr) return KVQ_ERR_INVALID_ARG;
  if (!aligned16(q) || !aligned16(out)) return KVQ_ERR_INVALID_ARG;
  const kvq_status vs = validate_config(&cache->cfg);
  if (vs != KVQ_OK) return vs;
  if (!buffers_set(cache)) return KVQ_ERR_INVALID_ARG;
  if (num_q_heads <= 0) return KVQ_ERR_INVALID_ARG;
  if (num_q_heads % cache->cfg.num_kv_heads != 0) return KVQ_ERR_UNSUPPORTED;
  if (!state_ok(cache, dims_of(cache->cfg))) return KVQ_ERR_STATE;
  const bool ragged = is_ragged(cache);
  if (ragged) {
    for (int32_t b = 0; b < cache->cfg.batch; ++b)
      if (cache->seq_n_quant[b] + cache->seq_n_resid[b] <= 0) return KVQ_ERR_STATE;
  } else if (cache->n_quant + cache->n_resid <= 0) {
    return KVQ_ERR_STATE;
  }
  return KVQ_OK;
}

// Every check of one decode call with a caller's workspace.
static kvq_status decode_check(const kvq_cache* cache, const float* q, int32_t num_q_heads,
                               float* out, void* workspace, size_t workspace_bytes) {
  const kvq_status st = decode_check_args(cache, q, num_q_heads, out);
  if (st != KVQ_OK) return st;
  const size_t need = kvq_decode_workspace_bytes(&cache->cfg, num_q_heads);
  if (workspace == nullptr || workspace_bytes < need || !aligned16(workspace))
    return KVQ_ERR_WORKSPACE;
  return KVQ_OK;
}

// The launches of one checked decode call (dry: plan only, enqueue nothing).
// WORKSPACE when the plan's partials do not fit in workspace_bytes.
static kvq_status decode_enqueue(const kvq_cache* cache, const float* q, int32_t num_q_heads,
                                 float* out, void* workspace, size_t workspace_bytes,
                                 void* stream, bool dry, const __half* k_new = nullptr,
                                 const __half* v_new = nullptr) {
  const bool ragged = is_ragged(cache);

  const Dims d = dims_of(cache->cfg);
  const int nq = num_q_heads / int(d.H);
  const bool kivi = cache->cfg.format == KVQ_FMT_KIVI;
  const int n_win = kivi ? cache->n_resid : 0;
  kvq::DecodeArgs a{};
  a.src = kivi ? (d.bits == 2 ? kvq::kSrcKivi2 : kvq::kSrcKivi4)
       : cache->cfg.format == KVQ_FMT_FP8_E4M3 ? kvq::kSrcFp8
       : cache->cfg.format == KVQ_FMT_FP8_E5M2 ? kvq::kSrcE5M2
                                               : kvq::kSrcFp16;
  a.kbits = int(d.bits);
  a.vbits = int(d.vbits);
  a.nvs = int(d.nvs);
  a.qfp8 = is_fp8(cache->cfg.format) && cache->cfg.fp8_attention ? 1 : 0;
  // Unit-sized workgroups when every (b, h, head chunk) block can have a
  // compute unit to itself, four-wavefront ones otherwise. KIVI: either
  // order of tiles; FP8: only for caches that need not be deterministic (the
  // unit shape pays only with tiles shared); FP16: four wavefronts always.
  if (kivi || (is_fp8(cache->cfg.format) && !cache->cfg.deterministic)) {
    const int64_t x = d.B * d.H * (nq / heads_per_chunk(nq));
    const int cus = kvq::device_compute_units();
    a.unit = cus > 0 && x <= cus ? 1 : 0;
  }
  int64_t target = int64_t(kvq::decode_resident_workgroups(a)) * KVQ_SPLIT_ROUNDS;
  // KVQ_DECODE_TARGET_WORKGROUPS (environment, read per call) replaces the
  // workgroup target: the same cache can then be decoded under other split
  // plans (a test of the split merge) or the plan tuned without a rebuild
  if (const char* env = getenv("KVQ_DECODE_TARGET_WORKGROUPS")) {
    const long t = strtol(env, nullptr, 10);
    if (t > 0) target = t;
  }
  const Plan p = ragged ? make_plan_ragged(d, nq, cache, target)
                        : make_plan(d, nq, cache->n_quant, n_win, target);
  if (p.n_split > max_splits(d, nq)) return KVQ_ERR_WORKSPACE;
  const double part_bytes =
      double(d.B) * num_q_heads * p.n_split * (kHeadDim + 2) * sizeof(float);
  if (part_bytes > double(workspace_bytes)) return KVQ_ERR_WORKSPACE;
  if (dry) return KVQ_OK;

  a.B = int(d.B);
  a.H = int(d.H);
  a.Hq = num_q_heads;
  a.nq = nq;
  a.heads_per_chunk = p.hpc;
  a.k_main = cache->k_codes;
  a.v_main = cache->v_codes;
  a.k_scale = cache->k_scale;
  a.k_zero = cache->k_zero;
  a.v_scale = cache->v_scale;
  a.v_zero = cache->v_zero;
  a.tensor_scale = cache->tensor_scale;
  a.scale_stride = is_fp8(cache->cfg.format) && cache->cfg.scale_per_head ? 4 : 0;
  a.NG = d.NG;
  a.NT = d.NT;
  a.gshift = d.G == 128 ? 2 : d.G == 64 ? 1 : 0;
  a.main_bh_tokens = d.CT;
  if (d.P > 0) {            // blocks are (page, h): a page's groups, tiles, slots
    a.paged = 1;
    a.NG = d.P / d.G;
    a.NT = d.P / kGroup;
    a.main_bh_tokens = d.P;
    a.block_table = cache->block_table;
    a.max_pages = int(d.max_pages);
    a.page_tile_shift = ilog2(d.P / kGroup);
    a.num_pages = int(d.NP);
  }
  a.n_main = cache->n_quant;
  a.k_win = static_cast<const __half*>(cache->k_resid);
  a.v_win = static_cast<const __half*>(cache->v_resid);
  a.win_cap = int(d.Rcap);
  a.n_win = n_win;
  a.tiles_per_split = p.tiles_per_split;
  a.n_split_main = p.n_split_main;
  a.n_split = p.n_split;
  a.win_split = p.win_split;
  a.fixed_order = cache->cfg.deterministic;
  if (ragged) {
    a.ragged = 1;
    for (int64_t b = 0; b < d.B; ++b) {
      a.seq.x[b] = int32_t(cache->seq_n_quant[b] / kGroup);
      a.seq.y[b] = cache->seq_n_resid[b];
    }
  }
  if (k_new != nullptr) {   // the token just appended, stored by this launch
    a.k_new = k_new;
    a.v_new = v_new;
    a.k_win_store = static_cast<__half*>(cache->k_resid);
    a.v_win_store = static_cast<__half*>(cache->v_resid);
  }
  a.q = q;
  a.out = out;
  a.ws = static_cast<float*>(workspace);
  a.qscale = float(1.4426950408889634 / sqrt(double(kHeadDim)));
  return device_status(kvq::launch_decode(a, static_cast<hipStream_t>(stream)));
}

extern "C" {

kvq_status kvq_decode_attention(const kvq_cache* cache, const float* q, int32_t num_q_heads,
                                float* out, void* workspace, size_t workspace_bytes,
                                void* stream) {
  const kvq_status st = decode_check(cache, q, num_q_heads, out, workspace, workspace_bytes);
  if (st != KVQ_OK) return st;
  return decode_enqueue(cache, q, num_q_heads, out, workspace, workspace_bytes, stream, false);
}

kvq_status kvq_append_decode(kvq_cache* cache, const void* k_new, const void* v_new,
                             const float* q, int32_t num_q_heads, float* out, void* workspace,
                             size_t workspace_bytes, void* stream) {
  kvq_status st = append_check(cache, k_new, v_new);
  if (st != KVQ_OK) return st;
  // the fill state after the append, on a copy (a ragged cache's levels in
  // local arrays): the decode is checked and planned on it before anything
  // is enqueued
  const Dims d = dims_of(cache->cfg);
  const bool ragged = is_ragged(cache);
  const bool kivi = cache->cfg.format == KVQ_FMT_KIVI;
  kvq_cache after = *cache;
  int64_t nq_after[kvq::kMaxRagged];
  int32_t nr_after[kvq::kMaxRagged];
  bool flush = false;
  if (ragged) {
    for (int64_t b = 0; b < d.B; ++b) {
      const bool full = cache->seq_n_resid[b] == d.Rcap;
      flush = flush || full;
      nq_after[b] = cache->seq_n_quant[b] + (full ? d.Rcap : 0);
      nr_after[b] = (full ? 0 : cache->seq_n_resid[b]) + 1;
    }
    after.seq_n_quant = nq_after;
    after.seq_n_resid = nr_after;
  } else if (kivi) {
    flush = cache->n_resid == d.Rcap;
    after.n_quant = cache->n_quant + (flush ? d.Rcap : 0);
    after.n_resid = (flush ? 0 : cache->n_resid) + 1;
  } else {
    after.n_quant = cache->n_quant + 1;
  }
  st = decode_check(&after, q, num_q_heads, out, workspace, workspace_bytes);
  if (st != KVQ_OK) return st;
  st = decode_enqueue(&after, q, num_q_heads, out, workspace, workspace_bytes, stream, true,
                      nullptr, nullptr);
  if (st != KVQ_OK) return st;
  if (!kivi || flush) {
    // a flush (or an FP8 / FP16 append) goes first in launches of its own
    st = kvq_append_token(cache, k_new, v_new, stream);
    if (st != KVQ_OK) return st;
    return decode_enqueue(cache, q, num_q_heads, out, workspace, workspace_bytes, stream, false,
                          nullptr, nullptr);
  }
  // one launch: the decode stores the token into its window slot itself
  if (ragged) {
    for (int64_t b = 0; b < d.B; ++b) cache->seq_n_resid[b] += 1;
  } else {
    cache->n_resid += 1;
  }
  return decode_enqueue(cache, q, num_q_heads, out, workspace, workspace_bytes, stream, false,
                        static_cast<const __half*>(k_new), static_cast<const __half*>(v_new));
}

kvq_status kvq_decode_attention_static(const kvq_cache* cache, const float* q,
                                       int32_t num_q_heads, float* out, void* stream) {
  const kvq_status st = decode_check_args(cache, q, num_q_heads, out);
  if (st != KVQ_OK) return st;
  void* ws = nullptr;
  if (kvq::static_workspace(&ws) != hipSuccess) return KVQ_ERR_DEVICE;
  return decode_enqueue(cache, q, num_q_heads, out, ws, KVQ_STATIC_WORKSPACE_BYTES, stream,
                        false);
}

kvq_status kvq_decode_attention_layers(const kvq_cache* const* caches, int32_t n_layers,
                                       const float* q, int32_t num_q_heads, float* out,
                                       void* workspace, size_t workspace_bytes, void* stream) {
  if (caches == nullptr || n_layers < 1 || q == nullptr || out == nullptr)
    return KVQ_ERR_INVALID_ARG;
  // every layer checked and planned before the first launch
  int64_t row = 0;   // floats of one layer's q / out: B·Hq·D
  for (int32_t l = 0; l < n_layers; ++l) {
    const kvq_cache* c = caches[l];
    if (c == nullptr) return KVQ_ERR_INVALID_ARG;
    if (l > 0 && c->cfg.batch != caches[0]->cfg.batch) return KVQ_ERR_INVALID_ARG;
    const kvq_status st = decode_check(c, q + l * row, num_q_heads, out + l * row, workspace,
                                       workspace_bytes);
    if (st != KVQ_OK) return st;
    if (l == 0) row = int64_t(c->cfg.batch) * num_q_heads * kHeadDim;
  }
  for (int32_t l = 0; l < n_layers; ++l) {
    const kvq_status st = decode_enqueue(caches[l], q + l * row, num_q_heads, out + l * row,
                                         workspace, workspace_bytes, stream, true);
    if (st != KVQ_OK) return st;
  }
  for (int32_t l = 0; l < n_layers; ++l) {
    const kvq_status st = decode_enqueue(caches[l], q + l * row, num_q_heads, out + l * row,
                                         workspace, workspace_bytes, stream, false);
    if (st != KVQ_OK) return st;
  }
  return KVQ_OK;
}

kvq_status kvq_quantize_query_fp8(const float* q, int32_t batch, int32_t num_q_heads,
                                  int32_t head_dim, uint8_t* codes, float* scales,
                                  void* stream) {
  if (q == nullptr || codes == nullptr || scales == nullptr) return KVQ_ERR_INVALID_ARG;
  if (!aligned16(q) || !aligned16(codes) || (reinterpret_cast<uintptr_t>(scales) & 3u) != 0)
    return KVQ_ERR_INVALID_ARG;
  if (batch <= 0 || num_q_heads <= 0 || head_dim <= 0) return KVQ_ERR_INVALID_ARG;
  if (head_dim != kHeadDim) return KVQ_ERR_UNSUPPORTED;
  const int64_t rows = int64_t(batch) * num_q_heads;
  if (rows > 0x7FFFFFFF) return KVQ_ERR_UNSUPPORTED;
  kvq::QueryQuantArgs qa{};
  qa.q = q;
  qa.codes = codes;
  qa.scales = scales;
  qa.rows = rows;
  return device_status(kvq::launch_query_fp8(qa, static_cast<hipStream_t>(stream)));
}

int64_t kvq_decode_bytes(const kvq_cache* cache, int32_t num_q_heads) {
  if (cache == nullptr || validate_config(&cache->cfg) != KVQ_OK) return -1;
  if (num_q_heads <= 0 || num_q_heads % cache->cfg.num_kv_heads != 0) return -1;
  const Dims d = dims_of(cache->cfg);
  if (!state_ok(cache, d)) return -1;
  const int64_t bh = d.B * d.H;
  const int64_t nq = cache->n_quant;
  if (cache->cfg.format == KVQ_FMT_KIVI) {
    // per (b, h) with nq grouped and nr window tokens
    auto per_bh = [&](int64_t q, int64_t nr) {
      const int64_t code_bytes = q * d.D * (d.bits + d.vbits) / 8;   // K and V codes
      const int64_t k_meta = (q / d.G) * d.D * 2 * 4;        // fp32 s, z per channel
      const int64_t v_meta = q * 2 * 4 * d.nvs;              // fp32 s, z per token (run)
      const int64_t window = 2 * nr * d.D * 2;
      return code_bytes + k_meta + v_meta + window;
    };
    if (is_ragged(cache)) {
      int64_t sum = 0;
      for (int64_t b = 0; b < d.B; ++b) sum += per_bh(cache->seq_n_quant[b], cache->seq_n_resid[b]);
      return d.H * sum;
    }
    return bh * per_bh(nq, cache->n_resid);
  }
  if (is_fp8(cache->cfg.format)) return 2 * bh * nq * d.D + 2 * 4 * fp8_scale_rows(cache->cfg);
  return 2 * bh * nq * d.D * 2;
}

double kvq_theoretical_bytes(int32_t num_layers, int32_t batch, int64_t seq_len,
                             int32_t num_kv_heads, int32_t head_dim, double bytes_per_elem) {
  return 2.0 * num_layers * double(batch) * double(seq_len) * num_kv_heads * head_dim *
         bytes_per_elem;
}

double kvq_theoretical_bytes_layers(int32_t n_layers, int32_t batch, const int64_t* seq_len,
                                    const int32_t* num_kv_heads, const int32_t* head_dim,
                                    double bytes_per_elem) {
  if (n_layers < 1 || batch < 0 || seq_len == nullptr || num_kv_heads == nullptr ||
      head_dim == nullptr || !(bytes_per_elem >= 0.0))
    return -1.0;
  double tokens = 0.0;   // Σ_l S_l·H_kv,l·D_l
  for (int32_t l = 0; l < n_layers; ++l) {
    if (seq_len[l] < 0 || num_kv_heads[l] < 0 || head_dim[l] < 0) return -1.0;
    tokens += double(seq_len[l]) * num_kv_heads[l] * head_dim[l];
  }
  return 2.0 * double(batch) * bytes_per_elem * tokens;
}

}  // extern "C"
