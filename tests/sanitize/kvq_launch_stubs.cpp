// Host-only stand-ins for libkvq's device launches, linked with the C ABI
// (kvq_api.cpp) into a sanitizer build that runs on a machine without a GPU.
// Every stand-in checks that the launch block it receives stays inside the
// buffers the cache layout gives (ranges of group slots, window slots, split
// tiles, pages), counts the launch, and returns success without touching any
// device memory. A failed check aborts the process with a message.
#include <stdio.h>
#include <stdlib.h>

#include "../../kv_cache_quantization_quant_amd/csrc/kvq_internal.h"

extern "C" {
// launches seen, by kind (read by the driver)
long kvq_stub_launches[8];
}

namespace {

void require(bool ok, const char* what) {
  if (!ok) {
    fprintf(stderr, "launch check failed: %s\n", what);
    abort();
  }
}

// group slots a quantize launch may write: [0, NG) of each (b, h) block,
// or, paged, logical groups below max_pages pages
bool group_range_ok(const kvq::KiviQuantArgs& a, int64_t first, int64_t count) {
  if (first < 0 || count < 0) return false;
  if (!a.paged) return first + count <= a.NG;
  const int64_t per_page = int64_t(1) << a.page_group_shift;
  return per_page == a.NG && first + count <= int64_t(a.max_pages) * per_page &&
         a.num_pages >= 1 && a.block_table != nullptr;
}

}  // namespace

namespace kvq {

hipError_t launch_kivi_quantize(const KiviQuantArgs& a, hipStream_t) {
  ++kvq_stub_launches[0];
  require(a.group == 32 || a.group == 64 || a.group == 128, "quantize: group size");
  require(a.NT * kGroup == a.NG * a.group, "quantize: tiles per block");
  require(a.bits == 2 || a.bits == 4, "quantize: K bits");
  require(a.vbits == 2 || a.vbits == 4, "quantize: V bits");
  require(a.nvs == 1 || a.nvs == 4, "quantize: V scales per token");
  require(a.n_groups >= 0 && a.bh_count >= 1, "quantize: grid");
  require(a.src_bh_stride >= int64_t(a.n_groups) * a.group * kHeadDim, "quantize: source rows");
  if (a.ragged) {
    require(a.H >= 1 && a.bh_count % a.H == 0 && a.bh_count / a.H <= kMaxRagged,
            "quantize: ragged batch");
    for (int b = 0; b < a.bh_count / a.H; ++b) {
      require(a.seq.x[b] >= 0 && a.seq.x[b] <= a.n_groups, "quantize: ragged group count");
      require(group_range_ok(a, a.seq.y[b], a.seq.x[b]), "quantize: ragged group range");
    }
  } else {
    require(group_range_ok(a, a.g0, a.n_groups), "quantize: group range");
  }
  if (a.k_new != nullptr) {
    // the folded append: one token per (b, h) block into a window slot
    require(a.v_new != nullptr && a.k_win != nullptr && a.v_win != nullptr,
            "quantize: new token buffers");
    require(a.n_groups >= 1, "quantize: a group-0 workgroup per block writes the new token");
    require(a.win_bh_stride % kHeadDim == 0, "quantize: window rows");
    const int64_t cap = a.win_bh_stride / kHeadDim;
    if (a.ragged) {
      for (int b = 0; b < a.bh_count / a.H; ++b)
        require(a.seq.z[b] >= 0 && a.seq.z[b] < cap && (a.seq.x[b] == 0 || a.seq.z[b] == 0),
                "quantize: new token slot");
    } else {
      require(cap >= 1, "quantize: new token slot");
    }
  }
  return hipSuccess;
}

hipError_t launch_copy_tokens(const CopyTokensArgs& a, hipStream_t) {
  ++kvq_stub_launches[1];
  require(a.n_tokens >= 0 && a.bh_count >= 1, "copy: grid");
  require(a.dst_bh_stride % kHeadDim == 0, "copy: destination rows");
  const int64_t cap = a.dst_bh_stride / kHeadDim;     // token slots per (b, h)
  if (a.ragged) {
    for (int b = 0; b < a.bh_count / a.H; ++b) {
      require(a.seq.y[b] >= 0 && a.seq.y[b] <= a.n_tokens, "copy: ragged count");
      require(a.seq.z[b] >= 0 && a.seq.z[b] + a.seq.y[b] <= cap, "copy: ragged destination");
      require(a.seq.x[b] >= 0 && (a.seq.x[b] + a.seq.y[b]) * kHeadDim <= a.src_bh_stride,
              "copy: ragged source");
    }
  } else {
    require(a.dst_t0 >= 0 && a.dst_t0 + a.n_tokens <= cap, "copy: destination range");
    require(a.n_tokens * kHeadDim <= a.src_bh_stride, "copy: source range");
  }
  return hipSuccess;
}

hipError_t launch_v_tiles(const VTileArgs& a, hipStream_t) {
  ++kvq_stub_launches[2];
  require(a.dst_t0 >= 0 && a.n_tokens >= 0, "v tiles: range");
  require(a.dst_t0 + a.n_tokens <= a.NT * kGroup, "v tiles: destination");
  return hipSuccess;
}

hipError_t launch_fp8_prefill(const Fp8QuantArgs& a, hipStream_t) {
  ++kvq_stub_launches[3];
  require(a.dst_t0 == 0 && a.n_tokens * kHeadDim <= a.dst_bh_stride, "fp8 prefill: range");
  require(a.tensor_scale != nullptr, "fp8 prefill: scales");
  return hipSuccess;
}

hipError_t launch_fp8_append(const Fp8QuantArgs& a, hipStream_t) {
  ++kvq_stub_launches[4];
  require((a.dst_t0 + a.n_tokens) * kHeadDim <= a.dst_bh_stride, "fp8 append: range");
  return hipSuccess;
}

hipError_t launch_query_fp8(const QueryQuantArgs& a, hipStream_t) {
  ++kvq_stub_launches[5];
  require(a.rows >= 1, "query fp8: rows");
  return hipSuccess;
}

hipError_t launch_decode(const DecodeArgs& a, hipStream_t) {
  ++kvq_stub_launches[6];
  require(a.nq >= 1 && a.Hq == a.nq * a.H, "decode: heads");
  require(a.heads_per_chunk >= 1 && a.heads_per_chunk <= 8 && a.nq % a.heads_per_chunk == 0,
          "decode: head chunks");
  require(a.tiles_per_split >= 1, "decode: split size");
  require(a.n_split >= 1 && a.n_split_main >= 0 && a.n_split_main <= a.n_split &&
              a.n_split <= a.n_split_main + 1,
          "decode: split counts");
  require(a.win_split >= -1 && a.win_split < a.n_split, "decode: window split");
  require(a.n_split == 1 || a.ws != nullptr, "decode: workspace");
  if (a.k_new != nullptr) {
    // a folded append: KIVI, its token in window slot n_win - 1 of each block
    require(a.src == kSrcKivi2 || a.src == kSrcKivi4, "decode: folded append format");
    require(a.v_new != nullptr && a.k_win_store != nullptr && a.v_win_store != nullptr,
            "decode: folded append buffers");
    if (a.ragged) {
      for (int b = 0; b < a.B; ++b)
        require(a.seq.y[b] >= 1 && a.seq.y[b] <= a.win_cap, "decode: folded append slot");
    } else {
      require(a.n_win >= 1 && a.n_win <= a.win_cap, "decode: folded append slot");
    }
  }
  const int64_t per_block = a.paged ? int64_t(a.max_pages) * a.main_bh_tokens : a.main_bh_tokens;
  if (a.paged)
    require(a.main_bh_tokens == (int64_t(32) << a.page_tile_shift) && a.num_pages >= 1 &&
                a.block_table != nullptr,
            "decode: pages");
  auto tiles_ok = [&](int64_t tiles) {
    return tiles >= 0 && tiles * kGroup <= per_block &&
           tiles <= int64_t(a.n_split_main) * a.tiles_per_split;
  };
  if (a.ragged) {
    for (int b = 0; b < a.B; ++b) {
      require(tiles_ok(a.seq.x[b]), "decode: ragged tiles");
      require(a.seq.y[b] >= 0 && a.seq.y[b] <= a.win_cap, "decode: ragged window");
    }
  } else {
    require(a.n_main % kGroup == 0 || a.src == kSrcFp16 || a.src == kSrcFp8 || a.src == kSrcE5M2,
            "decode: grouped tokens");
    require(tiles_ok((a.n_main + kGroup - 1) / kGroup), "decode: tiles");
    require(a.n_win >= 0 && a.n_win <= a.win_cap, "decode: window");
    require(a.n_win == 0 || a.win_split >= 0, "decode: window has a split");
  }
  return hipSuccess;
}

int decode_resident_workgroups(const DecodeArgs& a) {
  return a.unit ? 256 : 768;     // the MI355X's compute units, one or three per unit
}

int device_compute_units() { return 256; }

hipError_t static_workspace(void** ptr) {
  static char host_stand_in[256];   // never dereferenced by the stand-ins
  *ptr = host_stand_in;
  return hipSuccess;
}

hipError_t launch_kivi_mfma(const DecodeArgs&, hipStream_t) { return hipSuccess; }
hipError_t launch_dense_mfma(const DecodeArgs&, hipStream_t) { return hipSuccess; }

}  // namespace kvq
