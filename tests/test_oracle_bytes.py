"""Pins of the oracle's byte accounting against the numbers the pages print."""
import json
import os

import pytest

from oracle import bytes_model as bm

GIB = 2 ** 30
KIB = 2 ** 10


@pytest.fixture(scope="module")
def pages(golden_dir):
    with open(os.path.join(golden_dir, "pages_worked_numbers.json")) as f:
        return json.load(f)


def test_per_token_mha(pages):
    e = pages["per_token_mha_bf16"]
    got = bm.kv_cache_bytes(e["layers"], e["batch"], 1, e["kv_heads"], e["head_dim"],
                            e["bytes_per_elem"])
    assert got == e["bytes"] == e["kib"] * KIB


def test_mha_context_table(pages):
    e = pages["mha_context_table_bf16_gib"]
    for S, gib in e["rows"]:
        got = bm.kv_cache_bytes(e["layers"], e["batch"], S, e["kv_heads"], e["head_dim"],
                                e["bytes_per_elem"])
        assert got == gib * GIB


def test_precision_table(pages):
    e = pages["precision_table_128k_gib"]
    for _, bpe, gib in e["rows"]:
        got = bm.kv_cache_bytes(e["layers"], e["batch"], e["seq_len"], e["kv_heads"],
                                e["head_dim"], bpe)
        assert got == gib * GIB


def test_gqa_vs_mha(pages):
    e = pages["gqa_vs_mha"]
    for hkv, kib in e["per_token_kib"]:
        assert bm.kv_cache_bytes(e["layers"], 1, 1, hkv, e["head_dim"],
                                 e["bytes_per_elem"]) == kib * KIB
    for hkv, gib in e["ctx_32k_gib"]:
        assert bm.kv_cache_bytes(e["layers"], 1, 32768, hkv, e["head_dim"],
                                 e["bytes_per_elem"]) == gib * GIB


def test_gqa_times_quant(pages):
    e = pages["gqa_times_quant_32k_gib"]
    for _, bpe, gib in e["rows"]:
        assert bm.kv_cache_bytes(e["layers"], 1, e["seq_len"], e["kv_heads"],
                                 e["head_dim"], bpe) == gib * GIB


def test_interview_example(pages):
    e = pages["interview_example"]
    assert bm.kv_elements_per_token(e["layers"], e["kv_heads"], e["head_dim"]) \
        == e["elements_per_token"]
    assert bm.kv_cache_bytes(e["layers"], 1, 1, e["kv_heads"], e["head_dim"], 2) \
        == e["fp16_kib_per_token"] * KIB
    assert bm.kv_cache_bytes(e["layers"], 1, 8192, e["kv_heads"], e["head_dim"], 2) \
        == e["ctx_8k_gib"] * GIB


def test_average_bits(pages):
    e = pages["residual_average_bits"]
    got = bm.average_bits(e["seq_len"], e["residual"], e["main_bits"], e["residual_bits"])
    assert round(got, 2) == e["average_bits_rounded_2dp"]
    # exact value of the page's expression
    assert got == (8064 * 4 + 128 * 16) / 8192


def test_metadata_overhead(pages):
    e = pages["metadata_overhead"]
    assert e["group"] * e["bits"] / 8 == e["data_bytes"]
    got = bm.metadata_overhead(e["group"], e["bits"], e["scale_bytes"], e["zero_bytes"])
    assert round(100 * got, 1) == e["overhead_percent_1dp"]


@pytest.mark.parametrize("bits", [2, 4])
def test_kivi_decode_bytes_decomposition(bits):
    """The KIVI step bytes split into the page formula's ideal code bytes, the
    metadata, and the fp16 window — each term checked on its own, so a dropped
    or doubled term fails."""
    B, H, D, G = 3, 5, 128, 32
    for nq, nr in [(0, 7), (64, 0), (4096, 128), (32640, 128)]:
        total = bm.decode_bytes_kivi(B, H, D, bits, G, nq, nr)
        ideal_codes = bm.kv_cache_bytes(1, B, nq, H, D, bits / 8)      # K and V codes
        k_meta = B * H * (nq // G) * D * 2 * 4                          # fp32 s, z per channel per group
        v_meta = B * H * nq * 2 * 4                                     # fp32 s, z per token
        window = bm.kv_cache_bytes(1, B, nr, H, D, 2)
        assert total == ideal_codes + k_meta + v_meta + window


def test_fp8_fp16_decode_bytes():
    assert bm.decode_bytes_fp16(2, 3, 128, 10) == bm.kv_cache_bytes(1, 2, 10, 3, 128, 2)
    assert bm.decode_bytes_fp8(2, 3, 128, 10) == bm.kv_cache_bytes(1, 2, 10, 3, 128, 1) + 8


# ---- decode step bytes of the benchmark workloads, worked out by hand ----
# Each total below is written out term by term from the workload's shape
# (prefill split: the newest 128 tokens stay in the fp16 window, the rest are
# whole 32-token groups), so a dropped, doubled or mis-scaled term of the
# byte model fails one of them. Per (b, KV head) block, with n = grouped
# tokens, r = window tokens, D = 128:
#   K codes n·D·b/8, K scale + zero (n/G)·D·4·2, V codes n·D·b_V/8,
#   V scale + zero n·4·2 (per run of channels with V sub-groups),
#   window 2·r·D·2.

def test_decode_bytes_llama2_7b_layer():
    # B=8, 32 MHA heads, S=4096, 2-bit: n = 3968, r = 128
    per = (3968 * 32          # K codes: 126,976
           + 124 * 1024       # K scale + zero: 126,976
           + 3968 * 32        # V codes: 126,976
           + 3968 * 8         # V scale + zero: 31,744
           + 65536)           # window: 65,536
    assert per == 478208
    assert bm.decode_bytes_kivi(8, 32, 128, 2, 32, 3968, 128) == 256 * per == 122421248


def test_decode_bytes_gqa_32k_layer():
    # B=16, 8 KV heads, S=32768, 2-bit, before the first append: n = 32640, r = 128
    per = 1044480 + 1044480 + 1044480 + 261120 + 65536
    assert per == 3460096
    assert bm.decode_bytes_kivi(16, 8, 128, 2, 32, 32640, 128) == 128 * per == 442892288
    # after the first append flushed the window: n = 32768, r = 1
    per1 = 1048576 + 1048576 + 1048576 + 262144 + 512
    assert bm.decode_bytes_kivi(16, 8, 128, 2, 32, 32768, 1) == 128 * per1 == 436273152


def test_decode_bytes_large_batch_4bit():
    # B=64, 32 heads, S=8192, 4-bit: n = 8064, r = 128
    per = (8064 * 64          # K codes: 516,096
           + 252 * 1024       # K scale + zero: 258,048
           + 8064 * 64        # V codes: 516,096
           + 8064 * 8         # V scale + zero: 64,512
           + 65536)
    assert per == 1420288
    assert bm.decode_bytes_kivi(64, 32, 128, 4, 32, 8064, 128) == 2048 * per == 2908749824


def test_decode_bytes_long_context_three_formats():
    # B=4, 8 KV heads, S=131072
    B, H, S = 4, 8, 131072
    # KIVI 2-bit: n = 130944, r = 128
    per = 4190208 + 4190208 + 4190208 + 1047552 + 65536
    assert per == 13683712
    assert bm.decode_bytes_kivi(B, H, 128, 2, 32, 130944, 128) == 32 * per == 437878784
    # FP8: one byte per K and V element, plus s_K and s_V (fp32)
    assert bm.decode_bytes_fp8(B, H, 128, S) == 1073741824 + 8 == 1073741832
    # FP8 with one (s_K, s_V) pair per KV head: 8 pairs
    assert bm.decode_bytes_fp8(B, H, 128, S, per_head=True) == 1073741824 + 64
    # FP16: two bytes per K and V element
    assert bm.decode_bytes_fp16(B, H, 128, S) == 2147483648


def test_decode_bytes_variant_terms():
    """The V width and V channel sub-group terms on the 32K GQA layer
    (n = 32640, r = 128), against hand-computed per-block bytes."""
    # K 4-bit / V 2-bit: K codes double, V codes stay
    per = 2088960 + 1044480 + 1044480 + 261120 + 65536
    assert bm.decode_bytes_kivi(16, 8, 128, 4, 32, 32640, 128, v_bits=2) == 128 * per == 576585728
    # K 2-bit / V 4-bit: the same total, the other side doubled
    per = 1044480 + 1044480 + 2088960 + 261120 + 65536
    assert bm.decode_bytes_kivi(16, 8, 128, 2, 32, 32640, 128, v_bits=4) == 128 * per
    # V scale and zero per run of 32 channels: four pairs per token
    per = 1044480 + 1044480 + 1044480 + 4 * 261120 + 65536
    assert bm.decode_bytes_kivi(16, 8, 128, 2, 32, 32640, 128, v_group_channels=32) \
        == 128 * per == 543162368
    # G = 64 and 128: K metadata halves / quarters, nothing else moves
    per64 = 1044480 + 1044480 // 2 + 1044480 + 261120 + 65536
    per128 = 1044480 + 1044480 // 4 + 1044480 + 261120 + 65536
    assert bm.decode_bytes_kivi(16, 8, 128, 2, 64, 32640, 128) == 128 * per64 == 376045568
    assert bm.decode_bytes_kivi(16, 8, 128, 2, 128, 32640, 128) == 128 * per128 == 342622208
