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
