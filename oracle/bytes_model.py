"""Byte accounting of a KV cache (oracle side).

kv_cache_bytes: the pages' formula, KV bytes = 2 · L · B · S · H_kv · D · b,
the leading 2 counting one K and one V ([KIVI-page] §1 equation;
[Tutorial] §四 and §四.1 per-token form; [Interview] §三).

decode_bytes_*: what one decode step must read from a cache in the layouts
this project defines (codes, fp32 scales and zero-points, fp16 window, FP8
codes plus two fp32 scales). [Tutorial] §四.3 and §十.4 warn that scales,
zero-points and the residual window add to the ideal size; these functions
count them.
"""
from __future__ import annotations


def kv_cache_bytes(num_layers: int, batch: int, seq_len: int, num_kv_heads: int,
                   head_dim: int, bytes_per_elem: float) -> float:
    """2 · L · B · S · H_kv · D · bytes ([Tutorial] §四)."""
    return 2.0 * num_layers * batch * seq_len * num_kv_heads * head_dim * bytes_per_elem


def kv_elements_per_token(num_layers: int, num_kv_heads: int, head_dim: int) -> int:
    """Cached elements per token over all layers, K and V ([Interview] §三)."""
    return num_layers * 2 * num_kv_heads * head_dim


def average_bits(seq_len: int, residual: int, main_bits: float,
                 residual_bits: float = 16.0) -> float:
    """Average stored bits per element with an FP16 window ([Tutorial] §十.3):
    (S−R)·b + R·16 over S, metadata not counted."""
    return ((seq_len - residual) * main_bits + residual * residual_bits) / seq_len


def metadata_overhead(group: int, bits: int, scale_bytes: float,
                      zero_bytes: float) -> float:
    """Per-group metadata over per-group code bytes ([Tutorial] §十.4)."""
    return (scale_bytes + zero_bytes) / (group * bits / 8.0)


def decode_bytes_kivi(batch: int, num_kv_heads: int, head_dim: int, bits: int,
                      group: int, n_quant: int, n_resid: int, v_bits: int | None = None,
                      v_group_channels: int | None = None) -> int:
    """Bytes one KIVI decode step reads: per (b, h), K codes n_quant·D·b/8,
    K scale+zero (n_quant/G)·D·8, V codes n_quant·D·b_V/8 (b_V = b unless
    given), V scale+zero n_quant·8 (times D/Gc with channel sub-groups of Gc),
    fp16 window 2·n_resid·D·2."""
    assert n_quant % group == 0
    v_bits = bits if v_bits is None else v_bits
    n_vs = 1 if v_group_channels is None else head_dim // v_group_channels
    per_pair = (n_quant * head_dim * bits // 8            # K codes
                + (n_quant // group) * head_dim * 8       # K scale, zero
                + n_quant * head_dim * v_bits // 8        # V codes
                + n_quant * 8 * n_vs                      # V scale, zero
                + 2 * n_resid * head_dim * 2)             # K, V window
    return batch * num_kv_heads * per_pair


def decode_bytes_fp8(batch: int, num_kv_heads: int, head_dim: int,
                     n_tokens: int, per_head: bool = False) -> int:
    """FP8: one byte per K and V element plus the fp32 K and V scales (one
    pair per tensor, or per KV head)."""
    return (2 * batch * num_kv_heads * n_tokens * head_dim
            + 8 * (num_kv_heads if per_head else 1))


def decode_bytes_fp16(batch: int, num_kv_heads: int, head_dim: int,
                      n_tokens: int) -> int:
    return 2 * batch * num_kv_heads * n_tokens * head_dim * 2
