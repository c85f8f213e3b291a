"""Seeded synthetic K/V/query generators shared by the oracle and the HIP path.

This module holds none of the quantization or attention arithmetic: it only
draws the inputs. Both sides consume the same generated tensors.

Random numbers come from Threefry-2x32 with 20 rounds (Salmon, Moraes, Dror,
Shaw, "Parallel random numbers: as easy as 1, 2, 3", SC'11), a counter-based
generator made of 32-bit add / rotate / xor only. It is evaluated here with
int64 torch tensors holding 32-bit values, so it is exact on CPU and GPU and
any chunking of the index space reproduces the same values (token S+i of a
streamed decode is exactly element S+i of the prefill stream).

Distributions (the workload description of the benchmark configurations):
  K[b,h,t,d] = N(0,1) · f[h,d],  f = LogNormal(0,1) per (KV head, channel),
               with two distinct outlier channels per KV head scaled ×10
  V[b,h,t,d] = N(0,1) · g[b,h,t], g = LogNormal(0,0.5) per token
  q[b,hq,d]  = N(0,1) (fp32)
K and V are formed in fp64, rounded to fp32 and then to fp16 (each RNE).
Normals use Box–Muller (cosine branch) on two 32-bit uniforms.

Streams (second key word): 0 K normals, 1 V normals, 2 query normals,
3 K channel log-factors, 4 outlier channel picks, 5 V token log-factors.
"""
from __future__ import annotations

import math

import torch

MASK32 = 0xFFFFFFFF
# Threefry-2x32 rotation constants and key-schedule parity constant.
_ROT = (13, 15, 26, 6, 17, 29, 16, 24)
_PARITY = 0x1BD11BDA

STREAM_K, STREAM_V, STREAM_Q, STREAM_KF, STREAM_OUTLIER, STREAM_VF = range(6)

# Token index bits reserved in the counter, so that element (b, h, t, d) has
# the same counter whatever the total sequence length is.
_TOKEN_BITS = 24


def _rotl(x: torch.Tensor, r: int) -> torch.Tensor:
    return ((x << r) | (x >> (32 - r))) & MASK32


def threefry2x32(k0: int, k1: int, c0: torch.Tensor, c1: torch.Tensor):
    """Threefry-2x32-20 block function; key (k0, k1), counters (c0, c1).

    Counters are int64 tensors holding values in [0, 2^32). Returns two int64
    tensors of 32-bit outputs.
    """
    k0 &= MASK32
    k1 &= MASK32
    ks = (k0, k1, (_PARITY ^ k0 ^ k1) & MASK32)
    x0 = (c0 + ks[0]) & MASK32
    x1 = (c1 + ks[1]) & MASK32
    for r in range(20):
        x0 = (x0 + x1) & MASK32
        x1 = _rotl(x1, _ROT[r % 8]) ^ x0
        if r % 4 == 3:
            j = (r + 1) // 4
            x0 = (x0 + ks[j % 3]) & MASK32
            x1 = (x1 + ks[(j + 1) % 3] + j) & MASK32
    return x0, x1


def normal(seed: int, stream: int, index: torch.Tensor) -> torch.Tensor:
    """Standard normals (fp64), one per int64 counter index (< 2^64)."""
    c0 = index & MASK32
    c1 = (index >> 32) & MASK32
    x0, x1 = threefry2x32(seed, stream, c0, c1)
    u1 = (x0.to(torch.float64) + 1.0) * (1.0 / 4294967296.0)   # (0, 1]
    u2 = x1.to(torch.float64) * (1.0 / 4294967296.0)           # [0, 1)
    return torch.sqrt(-2.0 * torch.log(u1)) * torch.cos((2.0 * math.pi) * u2)


def uint32(seed: int, stream: int, index: torch.Tensor) -> torch.Tensor:
    """Raw 32-bit words (first Threefry output), as int64."""
    x0, _ = threefry2x32(seed, stream, index & MASK32, (index >> 32) & MASK32)
    return x0


def _to_fp16(x64: torch.Tensor) -> torch.Tensor:
    return x64.to(torch.float32).to(torch.float16)


def outlier_channels(num_kv_heads: int, head_dim: int, seed: int = 0):
    """Two distinct outlier channels per KV head: list of (c0, c1)."""
    idx = torch.arange(2 * num_kv_heads, dtype=torch.int64)
    w = uint32(seed, STREAM_OUTLIER, idx).tolist()
    out = []
    for h in range(num_kv_heads):
        c0 = w[2 * h] % head_dim
        c1 = (c0 + 1 + w[2 * h + 1] % (head_dim - 1)) % head_dim
        out.append((c0, c1))
    return out


def k_channel_factors(num_kv_heads: int, head_dim: int, seed: int = 0,
                      device="cpu") -> torch.Tensor:
    """f[h, d] (fp64): LogNormal(0,1), ×10 on the two outlier channels."""
    idx = torch.arange(num_kv_heads * head_dim, dtype=torch.int64, device=device)
    f = torch.exp(normal(seed, STREAM_KF, idx)).view(num_kv_heads, head_dim)
    for h, (c0, c1) in enumerate(outlier_channels(num_kv_heads, head_dim, seed)):
        f[h, c0] *= 10.0
        f[h, c1] *= 10.0
    return f


def _token_index(b: int, H: int, t0: int, t1: int, device, heads=None):
    """Counter base of tokens [t0, t1) of the KV heads `heads` (default: all
    H) of batch element b: int64 [len(heads), t1 - t0]."""
    if heads is None:
        h = torch.arange(H, dtype=torch.int64, device=device)
    else:
        h = torch.tensor(list(heads), dtype=torch.int64, device=device)
    t = torch.arange(t0, t1, dtype=torch.int64, device=device)
    return ((b * H + h[:, None]) << _TOKEN_BITS) + t[None, :]


def make_k(batch: int, num_kv_heads: int, t0: int, t1: int, head_dim: int,
           seed: int = 0, device="cpu", b0: int = 0, heads=None) -> torch.Tensor:
    """fp16 K for tokens [t0, t1) of batch elements [b0, b0 + B):
    shape [B, H, t1 - t0, D]; with `heads` (KV head indices), only those
    heads: [B, len(heads), t1 - t0, D], each equal to its slice of the full
    tensor."""
    assert 0 <= t0 <= t1 < (1 << _TOKEN_BITS)
    f = k_channel_factors(num_kv_heads, head_dim, seed, device)
    hs = list(range(num_kv_heads)) if heads is None else list(heads)
    out = torch.empty(batch, len(hs), t1 - t0, head_dim,
                      dtype=torch.float16, device=device)
    d = torch.arange(head_dim, dtype=torch.int64, device=device)
    for b in range(batch):
        tok = _token_index(b0 + b, num_kv_heads, t0, t1, device, hs)
        idx = tok[:, :, None] * head_dim + d
        out[b] = _to_fp16(normal(seed, STREAM_K, idx) * f[hs][:, None, :])
    return out


def make_v(batch: int, num_kv_heads: int, t0: int, t1: int, head_dim: int,
           seed: int = 0, device="cpu", b0: int = 0, heads=None) -> torch.Tensor:
    """fp16 V for tokens [t0, t1) of batch elements [b0, b0 + B):
    shape [B, H, t1 - t0, D] (only the KV heads `heads` when given)."""
    assert 0 <= t0 <= t1 < (1 << _TOKEN_BITS)
    hs = list(range(num_kv_heads)) if heads is None else list(heads)
    out = torch.empty(batch, len(hs), t1 - t0, head_dim,
                      dtype=torch.float16, device=device)
    d = torch.arange(head_dim, dtype=torch.int64, device=device)
    for b in range(batch):
        tok = _token_index(b0 + b, num_kv_heads, t0, t1, device, hs)
        g = torch.exp(0.5 * normal(seed, STREAM_VF, tok))
        idx = tok[:, :, None] * head_dim + d
        out[b] = _to_fp16(normal(seed, STREAM_V, idx) * g[:, :, None])
    return out


def make_q(batch: int, num_q_heads: int, head_dim: int, seed: int = 0,
           step: int = 0, device="cpu") -> torch.Tensor:
    """fp32 queries [B, Hq, D]; `step` selects an independent query per step."""
    n = batch * num_q_heads * head_dim
    idx = torch.arange(n, dtype=torch.int64, device=device) + step * n
    return normal(seed, STREAM_Q, idx).to(torch.float32).view(
        batch, num_q_heads, head_dim)


# The benchmark configurations, by workload name: shape, format and steps.
CONFIGS = {
    "tiny_mha": dict(batch=1, num_q_heads=1, num_kv_heads=1, head_dim=128,
                     seq_len=256, formats=("kivi",), bits=2, group_size=32,
                     residual_length=128, decode_steps=0),
    "llama2_7b_layer": dict(batch=8, num_q_heads=32, num_kv_heads=32,
                            head_dim=128, seq_len=4096, formats=("kivi",),
                            bits=2, group_size=32, residual_length=128,
                            decode_steps=0),
    "gqa70b_32k": dict(batch=16, num_q_heads=64, num_kv_heads=8, head_dim=128,
                       seq_len=32768, formats=("kivi",), bits=2,
                       group_size=32, residual_length=128, decode_steps=256),
    "mha_large_batch_4bit": dict(batch=64, num_q_heads=32, num_kv_heads=32,
                                 head_dim=128, seq_len=8192,
                                 formats=("kivi",), bits=4, group_size=32,
                                 residual_length=128, decode_steps=0),
    "gqa_128k": dict(batch=4, num_q_heads=32, num_kv_heads=8, head_dim=128,
                     seq_len=131072, formats=("fp8", "kivi", "fp16"), bits=2,
                     group_size=32, residual_length=128, decode_steps=0),
}
