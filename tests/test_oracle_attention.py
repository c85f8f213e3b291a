"""Pins of the oracle's fp64 decode attention."""
import math

import numpy as np
import torch

from oracle import attention

RNG = np.random.default_rng(99)


def test_matches_torch_sdpa_fp64():
    B, Hq, H, T, D = 2, 8, 2, 37, 128
    q = RNG.normal(0, 1, (B, Hq, D))
    k = RNG.normal(0, 2, (B, H, T, D))
    v = RNG.normal(0, 1, (B, H, T, D))
    got = attention.decode_attention(q, k, v)
    rep = Hq // H
    kr = torch.from_numpy(np.repeat(k, rep, axis=1))
    vr = torch.from_numpy(np.repeat(v, rep, axis=1))
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q)[:, :, None, :], kr, vr).numpy()[:, :, 0, :]
    assert np.max(np.abs(got - ref)) < 1e-12


def test_brute_force_small():
    """Pure-Python softmax on S ≤ 8 tokens."""
    D = 128
    for T in range(1, 9):
        q = RNG.normal(0, 1, D)
        k = RNG.normal(0, 3, (T, D))
        v = RNG.normal(0, 1, (T, D))
        scores = [sum(q[d] * k[t, d] for d in range(D)) / math.sqrt(D) for t in range(T)]
        w = [math.exp(s) for s in scores]
        tot = sum(w)
        ref = [sum(w[t] * v[t, d] for t in range(T)) / tot for d in range(D)]
        got = attention.attend_one(q, k, v)
        assert np.max(np.abs(got - np.array(ref))) < 1e-12


def test_single_token_returns_its_value():
    q = RNG.normal(0, 1, (1, 3, 128))
    k = RNG.normal(0, 1, (1, 1, 1, 128))
    v = RNG.normal(0, 1, (1, 1, 1, 128))
    out = attention.decode_attention(q, k, v)
    assert np.array_equal(out, np.broadcast_to(v[0, 0, 0], (1, 3, 128)))


def test_identical_keys_give_mean_of_values():
    k = np.tile(RNG.normal(0, 1, 128), (50, 1))[None, None]
    v = RNG.normal(0, 1, (1, 1, 50, 128))
    q = RNG.normal(0, 5, (1, 1, 128))
    out = attention.decode_attention(q, k, v)
    assert np.max(np.abs(out[0, 0] - v[0, 0].mean(axis=0))) < 1e-12


def test_gqa_equals_mha_with_repeated_heads():
    B, Hq, H, T, D = 1, 8, 2, 20, 128
    q = RNG.normal(0, 1, (B, Hq, D))
    k = RNG.normal(0, 1, (B, H, T, D))
    v = RNG.normal(0, 1, (B, H, T, D))
    gqa = attention.decode_attention(q, k, v)
    mha = attention.decode_attention(q, np.repeat(k, 4, axis=1), np.repeat(v, 4, axis=1))
    assert np.array_equal(gqa, mha)
    # consecutive query heads share: heads 0..3 → KV 0, heads 4..7 → KV 1
    assert [attention.kv_head_of(h, 8, 2) for h in range(8)] == [0] * 4 + [1] * 4


def test_large_scores_stable():
    q = np.full((1, 1, 128), 50.0)
    k = RNG.normal(0, 30, (1, 1, 64, 128))
    v = RNG.normal(0, 1, (1, 1, 64, 128))
    out = attention.decode_attention(q, k, v)
    assert np.all(np.isfinite(out))
    top = np.argmax(k[0, 0] @ q[0, 0])
    assert np.max(np.abs(out[0, 0] - v[0, 0, top])) < 1e-6
