"""Single-query decode attention in fp64 (oracle side).

Definition ([Tutorial] §二: Attention(Q, K, V) = softmax(QKᵀ/√d)·V; §二.1: a
decode step's query attends to every cached token, including the one just
appended; §八.1–八.2 write the same per token: score_i = q·k_i/√d,
p_i = exp(score_i)/Σ_j exp(score_j), o = Σ_i p_i v_i).

GQA ([Tutorial] §五.3: with 32 query heads and 8 KV heads every 4 query heads
share one K/V). Which query heads share is not stated; the reading used is
that consecutive query heads share: hq reads KV head hq // (Hq / H).

Everything is promoted to fp64; the softmax subtracts the row maximum before
exponentiating (an exact rewrite of the same formula).
"""
from __future__ import annotations

import numpy as np


def kv_head_of(hq: int, num_q_heads: int, num_kv_heads: int) -> int:
    return hq // (num_q_heads // num_kv_heads)


def attend_one(q: np.ndarray, k: np.ndarray, v: np.ndarray) -> np.ndarray:
    """q [D], k [T, D], v [T, D] → o [D], all in fp64."""
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    scores = (k @ q) / np.sqrt(np.float64(q.shape[0]))
    e = np.exp(scores - scores.max())
    p = e / e.sum()
    return p @ v


def decode_attention(q: np.ndarray, k: np.ndarray, v: np.ndarray) -> np.ndarray:
    """q [B, Hq, D]; k, v [B, H, T, D] (any float dtype) → out [B, Hq, D] fp64."""
    B, Hq, D = q.shape
    H = k.shape[1]
    assert Hq % H == 0 and k.shape[0] == B and k.shape[3] == D
    out = np.empty((B, Hq, D), np.float64)
    for b in range(B):
        for hq in range(Hq):
            h = kv_head_of(hq, Hq, H)
            out[b, hq] = attend_one(q[b, hq], k[b, h], v[b, h])
    return out
