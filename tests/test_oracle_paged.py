"""Pins of the paged-cache oracle (oracle.cache.PagedKiviCache).

Reading ("大模型量化从0到1（十三）：KV Cache 量化", §十三.1: paged attention maps a
sequence's logical token blocks onto discrete physical blocks, and KV
quantization composes with it): the grouped region of a ragged KIVI batch is
stored in pages of P tokens of every KV head, logical page j of sequence b
in physical page table[b][j]; what is quantized, flushed and attended is
exactly the ragged cache's. Pinned by:
  * one page per sequence with the identity table: the pool is the ragged
    cache's contiguous buffers (pinned on their own) byte for byte;
  * any table: each logical page's tokens sit in the right physical page at
    the right slots (read back from a cache of that sequence alone), and
    pages no sequence uses stay zero;
  * attention read back from the pool through the table equals the ragged
    cache's attention (pages shuffled, ragged lengths, flushes crossing page
    boundaries, G = 32 and 64, R = 0 and 128, 2- and 4-bit).
"""
import numpy as np
import pytest

import synth
from oracle import cache as ocache

pytestmark = pytest.mark.filterwarnings("ignore::RuntimeWarning")

POOL = ("k_codes", "v_codes", "k_scale", "k_zero", "v_scale", "v_zero")


def _kv(B, H, S):
    return (synth.make_k(B, H, 0, S, 128).numpy(), synth.make_v(B, H, 0, S, 128).numpy())


def test_one_page_per_sequence_is_the_contiguous_layout():
    B, H, C = 3, 2, 256
    lens = [256, 77, 190]
    k, v = _kv(B, H, 256)
    rag = ocache.RaggedKiviCache(B, H, 128, 2, 32, 128, C)
    pag = ocache.PagedKiviCache(B, H, 128, 2, 32, 128, C, page_tokens=256, num_pages=B,
                                table=[[b] for b in range(B)])
    rag.prefill(k, v, lens)
    pag.prefill(k, v, lens)
    for name in POOL:
        assert np.array_equal(pag.__dict__[name], rag.array(name)), name
    assert np.array_equal(pag.window("k_resid"), rag.array("k_resid"))


def test_pages_hold_their_logical_tokens():
    B, H, C, P = 2, 2, 512, 64
    lens = [500, 200]
    k, v = _kv(B, H, 512)
    NP = 20
    # sequence 0 in pages 19, 3, 7, ... ; sequence 1 in pages 0, 1, 2, 4
    table = [[19, 3, 7, 11, 13, 5, 9, 15], [0, 1, 2, 4, 6, 8, 10, 12]]
    pag = ocache.PagedKiviCache(B, H, 128, 2, 32, 128, C, page_tokens=P, num_pages=NP,
                                table=table)
    pag.prefill(k, v, lens)
    for b in range(B):
        alone = ocache.KiviCache(1, H, 128, 2, 32, 128, C)
        alone.prefill(k[b:b + 1, :, :lens[b]], v[b:b + 1, :, :lens[b]])
        nq = alone.n_quant
        assert pag.seq_n_quant[b] == nq
        for j in range(-(-nq // P)):
            p, t0, n = table[b][j], j * P, min(P, nq - j * P)
            assert np.array_equal(pag.k_codes[p, :, :n], alone.k_codes[0, :, t0:t0 + n])
            assert np.array_equal(pag.v_codes[p, :, :n // 32],
                                  alone.v_codes[0, :, t0 // 32:(t0 + n) // 32])
            assert np.array_equal(pag.k_scale[p, :, :n // 32], alone.k_scale[0, :, t0 // 32:(t0 + n) // 32])
            assert np.array_equal(pag.v_zero[p, :, :n], alone.v_zero[0, :, t0:t0 + n])
    used = {table[b][j] for b in range(B) for j in range(-(-pag.seq_n_quant[b] // P))}
    for p in set(range(NP)) - used:
        for name in POOL:
            assert not pag.__dict__[name][p].any(), (name, p)


@pytest.mark.parametrize("bits,G,R,P", [(2, 32, 128, 64), (4, 64, 128, 128), (2, 32, 0, 32),
                                        (2, 64, 64, 256)])
def test_attention_through_the_table_equals_ragged(bits, G, R, P):
    B, H, Hq, C = 3, 2, 8, 640
    lens = [600, 130, 257]
    steps = 40
    k, v = _kv(B, H, C)
    rng = np.random.default_rng(7)
    max_pages = -(-C // P)
    NP = B * max_pages + 3
    perm = rng.permutation(NP)[:B * max_pages].reshape(B, max_pages)
    rag = ocache.RaggedKiviCache(B, H, 128, bits, G, R, C)
    pag = ocache.PagedKiviCache(B, H, 128, bits, G, R, C, page_tokens=P, num_pages=NP,
                                table=perm)
    kp = np.zeros_like(k[:, :, :max(lens)])
    vp = np.zeros_like(kp)
    for b, S in enumerate(lens):
        kp[b, :, :S], vp[b, :, :S] = k[b, :, :S], v[b, :, :S]
    rag.prefill(kp, vp, lens)
    pag.prefill(kp, vp, lens)
    for t in range(steps):
        k1 = np.stack([k[b, :, lens[b] + t] for b in range(B)])
        v1 = np.stack([v[b, :, lens[b] + t] for b in range(B)])
        rag.append(k1, v1)
        pag.append(k1, v1)
        if t % 13 == 0 or t == steps - 1:
            q = synth.make_q(B, Hq, 128, step=t).numpy()
            assert np.array_equal(pag.attention(q), rag.attention(q))
    assert pag.seq_n_quant == rag.seq_n_quant and pag.seq_n_resid == rag.seq_n_resid
