"""Pins of the ragged-batch oracle (oracle.cache.RaggedKiviCache).

The ragged reading: every sequence of a ragged batch is quantized, flushed
and attended as a batch of one holding only its own tokens ("4.4 KV Cache
量化：KIVI 2-bit 与 FP8 KV Cache", §3.1-3.2, stated per sequence). Pinned by:
  * equal lengths: the ragged cache equals the uniform batched cache (which is
    pinned on its own) array for array and in attention;
  * padding past a sequence's length is never read (planting huge values
    there changes nothing);
  * each sequence flushes on its own schedule (a window of w tokens flushes
    on append Rcap - w + 1);
  * attention of each sequence equals plain softmax attention over that
    sequence's dequantized tokens (brute force, fp64).
"""
import numpy as np
import pytest

from oracle import cache as ocache
from oracle import kivi as okivi
import synth

pytestmark = pytest.mark.filterwarnings("ignore::RuntimeWarning")

ARRAYS = ("k_codes", "v_codes", "k_scale", "k_zero", "v_scale", "v_zero", "k_resid", "v_resid")


def _kv(B, H, S, seed=0):
    return (synth.make_k(B, H, 0, S, 128, seed=seed).numpy(),
            synth.make_v(B, H, 0, S, 128, seed=seed).numpy())


def test_equal_lengths_equal_uniform_batch():
    B, H, S, C = 3, 2, 200, 232
    k, v = _kv(B, H, S + 6)
    rag = ocache.RaggedKiviCache(B, H, 128, 2, 32, 128, C)
    uni = ocache.KiviCache(B, H, 128, 2, 32, 128, C)
    rag.prefill(k[:, :, :S], v[:, :, :S], [S] * B)
    uni.prefill(k[:, :, :S], v[:, :, :S])
    for t in range(6):
        rag.append(k[:, :, S + t], v[:, :, S + t])
        uni.append(k[:, :, S + t], v[:, :, S + t])
    assert rag.seq_n_quant == [uni.n_quant] * B and rag.seq_n_resid == [uni.n_resid] * B
    for name in ARRAYS:
        assert np.array_equal(rag.array(name), getattr(uni, name)), name
    q = synth.make_q(B, 2 * H, 128).numpy()
    assert np.array_equal(rag.attention(q), uni.attention(q))


def test_padding_is_never_read():
    B, H, Smax, C = 3, 1, 300, 320
    lens = [300, 45, 161]
    k, v = _kv(B, H, Smax)
    kp, vp = k.copy(), v.copy()
    for b, S in enumerate(lens):
        kp[b, :, S:] = np.float16(60000.0)
        vp[b, :, S:] = np.float16(-60000.0)
    a = ocache.RaggedKiviCache(B, H, 128, 2, 32, 128, C)
    p = ocache.RaggedKiviCache(B, H, 128, 2, 32, 128, C)
    a.prefill(k, v, lens)
    p.prefill(kp, vp, lens)
    for name in ARRAYS:
        assert np.array_equal(a.array(name), p.array(name)), name
    q = synth.make_q(B, H, 128).numpy()
    assert np.array_equal(a.attention(q), p.attention(q))


def test_each_sequence_flushes_on_its_own_schedule():
    B, H, C = 3, 1, 512
    lens = [256, 228, 131]            # windows of 128, 100 and 99 tokens
    k, v = _kv(B, H, 256 + 40)
    c = ocache.RaggedKiviCache(B, H, 128, 2, 32, 128, C)
    c.prefill(k[:, :, :256], v[:, :, :256], lens)
    nq0 = c.seq_n_quant
    nr0 = c.seq_n_resid
    assert nq0 == [okivi.prefill_split(S, 32, 128)[0] for S in lens]
    for t in range(40):
        c.append(k[:, :, 256 + t], v[:, :, 256 + t])
    for b in range(B):
        expect = [128 - nr0[b] + 1] if 128 - nr0[b] + 1 <= 40 else []
        assert c.seqs[b].flush_steps == expect, (b, nr0[b], c.seqs[b].flush_steps)


def test_attention_is_softmax_over_own_tokens():
    B, H, Hq, Smax, C = 2, 1, 2, 120, 160
    lens = [120, 70]
    k, v = _kv(B, H, Smax)
    c = ocache.RaggedKiviCache(B, H, 128, 4, 32, 0, C)
    c.prefill(k, v, lens)
    q = synth.make_q(B, Hq, 128).numpy().astype(np.float64)
    out = c.attention(q.astype(np.float32))
    for b in range(B):
        Kh, Vh = c.seqs[b].dequantized()
        assert Kh.shape[2] == lens[b]
        for hq in range(Hq):
            s = Kh[0, 0].astype(np.float64) @ q[b, hq] / np.sqrt(128.0)
            p = np.exp(s - s.max())
            ref = (p / p.sum()) @ Vh[0, 0].astype(np.float64)
            assert np.allclose(out[b, hq], ref, rtol=0, atol=1e-9)
