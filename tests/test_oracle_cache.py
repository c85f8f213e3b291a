"""Pins of the oracle's cache state machines (prefill split, lazy flush,
residual semantics, group locality, FP8 frozen scale)."""
import numpy as np
import pytest
import torch

import synth
from oracle import attention, cache, fp8, kivi

D = 128


def _kv(B, H, T, seed=0):
    k = synth.make_k(B, H, 0, T, D, seed).numpy()
    v = synth.make_v(B, H, 0, T, D, seed).numpy()
    return k, v


def test_tiny_mha_split():
    """S = 256, G = 32, R = 128 → 4 quantized groups + 128 FP16 tokens (the
    tiny MHA workload's statement)."""
    k, v = _kv(1, 1, 256)
    c = cache.KiviCache(1, 1, D, 2, 32, 128, 256)
    c.prefill(k, v)
    assert (c.n_quant, c.n_resid) == (128, 128)
    assert np.array_equal(c.k_resid[0, 0], k[0, 0, 128:])


def test_all_residual_equals_fp16_attention():
    """R ≥ S: nothing is quantized, so KIVI attention is FP16 attention."""
    k, v = _kv(2, 2, 100)
    q = synth.make_q(2, 4, D).numpy()
    ck = cache.KiviCache(2, 2, D, 2, 32, 128, 300)
    ck.prefill(k, v)
    cf = cache.Fp16Cache(2, 2, D, 300)
    cf.prefill(k, v)
    assert ck.n_quant == 0
    assert np.array_equal(ck.attention(q), cf.attention(q))


def test_r0_no_window_when_aligned():
    k, v = _kv(1, 1, 96)
    c = cache.KiviCache(1, 1, D, 2, 32, 0, 200)
    c.prefill(k, v)
    assert (c.n_quant, c.n_resid) == (96, 0)
    # the window of an R = 0 cache holds the incomplete group and flushes at G
    k2 = synth.make_k(1, 1, 96, 96 + 33, D).numpy()
    v2 = synth.make_v(1, 1, 96, 96 + 33, D).numpy()
    for i in range(33):
        c.append(k2[:, :, i], v2[:, :, i])
    assert (c.n_quant, c.n_resid) == (128, 1) and c.flush_steps == [33]


def test_residual_changes_the_result():
    """R = 128 keeps the newest tokens exact, R = 0 quantizes them: the two
    caches differ exactly in those tokens."""
    k, v = _kv(1, 1, 256)
    c128 = cache.KiviCache(1, 1, D, 2, 32, 128, 256)
    c0 = cache.KiviCache(1, 1, D, 2, 32, 0, 256)
    c128.prefill(k, v)
    c0.prefill(k, v)
    K128, _ = c128.dequantized()
    K0, _ = c0.dequantized()
    assert np.array_equal(K128[..., :128, :], K0[..., :128, :])
    assert np.array_equal(K128[..., 128:, :], k[..., 128:, :].astype(np.float32))
    assert not np.array_equal(K0[..., 128:, :], k[..., 128:, :].astype(np.float32))


def test_streaming_flush_schedule_32k():
    """Prefill 32768 then 256 appends (G = 32, R = 128): flushes at appends 1
    and 129, final state (32896, 128)."""
    S, steps = 32768, 256
    k = synth.make_k(1, 1, 0, S + steps, D).numpy()
    v = synth.make_v(1, 1, 0, S + steps, D).numpy()
    c = cache.KiviCache(1, 1, D, 2, 32, 128, S + steps)
    c.prefill(k[:, :, :S], v[:, :, :S])
    assert (c.n_quant, c.n_resid) == (32640, 128)
    for i in range(steps):
        c.append(k[:, :, S + i], v[:, :, S + i])
    assert c.flush_steps == [1, 129]
    assert (c.n_quant, c.n_resid) == (32896, 128)
    # group locality: a fresh prefill of the same tokens has identical groups
    c2 = cache.KiviCache(1, 1, D, 2, 32, 128, S + steps)
    c2.prefill(k, v)
    assert c2.n_quant == 32896
    n = c.n_quant
    assert np.array_equal(c.k_codes[..., :n, :], c2.k_codes[..., :n, :])
    assert np.array_equal(c.k_scale, c2.k_scale) and np.array_equal(c.k_zero, c2.k_zero)
    assert np.array_equal(c.v_codes, c2.v_codes)
    assert np.array_equal(c.v_scale, c2.v_scale) and np.array_equal(c.v_zero, c2.v_zero)
    assert np.array_equal(c.k_resid, c2.k_resid) and np.array_equal(c.v_resid, c2.v_resid)


@pytest.mark.parametrize("bits,G,R,Gc", [(2, 32, 64, None), (4, 32, 64, None),
                                          (2, 64, 64, None), (4, 128, 128, None),
                                          (2, 64, 256, None), (2, 32, 128, 32),
                                          (4, 64, 64, 32)])
def test_group_locality_ragged(bits, G, R, Gc):
    k, v = _kv(2, 3, 600)
    a = cache.KiviCache(2, 3, D, bits, G, R, 600, v_group_channels=Gc)
    a.prefill(k[:, :, :100], v[:, :, :100])
    for t in range(100, 600):
        a.append(k[:, :, t], v[:, :, t])
    b = cache.KiviCache(2, 3, D, bits, G, R, 600, v_group_channels=Gc)
    b.prefill(k, v)
    n = min(a.n_quant, b.n_quant)
    assert n >= 600 - 2 * R - G and n % G == 0
    assert np.array_equal(a.k_codes[:, :, :n], b.k_codes[:, :, :n])
    assert np.array_equal(a.v_scale[:, :, :n], b.v_scale[:, :, :n])
    assert np.array_equal(a.v_codes[:, :, :n // 32], b.v_codes[:, :, :n // 32])
    assert np.array_equal(a.k_scale[:, :, :n // G], b.k_scale[:, :, :n // G])


@pytest.mark.parametrize("G", [64, 128])
def test_k_scale_spans_the_whole_group(G):
    """With G = 64 or 128 one K scale and zero-point per channel cover all G
    tokens of a group (checked against plain per-slice minima and maxima of
    the input), while V stays per token and its codes stay in 32-token tiles:
    a group whose halves have very different ranges gets one shared scale."""
    k, v = _kv(1, 1, 4 * G)
    k = k.copy()
    k[0, 0, G // 2:G] *= 8          # second half of group 0 spans a wider range
    c = cache.KiviCache(1, 1, D, 2, G, 0, 4 * G)
    c.prefill(k, v)
    assert c.n_quant == 4 * G and c.k_scale.shape == (1, 1, 4, D)
    assert c.v_codes.shape == (1, 1, 4 * G // 32, D, 2)
    x = k[0, 0].astype(np.float32)
    for g in range(4):
        mn = x[g * G:(g + 1) * G].min(axis=0)
        mx = x[g * G:(g + 1) * G].max(axis=0)
        assert np.array_equal(c.k_zero[0, 0, g], mn)
        assert np.array_equal(c.k_scale[0, 0, g], (mx - mn) / np.float32(3))
    # V: per-token range, whatever G is
    xv = v[0, 0].astype(np.float32)
    assert np.array_equal(c.v_zero[0, 0, :4 * G], xv.min(axis=1))
    Kh, Vh = c.dequantized()
    # every K value within half a step of its group's scale (+ fp32 slack)
    err = np.abs(Kh[0, 0] - x)
    for g in range(4):
        s = c.k_scale[0, 0, g]
        assert np.all(err[g * G:(g + 1) * G] <= s / 2 + 1e-6 * np.abs(x[g * G:(g + 1) * G]) + 1e-7)


def test_dequantized_matches_unpacked_codes():
    """The cache's packed state decodes to the same values as quantizing the
    tokens directly."""
    k, v = _kv(1, 2, 256)
    c = cache.KiviCache(1, 2, D, 2, 32, 128, 256)
    c.prefill(k, v)
    Kh, Vh = c.dequantized()
    for h in range(2):
        kc, ks, kz = kivi.quantize_k(k[0, h, :128], 2, 32)
        vc, vs, vz = kivi.quantize_v(v[0, h, :128], 2)
        assert np.array_equal(Kh[0, h, :128], kivi.dequantize_k(kc, ks, kz, 32))
        assert np.array_equal(Vh[0, h, :128], kivi.dequantize_v(vc, vs, vz))


def test_fp8_fp16_tile_layout():
    """V of the FP8 / FP16 caches sits in 32-token tiles, one row per channel:
    element (t, d) at [t // 32][d][t % 32]; tile_rows / untile_rows invert
    each other and unfilled slots are zero."""
    x = np.arange(70 * D, dtype=np.float32).reshape(70, D)
    y = cache.tile_rows(x, 3)
    assert y.shape == (3, D, 32)
    assert y[1, 5, 7] == x[39, 5] and y[2, 127, 5] == x[69, 127]
    assert np.all(y[2, :, 6:] == 0)
    assert np.array_equal(cache.untile_rows(y, 70), x)
    k, v = _kv(1, 2, 45)
    c = cache.Fp16Cache(1, 2, D, 70)
    c.prefill(k, v)
    k1 = synth.make_k(1, 2, 45, 46, D).numpy()[:, :, 0]
    v1 = synth.make_v(1, 2, 45, 46, D).numpy()[:, :, 0]
    c.append(k1, v1)
    assert c.v.shape == (1, 2, 3, D, 32) and c.k.shape == (1, 2, 96, D)
    assert np.array_equal(c.v[0, 1, 1, :, 13], v1[0, 1])          # token 45
    assert np.array_equal(c.v[0, 0, 0, :, 3], v[0, 0, 3])
    Kh, Vh = c.dequantized()
    assert np.array_equal(Vh[0, 0, :45], v[0, 0].astype(np.float32))


def test_fp8_scale_frozen_after_prefill():
    k, v = _kv(1, 2, 64)
    c = cache.Fp8Cache(1, 2, D, 80)
    c.prefill(k, v)
    sk = c.tensor_scale[0]
    assert sk == fp8.tensor_scale(k)
    big = np.full((1, 2, D), 60000.0, np.float16)
    c.append(big, big)
    assert c.tensor_scale[0] == sk
    assert np.all(c.k_codes[:, :, 64] == 0x7E)            # saturated to +448


def test_synth_distributions():
    """The generator draws the stated shapes: K channel factors with 2 ×10
    outlier channels per KV head, V per-token factors."""
    f = synth.k_channel_factors(4, D).numpy()
    out = synth.outlier_channels(4, D)
    for h, (a, b) in enumerate(out):
        assert a != b
        ratio = f[h] / np.exp(synth.normal(0, synth.STREAM_KF,
                                           torch.arange(h * D, (h + 1) * D)).numpy())
        assert np.allclose(ratio[[a, b]], 10.0) and np.allclose(np.delete(ratio, [a, b]), 1.0)
    # streaming token t is element t of the prefill stream
    k_all = synth.make_k(2, 2, 0, 40, D)
    k_tail = synth.make_k(2, 2, 33, 40, D)
    assert torch.equal(k_all[:, :, 33:], k_tail)
    n = synth.normal(0, 0, torch.arange(200_000)).numpy()
    assert abs(n.mean()) < 0.01 and abs(n.std() - 1) < 0.01


@pytest.mark.parametrize("kb,vb", [(4, 2), (2, 4)])
def test_mixed_bit_widths(kb, vb):
    """K and V with their own bit widths: K codes span 2^kb − 1 levels with
    one per-channel scale (max − min)/(2^kb − 1) per group, V codes span
    2^vb − 1 levels per token; each reconstructs within half its own step."""
    k, v = _kv(1, 2, 192)
    c = cache.KiviCache(1, 2, D, kb, 32, 0, 192, v_bits=vb)
    c.prefill(k, v)
    assert c.k_codes.shape[-1] == D * kb // 32 and c.v_codes.shape[-1] == 32 * vb // 32
    Kh, Vh = c.dequantized()
    for h in range(2):
        x = k[0, h].astype(np.float32)
        y = v[0, h].astype(np.float32)
        for g in range(6):
            sl = slice(32 * g, 32 * g + 32)
            s_k = (x[sl].max(axis=0) - x[sl].min(axis=0)) / np.float32(2 ** kb - 1)
            assert np.array_equal(c.k_scale[0, h, g], s_k)
            assert np.all(np.abs(Kh[0, h, sl] - x[sl]) <= s_k / 2 + 1e-6 * np.abs(x[sl]) + 1e-7)
        s_v = (y.max(axis=1) - y.min(axis=1)) / np.float32(2 ** vb - 1)
        assert np.array_equal(c.v_scale[0, h, :192], s_v)
        assert np.all(np.abs(Vh[0, h] - y) <= s_v[:, None] / 2 + 1e-6 * np.abs(y) + 1e-7)


@pytest.mark.parametrize("fmt", ["e4m3", "e5m2"])
def test_fp8_per_head_is_per_tensor_on_each_head(fmt):
    """Per-KV-head scales ([Tutorial] §十八.6) reduce to the per-tensor cache
    run on each head's slice alone: same scales, same codes, after prefill and
    after appends (scales frozen at prefill)."""
    B, H, S, C = 2, 3, 70, 75
    k, v = _kv(B, H, C)
    k = k.copy()
    k[:, 1] *= 20                                        # one wide head
    c = cache.Fp8Cache(B, H, D, C, fmt=fmt, per_head=True)
    c.prefill(k[:, :, :S], v[:, :, :S])
    for t in range(S, C):
        c.append(k[:, :, t], v[:, :, t])
    for h in range(H):
        r = cache.Fp8Cache(B, 1, D, C, fmt=fmt)
        r.prefill(k[:, h:h + 1, :S], v[:, h:h + 1, :S])
        for t in range(S, C):
            r.append(k[:, h:h + 1, t], v[:, h:h + 1, t])
        assert np.array_equal(c.tensor_scale[h], r.tensor_scale)
        assert np.array_equal(c.k_codes[:, h], r.k_codes[:, 0])
        assert np.array_equal(c.v_codes[:, h], r.v_codes[:, 0])
    assert c.tensor_scale[1, 0] > 10 * c.tensor_scale[0, 0]


def test_fp8_query_attention_reduces_to_exact_on_grid_queries():
    """Attention in the FP8 domain: a query whose rows are E4M3 values at a
    power-of-two scale (amax exactly 448 · 2^-3) is unchanged by the query
    quantization, so the result equals the plain FP8-cache attention; a
    general query moves the output by a small amount only."""
    B, H, Hq, S = 1, 2, 4, 96
    k, v = _kv(B, H, S)
    c = cache.Fp8Cache(B, H, D, S)
    c.prefill(k, v)
    grid = fp8.decode_table()[:0x7F]
    rng = np.random.default_rng(4)
    q = grid[rng.integers(0, 0x7F, (B, Hq, D))].astype(np.float32)
    q[..., 0] = 448.0
    q *= np.float32(2.0 ** -3)
    assert np.array_equal(c.attention(q, fp8_query=True), c.attention(q))
    qn = rng.normal(0, 1, (B, Hq, D)).astype(np.float32)
    d = np.abs(c.attention(qn, fp8_query=True) - c.attention(qn)).max()
    assert 0 < d < 0.5


def test_v_subgroup_cache_layout_and_reduction():
    """V channel sub-groups in the cache: v_scale / v_zero gain a trailing
    D/32 axis; with Gc = D the cache equals the per-token cache."""
    k, v = _kv(1, 2, 200)
    c = cache.KiviCache(1, 2, D, 2, 32, 64, 200, v_group_channels=32)
    c.prefill(k, v)
    assert c.v_scale.shape == (1, 2, 224, 4) and c.n_quant == 160
    w = cache.KiviCache(1, 2, D, 2, 32, 64, 200, v_group_channels=D)
    w.prefill(k, v)
    p = cache.KiviCache(1, 2, D, 2, 32, 64, 200)
    p.prefill(k, v)
    assert np.array_equal(w.v_codes, p.v_codes) and np.array_equal(w.v_scale[..., 0], p.v_scale)
    Kh, Vh = c.dequantized()
    Kp, Vp = p.dequantized()
    assert np.array_equal(Kh, Kp)
    x = v[:, :, :160].astype(np.float32)
    assert np.abs(Vh[:, :, :160] - x).max() <= np.abs(Vp[:, :, :160] - x).max()


@pytest.mark.parametrize("G,R,T,state", [
    (32, 128, 256, (128, 128)),   # flush at append 129
    (32, 64, 192, (128, 64)),     # flushes at 65 and 129
    (64, 128, 384, (256, 128)),   # flushes of two 64-token groups
    (32, 0, 97, (96, 1)),         # R = 0: the window is the open group
])
def test_appends_alone_equal_the_prefill(G, R, T, state):
    """A cache that receives every token by an append into an empty cache
    ends, once its fill state is the one a prefill of the same T tokens gives,
    with the same stored arrays as that prefill: every flush quantizes whole
    groups at the positions the prefill puts them, and the window holds the
    newest tokens."""
    B, H, D = 2, 2, 128
    k = synth.make_k(B, H, 0, T, D).numpy()
    v = synth.make_v(B, H, 0, T, D).numpy()
    pre = cache.KiviCache(B, H, D, 2, G, R, T)
    pre.prefill(k, v)
    app = cache.KiviCache(B, H, D, 2, G, R, T)
    for t in range(T):
        app.append(k[:, :, t], v[:, :, t])
    assert (pre.n_quant, pre.n_resid) == (app.n_quant, app.n_resid) == state
    # a flush empties a full window: R tokens, or the open group when R = 0
    w = R or G
    assert app.flush_steps == [1 + w * (i + 1) for i in range(T // w - (T % w == 0))]
    for name in ("k_codes", "v_codes", "k_scale", "k_zero", "v_scale", "v_zero"):
        assert np.array_equal(getattr(pre, name), getattr(app, name)), name
    n = state[1]
    assert np.array_equal(pre.k_resid[:, :, :n], app.k_resid[:, :, :n])
    assert np.array_equal(pre.v_resid[:, :, :n], app.v_resid[:, :, :n])
    q = synth.make_q(B, 8, D).numpy()
    assert np.array_equal(pre.attention(q), app.attention(q))
