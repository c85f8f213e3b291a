"""Pins of the oracle's KIVI quantizer: invariants, brute force, axes, packing."""
import json
import os

import numpy as np
import pytest

from oracle import kivi

F32 = np.float32
RNG = np.random.default_rng(1234)


def _fp16(a):
    return np.asarray(a, np.float32).astype(np.float16)


def _random_k(T=128, D=128, scale_spread=3.0):
    f = np.exp(RNG.normal(0, 1, D)) * scale_spread
    return _fp16(RNG.normal(0, 1, (T, D)) * f[None, :] + RNG.normal(0, 2, D)[None, :])


def _random_v(T=128, D=128):
    g = np.exp(0.5 * RNG.normal(0, 1, T))
    return _fp16(RNG.normal(0, 1, (T, D)) * g[:, None] - RNG.normal(0, 1, T)[:, None])


@pytest.mark.parametrize("bits", [2, 4])
def test_error_bound_k(bits):
    """|x̂ − x| ≤ s/2 plus fp32 rounding slack ([Tutorial] §十: round to the
    nearest level, so the reconstruction is within half a step)."""
    k = _random_k()
    codes, s, z = kivi.quantize_k(k, bits, 32)
    xh = kivi.dequantize_k(codes, s, z, 32)
    x = k.astype(np.float64)
    s_t = np.repeat(s, 32, axis=0).astype(np.float64)
    mag = np.maximum(np.abs(np.repeat(z, 32, axis=0)), np.abs(x))
    slack = 2.0 ** -21 * mag + 2.0 ** -22 * s_t * (2 ** bits)
    assert np.all(np.abs(xh - x) <= s_t / 2 + slack)


@pytest.mark.parametrize("bits", [2, 4])
def test_error_bound_v(bits):
    v = _random_v()
    codes, s, z = kivi.quantize_v(v, bits)
    xh = kivi.dequantize_v(codes, s, z)
    x = v.astype(np.float64)
    s_t = s.astype(np.float64)[:, None]
    mag = np.maximum(np.abs(z)[:, None], np.abs(x))
    slack = 2.0 ** -21 * mag + 2.0 ** -22 * s_t * (2 ** bits)
    assert np.all(np.abs(xh - x) <= s_t / 2 + slack)


@pytest.mark.parametrize("bits", [2, 4])
def test_constant_groups_exact(bits):
    k = _random_k(64, 128)
    k[:32, 5] = np.float16(-3.1416)       # one constant channel in group 0
    k[32:, :] = np.float16(0.7)           # group 1 constant everywhere
    codes, s, z = kivi.quantize_k(k, bits, 32)
    xh = kivi.dequantize_k(codes, s, z, 32)
    assert s[0, 5] == 0 and np.all(codes[:32, 5] == 0)
    assert np.all(xh[:32, 5] == k[:32, 5].astype(F32))
    assert np.all(s[1] == 0) and np.all(xh[32:] == k[32:].astype(F32))
    v = _random_v(8, 128)
    v[3, :] = np.float16(-12.5)
    vc, vs, vz = kivi.quantize_v(v, bits)
    assert vs[3] == 0 and np.all(vc[3] == 0)
    assert np.all(kivi.dequantize_v(vc, vs, vz)[3] == v[3].astype(F32))


@pytest.mark.parametrize("bits", [2, 4])
def test_endpoints_and_monotone(bits):
    qmax = 2 ** bits - 1
    k = _random_k()
    codes, s, z = kivi.quantize_k(k, bits, 32)
    g = k.astype(F32).reshape(4, 32, 128)
    c = codes.reshape(4, 32, 128)
    amin = g.argmin(axis=1)
    amax = g.argmax(axis=1)
    for gi in range(4):
        for d in range(128):
            if s[gi, d] > 0:
                assert c[gi, amin[gi, d], d] == 0
                assert c[gi, amax[gi, d], d] == qmax
            order = np.argsort(g[gi, :, d], kind="stable")
            assert np.all(np.diff(c[gi, order, d].astype(int)) >= 0)


@pytest.mark.parametrize("bits", [2, 4])
def test_grid_values_round_trip(bits):
    """Values exactly on the grid mn + j·s get code j and reconstruct exactly."""
    qmax = 2 ** bits - 1
    mn, step = -1.5, 0.25                      # s = 0.25 exactly (power of 2)
    levels = mn + step * np.arange(qmax + 1)
    T = 32
    col = np.resize(levels, T)                 # every level present, incl. endpoints
    k = _fp16(np.tile(col[:, None], (1, 128)))
    codes, s, z = kivi.quantize_k(k, bits, 32)
    assert np.all(s == F32(step)) and np.all(z == F32(mn))
    expect = np.resize(np.arange(qmax + 1), T)
    assert np.all(codes == expect[:, None])
    assert np.all(kivi.dequantize_k(codes, s, z, 32) == k.astype(F32))


def _fp16_values_between(lo, hi):
    allv = np.arange(0, 1 << 16, dtype=np.uint32).astype(np.uint16).view(np.float16)
    allv = allv[np.isfinite(allv)].astype(np.float64)
    return np.unique(allv[(allv >= lo) & (allv <= hi)])


@pytest.mark.parametrize("bits,mn,mx", [(2, -1.0, 1.0), (2, 0.3, 7.9),
                                        (4, -2.5, 0.6), (4, -1000.0, 3.0)])
def test_brute_force_nearest_level(bits, mn, mx):
    """Every fp16 x in [mn, mx] as a member of a group whose other members pin
    the range to [mn, mx]: its code is the index of the nearest grid point
    mn + j·s (computed in fp64), except where two grid points are within
    1e-6·s of a tie — there fp32 rounding may go either way."""
    mn16, mx16 = np.float16(mn), np.float16(mx)
    xs = _fp16_values_between(float(mn16), float(mx16))
    T = 32
    k = np.empty((T, len(xs)), np.float16)
    k[0, :] = mn16
    k[1, :] = mx16
    k[2:, :] = mn16
    k[5, :] = xs.astype(np.float16)
    D = len(xs)
    pad = (-D) % 16
    k = np.concatenate([k, np.repeat(k[:, :1], pad, axis=1)], axis=1)
    codes, s, z = kivi.quantize_k(k, bits, 32)
    s64 = float(s[0, 0])
    qmax = 2 ** bits - 1
    grid = float(mn16) + s64 * np.arange(qmax + 1)
    dist = np.abs(xs[:, None] - grid[None, :])
    nearest = dist.argmin(axis=1)
    srt = np.sort(dist, axis=1)
    near_tie = (srt[:, 1] - srt[:, 0]) < 1e-6 * s64
    got = codes[5, :D].astype(int)
    bad = (got != nearest) & ~near_tie
    assert not bad.any(), (xs[bad][:5], got[bad][:5], nearest[bad][:5])
    assert len(xs) > 100


@pytest.mark.parametrize("bits", [2, 4])
def test_k_is_per_channel_v_is_per_token(bits):
    """Scaling one K channel changes only that channel's parameters and codes;
    scaling one V token changes only that token's. A transposed axis fails."""
    k = _random_k(64, 128)
    c0, s0, z0 = kivi.quantize_k(k, bits, 32)
    k2 = k.copy()
    k2[:, 17] = _fp16(k[:, 17].astype(F32) * 8)
    c1, s1, z1 = kivi.quantize_k(k2, bits, 32)
    other = np.arange(128) != 17
    assert np.array_equal(c0[:, other], c1[:, other])
    assert np.array_equal(s0[:, other], s1[:, other])
    assert not np.array_equal(s0[:, 17], s1[:, 17])
    v = _random_v(64, 128)
    c0, s0, z0 = kivi.quantize_v(v, bits)
    v2 = v.copy()
    v2[9, :] = _fp16(v[9].astype(F32) * 8)
    c1, s1, z1 = kivi.quantize_v(v2, bits)
    keep = np.arange(64) != 9
    assert np.array_equal(c0[keep], c1[keep]) and np.array_equal(s0[keep], s1[keep])
    assert s1[9] != s0[9]


def test_groups_are_token_aligned():
    """K statistics span exactly tokens [gG, gG+G): changing token 40 changes
    group 1 (tokens 32..63) only."""
    k = _random_k(96, 128)
    c0, s0, z0 = kivi.quantize_k(k, 2, 32)
    k2 = k.copy()
    k2[40, :] = _fp16(np.full(128, 60000.0))
    c1, s1, z1 = kivi.quantize_k(k2, 2, 32)
    assert np.array_equal(s0[[0, 2]], s1[[0, 2]]) and np.array_equal(c0[:32], c1[:32])
    assert np.array_equal(c0[64:], c1[64:])
    assert np.all(s1[1] > s0[1])


def test_prefill_split():
    G, R = 32, 128
    assert kivi.prefill_split(256, G, R) == (128, 128)      # tiny MHA workload
    assert kivi.prefill_split(32768, G, R) == (32640, 128)
    assert kivi.prefill_split(100, G, R) == (0, 100)        # S ≤ R: all FP16
    assert kivi.prefill_split(128, G, R) == (0, 128)
    assert kivi.prefill_split(129, G, R) == (32, 97)
    assert kivi.prefill_split(96, G, 0) == (96, 0)          # R = 0, S % G == 0
    assert kivi.prefill_split(100, G, 0) == (96, 4)
    for S in range(1, 700):
        for R_ in (0, 32, 64, 128):
            nq, nr = kivi.prefill_split(S, G, R_)
            assert nq % G == 0 and nq + nr == S and 0 <= nr <= kivi.window_capacity(G, R_)
            if R_ > 0 and S > R_:
                assert nr > R_ - G    # the newest R tokens stay FP16 (all but < G)


# ----------------------------------------------------------------- packing ---

@pytest.fixture(scope="module")
def words(golden_dir):
    with open(os.path.join(golden_dir, "packed_words.json")) as f:
        return json.load(f)


def test_pack_k_golden(words):
    e = words["k_2bit_one_token_16_channels"]
    codes = np.zeros((1, 128), np.uint8)
    codes[0, :16] = e["codes"]
    w = kivi.pack_k(codes, 2)
    assert w.shape == (1, 8) and int(w[0, 0]) == int(e["word_hex"], 16)
    assert np.all(w[0, 1:] == 0)
    e = words["k_4bit_one_token_8_channels"]
    codes = np.zeros((1, 128), np.uint8)
    codes[0, 8:16] = e["codes"]                          # second word
    w = kivi.pack_k(codes, 4)
    assert w.shape == (1, 16) and int(w[0, 1]) == int(e["word_hex"], 16)


def test_pack_v_golden(words):
    e = words["v_2bit_channel_tokens_0_to_15"]
    codes = np.zeros((32, 128), np.uint8)
    codes[:16, 3] = e["codes_by_token"]                  # channel 3, tokens 0..15
    w = kivi.pack_v(codes, 2, 32)
    assert w.shape == (1, 128, 2)
    assert int(w[0, 3, 0]) == int(e["word_hex"], 16)
    assert np.count_nonzero(w) == 1
    e = words["v_4bit_channel_tokens_0_to_7"]
    codes = np.zeros((32, 128), np.uint8)
    codes[8:16, 5] = e["codes_by_token"]                 # channel 5, tokens 8..15: word 1
    w = kivi.pack_v(codes, 4, 32)
    assert w.shape == (1, 128, 4)
    assert int(w[0, 5, 1]) == int(e["word_hex"], 16)
    assert np.count_nonzero(w) == 1


@pytest.mark.parametrize("bits", [2, 4])
def test_pack_round_trip(bits):
    codes = RNG.integers(0, 2 ** bits, (96, 128)).astype(np.uint8)
    assert np.array_equal(kivi.unpack_k(kivi.pack_k(codes, bits), bits, 128), codes)
    assert np.array_equal(kivi.unpack_v(kivi.pack_v(codes, bits, 32), bits, 32), codes)


@pytest.mark.parametrize("bits", [2, 4])
def test_v_channel_subgroups(bits):
    """V per token with one scale and zero per run of 32 channels: each run's
    scale is (max − min)/(2^b − 1) of those 32 values alone (a run with a ×50
    outlier does not widen its neighbours' steps); Gc = D reduces to plain
    per-token V; reconstruction within half of the run's own step."""
    rng = np.random.default_rng(21)
    v = rng.normal(0, 1, (40, 128)).astype(np.float16)
    v[:, 70] *= 50                                     # outlier channel in run 2
    c_sub, s_sub, z_sub = kivi.quantize_v(v, bits, 32)
    assert s_sub.shape == (40, 4) and z_sub.shape == (40, 4)
    x = v.astype(np.float32)
    for m in range(4):
        run = x[:, 32 * m:32 * m + 32]
        assert np.array_equal(z_sub[:, m], run.min(axis=1))
        assert np.array_equal(s_sub[:, m], (run.max(axis=1) - run.min(axis=1)) / np.float32(2 ** bits - 1))
    c_all, s_all, z_all = kivi.quantize_v(v, bits)
    assert np.all(s_sub[:, [0, 1, 3]] < s_all[:, None])   # runs without the outlier: finer
    c_one, s_one, z_one = kivi.quantize_v(v, bits, 128)
    assert np.array_equal(c_one, c_all) and np.array_equal(s_one[:, 0], s_all)
    xh = kivi.dequantize_v(c_sub, s_sub, z_sub)
    step = np.repeat(s_sub, 32, axis=1)
    assert np.all(np.abs(xh - x) <= step / 2 + 1e-6 * np.abs(x) + 1e-7)
    assert np.abs(xh - x)[:, :64].max() < np.abs(kivi.dequantize_v(c_all, s_all, z_all) - x)[:, :64].max()
