"""Pins of the oracle's E4M3 and E5M2 tables, encoders, per-tensor and
per-KV-head scales.

torch's CPU float8_e4m3fn and float8_e5m2 casts are used as black-box library
routines: they round to nearest-even but do not saturate, so inputs are
clamped to ±448 (±57344) first (the saturating reading the oracle follows).
The E5M2 table is also pinned by a fact of the formats alone: an E5M2 code is
the high byte of the fp16 of the same value."""
import json
import os

import numpy as np
import pytest
import torch

from oracle import fp8

F32 = np.float32


def _torch_encode(t: np.ndarray) -> np.ndarray:
    x = torch.from_numpy(np.asarray(t, np.float32)).clamp(-448.0, 448.0)
    return x.to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def test_table_structure(golden_dir):
    with open(os.path.join(golden_dir, "pages_worked_numbers.json")) as f:
        e4m3_max = json.load(f)["e4m3_max"]["value"]
    t = fp8.decode_table()
    finite = np.isfinite(t)
    assert finite.sum() == 254
    assert np.isnan(t[0x7F]) and np.isnan(t[0xFF])
    assert np.nanmax(t) == e4m3_max == t[0x7E]
    assert np.nanmin(t) == -e4m3_max == t[0xFE]
    assert t[0x01] == 2.0 ** -9                       # smallest subnormal
    assert t[0x08] == 2.0 ** -6                       # smallest normal
    assert t[0x38] == 1.0                             # exponent field = bias
    assert t[0x00] == 0 and np.signbit(t[0x80])
    pos = t[:0x7F]
    assert np.all(np.diff(pos) > 0)                   # codes ordered by value


def test_table_matches_torch():
    codes = torch.arange(256, dtype=torch.uint8)
    ref = codes.view(torch.float8_e4m3fn).to(torch.float32).numpy().astype(np.float64)
    t = fp8.decode_table()
    both_nan = np.isnan(ref) & np.isnan(t)
    assert np.all(both_nan | (ref == t))


def test_encode_all_fp16_patterns():
    allv = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16).view(np.float16)
    allv = allv[np.isfinite(allv)].astype(np.float32)
    for s in (1.0, 0.001953125, 3.0, 0.37, 150.1, 1e-3):
        t = allv / F32(s)
        assert np.array_equal(fp8.encode(t), _torch_encode(t)), s


def test_encode_random_fp32():
    rng = np.random.default_rng(7)
    t = np.concatenate([
        rng.normal(0, 1, 500_000), rng.normal(0, 100, 500_000),
        rng.uniform(-500, 500, 500_000), rng.normal(0, 1e-3, 500_000)]).astype(F32)
    assert np.array_equal(fp8.encode(t), _torch_encode(t))


def test_ties_and_saturation():
    # 464 lies halfway between 448 (code 0x7E, even) and the missing 480: → 448
    assert fp8.encode(np.array([464.0, 470.0, 1e6, -1e6]))[:].tolist() == [0x7E, 0x7E, 0x7E, 0xFE]
    # 1.0625 is halfway between 1.0 (0x38) and 1.125 (0x39): ties to even → 0x38
    assert fp8.encode(np.array([1.0625, 1.1875]))[:].tolist() == [0x38, 0x3A]
    # halfway between subnormals 1·2^-9 (0x01) and 2·2^-9 (0x02) → even 0x02
    assert fp8.encode(np.array([1.5 * 2 ** -9]))[0] == 0x02
    # below half the smallest subnormal → ±0 with the sign kept
    assert fp8.encode(np.array([2 ** -11, -2 ** -11]))[:].tolist() == [0x00, 0x80]


def test_representable_round_trip():
    t = fp8.decode_table()
    codes = np.array([c for c in range(256) if np.isfinite(t[c])], np.uint8)
    vals = t[codes].astype(F32)
    assert np.array_equal(fp8.encode(vals), codes)
    for s in (F32(0.5), F32(2.0 ** -4), F32(8.0)):      # power-of-2 scales: exact
        x = vals * s
        assert np.array_equal(fp8.quantize(x, s), codes)
        assert np.array_equal(fp8.dequantize(codes, s), x)


def test_tensor_scale():
    rng = np.random.default_rng(3)
    x = (rng.normal(0, 3, (4, 64)).astype(np.float16)).astype(F32)
    x[2, 7] = -37.25
    s = fp8.tensor_scale(x)
    assert s == F32(F32(37.25) / F32(448.0))
    codes = fp8.quantize(x, s)
    assert codes[2, 7] == 0xFE                          # −amax → −448
    err = np.abs(fp8.dequantize(codes, s) - x)
    # relative step of E4M3 is 2^-3: normal values within 2^-4 relative, plus subnormal floor
    assert np.all(err <= np.abs(x) * 2.0 ** -4 + s * 2.0 ** -10 + 1e-12)
    z = np.zeros((3, 5), F32)
    assert fp8.tensor_scale(z) == 0 and not fp8.quantize(z, fp8.tensor_scale(z)).any()


# ---------------------------------------------------------------- E5M2 ---

def _torch_encode_e5m2(t: np.ndarray) -> np.ndarray:
    # torch's cast rounds to nearest-even and overflows to inf: clamp first
    x = torch.from_numpy(np.asarray(t, np.float32)).clamp(-57344.0, 57344.0)
    return x.to(torch.float8_e5m2).view(torch.uint8).numpy()


def test_e5m2_table_structure():
    t = fp8.decode_table("e5m2")
    assert np.isfinite(t).sum() == 248
    assert t[0x7C] == np.inf and t[0xFC] == -np.inf
    assert all(np.isnan(t[c]) for c in (0x7D, 0x7E, 0x7F, 0xFD, 0xFE, 0xFF))
    assert t[0x7B] == 57344.0 == fp8.E5M2_MAX and t[0xFB] == -57344.0
    assert t[0x01] == 2.0 ** -16                      # smallest subnormal
    assert t[0x04] == 2.0 ** -14                      # smallest normal
    assert t[0x3C] == 1.0                             # exponent field = bias
    assert np.all(np.diff(t[:0x7C]) > 0)


def test_e5m2_is_the_high_byte_of_fp16():
    """E5M2 shares fp16's sign, exponent width and bias: every code, placed in
    the high byte of a 16-bit word, is the fp16 of the same value."""
    t = fp8.decode_table("e5m2")
    h = (np.arange(256, dtype=np.uint16) << 8).view(np.float16).astype(np.float64)
    assert np.all((np.isnan(t) & np.isnan(h)) | (t == h))


def test_e5m2_table_matches_torch():
    ref = torch.arange(256, dtype=torch.uint8).view(torch.float8_e5m2).to(torch.float32)
    ref = ref.numpy().astype(np.float64)
    t = fp8.decode_table("e5m2")
    assert np.all((np.isnan(ref) & np.isnan(t)) | (ref == t))


def test_e5m2_encode_all_fp16_patterns():
    allv = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16).view(np.float16)
    allv = allv[np.isfinite(allv)].astype(np.float32)
    for s in (1.0, 2.0 ** -8, 3.0, 0.37, 1.7e-3, 0.011):
        t = allv / F32(s)
        assert np.array_equal(fp8.encode(t, "e5m2"), _torch_encode_e5m2(t)), s


def test_e5m2_ties_and_saturation():
    enc = lambda *x: fp8.encode(np.array(x, np.float32), "e5m2").tolist()
    # 61440 is halfway between 57344 (0x7B) and the missing 65536: saturates
    assert enc(61440.0, 1e9, -1e9) == [0x7B, 0x7B, 0xFB]
    # 1.125 halfway between 1.0 (0x3C) and 1.25 (0x3D) → even 0x3C; 1.375 → 0x3E
    assert enc(1.125, 1.375) == [0x3C, 0x3E]
    # halfway between subnormals 2^-16 (0x01) and 2^-15 (0x02) → even 0x02
    assert enc(1.5 * 2 ** -16) == [0x02]
    assert enc(2 ** -18, -2 ** -18) == [0x00, 0x80]


def test_e5m2_scale_and_error():
    rng = np.random.default_rng(5)
    x = (rng.normal(0, 3, (4, 64)).astype(np.float16)).astype(F32)
    x[1, 3] = 41.5
    s = fp8.tensor_scale(x, "e5m2")
    assert s == F32(F32(41.5) / F32(57344.0))
    codes = fp8.quantize(x, s, "e5m2")
    assert codes[1, 3] == 0x7B
    err = np.abs(fp8.dequantize(codes, s, "e5m2") - x)
    # relative step of E5M2 is 2^-2: within 2^-3 relative, plus the subnormal floor
    assert np.all(err <= np.abs(x) * 2.0 ** -3 + s * 2.0 ** -17 + 1e-12)


# --------------------------------------------------- per-KV-head scales ---

@pytest.mark.parametrize("fmt", ["e4m3", "e5m2"])
def test_head_scales(fmt):
    """One scale per KV head: amax over (batch, tokens, channels) of that head;
    the same numbers as the per-tensor scale of each head's slice alone."""
    rng = np.random.default_rng(11)
    x = rng.normal(0, 1, (2, 3, 40, 16)).astype(np.float16)
    x[1, 2, 5, 9] = 300.0                              # an outlier head
    s = fp8.head_scales(x, fmt)
    fmax = F32(fp8.FMAX[fmt])
    for h in range(3):
        amax = F32(np.abs(x[:, h].astype(F32)).max())
        assert s[h] == F32(amax / fmax)
    assert s[2] == F32(F32(300.0) / fmax) and s[0] < s[2] / 50
    assert np.max(s) == fp8.tensor_scale(x, fmt)


# ------------------------------------------------- FP8-domain query ---

def test_query_quantization():
    """Per-(b, query head) E4M3 query codes ([Tutorial] §十八.7): each row is
    the per-tensor quantizer applied to that row alone; the row's largest
    magnitude maps to ±448 (0x7E / 0xFE); a zero row has scale 0 and codes 0;
    q̂ stays within E4M3's half step of q."""
    rng = np.random.default_rng(9)
    q = rng.normal(0, 1, (3, 4, 128)).astype(F32)
    q[1, 2] *= 1000
    q[2, 3] = 0
    q[0, 1, 17] = -9.5                         # this row's amax, negative
    codes, s = fp8.quantize_query(q)
    assert s.shape == (3, 4) and codes.shape == q.shape
    assert s[0, 1] == F32(F32(9.5) / F32(448)) and codes[0, 1, 17] == 0xFE
    assert s[2, 3] == 0 and not codes[2, 3].any()
    for b in range(3):
        for h in range(4):
            assert np.array_equal(codes[b, h], fp8.quantize(q[b, h], fp8.tensor_scale(q[b, h])))
    qh = fp8.dequantize_query(codes, s)
    assert np.all(np.abs(qh - q) <= np.abs(q) * 2.0 ** -4 + s[..., None] * 2.0 ** -10 + 1e-12)
    # a row that is already on the E4M3 grid at a power-of-two scale is exact
    g = fp8.decode_table()[np.arange(0, 0x7F, 1)][:128].astype(F32)
    g[-1] = 448.0
    row = (g * F32(0.25))[None, None, :]
    c2, s2 = fp8.quantize_query(row)
    assert s2[0, 0] == F32(0.25) and np.array_equal(fp8.dequantize_query(c2, s2), row)
