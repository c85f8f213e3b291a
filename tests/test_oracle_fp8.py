"""Pins of the oracle's E4M3 table, encoder and per-tensor scale.

torch's CPU float8_e4m3fn cast is used as a black-box library routine: it
rounds to nearest-even but does not saturate, so inputs are clamped to ±448
first (the saturating reading the oracle follows)."""
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
