"""FP8 E4M3 per-tensor quantization (oracle side).

Format ([KIVI-page] §5: E4M3 = 1 sign, 4 exponent, 3 mantissa bits). The OCP
"fn" variant named by the dtype `float8_e4m3fn` on [FP8-page] is used:
exponent bias 7, no infinities, the all-ones pattern S.1111.111 is NaN, so the
largest finite magnitude is 1.75 · 2^8 = 448 — the divisor of [FP8-page]
("FP8 E4M3 max value"). Exponent field 0 holds subnormals m · 2^-9.

Per-tensor dynamic scale ([FP8-page], section "自定义KV Cache量化的实现路径"):
  s = amax(|x|) / 448 over the whole tensor, computed in fp32.
Encoding ([Tutorial] §十, FP8 formula q = cast_fp8(x / s)):
  t = x / s (fp32, IEEE division), clamped to [−448, 448] (saturation; the
  pages give no overflow rule, [Tutorial] §十.2 warns about overflow), then
  rounded to the nearest E4M3 value, ties to the even code, sign of zero kept.
  s = 0 (an all-zero tensor) gives code 0 everywhere.
Decoding: x̂ = float(value(code)) · s in fp32 ([Tutorial] §十: cast to high
precision, multiply by s).
"""
from __future__ import annotations

import numpy as np

F32 = np.float32
E4M3_MAX = 448.0


def decode_table() -> np.ndarray:
    """Value of each of the 256 codes (fp64; NaN for 0x7F and 0xFF)."""
    vals = np.empty(256, np.float64)
    for code in range(256):
        sign = -1.0 if code & 0x80 else 1.0
        e = (code >> 3) & 0xF
        m = code & 0x7
        if e == 0xF and m == 0x7:
            vals[code] = np.nan
        elif e == 0:
            vals[code] = sign * m * 2.0 ** -9
        else:
            vals[code] = sign * (1.0 + m / 8.0) * 2.0 ** (e - 7)
    return vals


_TABLE = decode_table()
_POS = _TABLE[:0x7F]  # codes 0x00..0x7E: the non-negative finite values, increasing


def encode(t: np.ndarray) -> np.ndarray:
    """Nearest E4M3 code of each finite fp32 t, ties to even, saturating."""
    t = np.asarray(t, dtype=F32)
    neg = np.signbit(t)
    a = np.minimum(np.abs(t).astype(np.float64), E4M3_MAX)
    hi = np.searchsorted(_POS, a, side="left")            # first value ≥ a
    hi = np.minimum(hi, 0x7E)
    lo = np.maximum(hi - 1, 0)
    d_lo = a - _POS[lo]
    d_hi = _POS[hi] - a
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (hi % 2 == 0))
    code = np.where(pick_hi, hi, lo).astype(np.uint8)
    return code | (neg.astype(np.uint8) << np.uint8(7))


def decode(codes: np.ndarray) -> np.ndarray:
    """E4M3 codes → fp32 values."""
    return _TABLE[np.asarray(codes, dtype=np.uint8)].astype(F32)


def tensor_scale(x: np.ndarray) -> np.float32:
    """s = amax(|x|) / 448 in fp32 ([FP8-page])."""
    amax = F32(np.max(np.abs(np.asarray(x, dtype=F32)))) if np.size(x) else F32(0)
    return F32(amax / F32(E4M3_MAX))


def quantize(x: np.ndarray, s: np.float32) -> np.ndarray:
    """codes = E4M3(clamp(x / s)); all zero when s == 0."""
    x = np.asarray(x, dtype=F32)
    if s == 0:
        return np.zeros(x.shape, np.uint8)
    return encode(x / F32(s))


def dequantize(codes: np.ndarray, s: np.float32) -> np.ndarray:
    return decode(codes) * F32(s)
