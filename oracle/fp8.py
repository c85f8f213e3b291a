"""FP8 KV-cache quantization, E4M3 and E5M2 (oracle side; test infrastructure).

E4M3 ([KIVI-page] §5: 1 sign, 4 exponent, 3 mantissa bits). The OCP "fn"
variant named by the dtype `float8_e4m3fn` on [FP8-page] is used: exponent
bias 7, no infinities, the all-ones pattern S.1111.111 is NaN, so the largest
finite magnitude is 1.75 · 2^8 = 448 — the divisor of [FP8-page] ("FP8 E4M3
max value"). Exponent field 0 holds subnormals m · 2^-9.

E5M2 ([Tutorial] §十八.4: the wider-range, coarser FP8 format): 1 sign,
5 exponent, 2 mantissa bits, exponent bias 15, IEEE-style specials (exponent
field 31 is ±inf with mantissa 0, NaN otherwise), so the largest finite
magnitude is 1.75 · 2^15 = 57344; exponent field 0 holds subnormals m · 2^-16.
Reading: the scale divides by the format's largest finite value, as the E4M3
scale divides by 448.

Dynamic scale ([FP8-page], section "自定义KV Cache量化的实现路径"):
  s = amax(|x|) / FMAX, computed in fp32, over the whole tensor (per-tensor,
  [Tutorial] §十.1) or over each KV head (per-attention-head scales for K and
  V, one per KV head: [Tutorial] §十八.6, [KIVI-page] §6.3).
Encoding ([Tutorial] §十, FP8 formula q = cast_fp8(x / s)):
  t = x / s (fp32, IEEE division), clamped to [−FMAX, FMAX] (saturation; the
  pages give no overflow rule, [Tutorial] §十.2 warns about overflow), then
  rounded to the nearest value of the format, ties to the even code, sign of
  zero kept. s = 0 (an all-zero tensor or head) gives code 0 everywhere.
Decoding: x̂ = float(value(code)) · s in fp32 ([Tutorial] §十: cast to high
precision, multiply by s).

Attention in the FP8 domain ([Tutorial] §十八.7; [KIVI-page] §6, the tip
after §6.3): the query is quantized too, with one scale per query head
(q_scale has num_heads entries, [Tutorial] §十八.6). Reading: no calibrated
scale exists here, so each decode step takes the dynamic scale of its own
query row, s_q[b, hq] = amax_d |q[b, hq, d]| / 448 in fp32, and the E4M3
codes follow the encoder above; scores then use q̂ = value(code) · s_q.

Parity pins live in tests/test_oracle_fp8.py; only tests, the package's smoke
check and the benchmark's CPU baseline use this module.
"""
from __future__ import annotations

import numpy as np

F32 = np.float32
E4M3_MAX = 448.0
E5M2_MAX = 57344.0
FMAX = {"e4m3": E4M3_MAX, "e5m2": E5M2_MAX}


def decode_table(fmt: str = "e4m3") -> np.ndarray:
    """Value of each of the 256 codes (fp64; NaN / ±inf where the format has them)."""
    ebits, mbits, bias = {"e4m3": (4, 3, 7), "e5m2": (5, 2, 15)}[fmt]
    emax_field = (1 << ebits) - 1
    vals = np.empty(256, np.float64)
    for code in range(256):
        sign = -1.0 if code & 0x80 else 1.0
        e = (code >> mbits) & emax_field
        m = code & ((1 << mbits) - 1)
        if fmt == "e4m3" and e == emax_field and m == (1 << mbits) - 1:
            vals[code] = np.nan
        elif fmt == "e5m2" and e == emax_field:
            vals[code] = sign * np.inf if m == 0 else np.nan
        elif e == 0:
            vals[code] = sign * (m / (1 << mbits)) * 2.0 ** (1 - bias)
        else:
            vals[code] = sign * (1.0 + m / (1 << mbits)) * 2.0 ** (e - bias)
    return vals


_TABLE = {f: decode_table(f) for f in FMAX}
# codes 0x00 .. largest finite: the non-negative finite values, increasing
_POS = {f: t[:int(np.flatnonzero(t[:0x80] == FMAX[f])[0]) + 1] for f, t in _TABLE.items()}


def encode(t: np.ndarray, fmt: str = "e4m3") -> np.ndarray:
    """Nearest code of each finite fp32 t, ties to even, saturating at ±FMAX."""
    pos = _POS[fmt]
    top = len(pos) - 1
    t = np.asarray(t, dtype=F32)
    neg = np.signbit(t)
    a = np.minimum(np.abs(t).astype(np.float64), FMAX[fmt])
    hi = np.searchsorted(pos, a, side="left")             # first value ≥ a
    hi = np.minimum(hi, top)
    lo = np.maximum(hi - 1, 0)
    d_lo = a - pos[lo]
    d_hi = pos[hi] - a
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (hi % 2 == 0))
    code = np.where(pick_hi, hi, lo).astype(np.uint8)
    return code | (neg.astype(np.uint8) << np.uint8(7))


def decode(codes: np.ndarray, fmt: str = "e4m3") -> np.ndarray:
    """Codes → fp32 values."""
    return _TABLE[fmt][np.asarray(codes, dtype=np.uint8)].astype(F32)


def tensor_scale(x: np.ndarray, fmt: str = "e4m3") -> np.float32:
    """s = amax(|x|) / FMAX in fp32 ([FP8-page])."""
    amax = F32(np.max(np.abs(np.asarray(x, dtype=F32)))) if np.size(x) else F32(0)
    return F32(amax / F32(FMAX[fmt]))


def head_scales(x: np.ndarray, fmt: str = "e4m3") -> np.ndarray:
    """One scale per KV head of a [B, H, S, D] tensor: amax over (b, t, d) of
    that head, / FMAX in fp32 ([Tutorial] §十八.6)."""
    x = np.asarray(x, dtype=F32)
    return np.array([tensor_scale(x[:, h], fmt) for h in range(x.shape[1])], F32)


def quantize(x: np.ndarray, s: np.float32, fmt: str = "e4m3") -> np.ndarray:
    """codes = FP8(clamp(x / s)); all zero when s == 0."""
    x = np.asarray(x, dtype=F32)
    if s == 0:
        return np.zeros(x.shape, np.uint8)
    return encode(x / F32(s), fmt)


def dequantize(codes: np.ndarray, s: np.float32, fmt: str = "e4m3") -> np.ndarray:
    return decode(codes, fmt) * F32(s)


def quantize_query(q: np.ndarray) -> tuple[np.ndarray, np.ndarray]:
    """E4M3 codes and per-row scales of a [B, Hq, D] fp32 query: one scale
    per (b, query head), amax over that head's D values / 448."""
    q = np.asarray(q, dtype=F32)
    B, Hq, _ = q.shape
    scales = np.zeros((B, Hq), F32)
    codes = np.zeros(q.shape, np.uint8)
    for b in range(B):
        for h in range(Hq):
            scales[b, h] = tensor_scale(q[b, h])
            codes[b, h] = quantize(q[b, h], scales[b, h])
    return codes, scales


def dequantize_query(codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """q̂[b, hq, d] = value(code) · s_q[b, hq] in fp32."""
    return decode(codes) * np.asarray(scales, F32)[..., None]
