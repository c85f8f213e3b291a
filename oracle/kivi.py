"""KIVI asymmetric group quantization (oracle side).

Method ([KIVI-page] §2, §3.2, §3.4; [Tutorial] §九.1–九.3):
  * K is quantized per channel: the tokens of one group (G = 32 consecutive
    tokens, aligned to multiples of G) share one scale and zero-point per
    channel.
  * V is quantized per token: each token has one scale and zero-point over its
    head_dim channels, or, as a variant, one per run of Gc consecutive channels
    of the token (channel sub-groups [Gc·m, Gc·m + Gc); reading: the
    per-token axis of [Tutorial] §九.2 with the group granularity of
    [Tutorial] §十.1 applied along the channels, as the q_group_size knob of
    the quantized caches the pages describe does).
  * Codes have 2 or 4 bits.

Quantizer ([Tutorial] §十, affine formula q = clamp(round(x/s) + z, qmin, qmax),
x̂ = (q − z)·s). The pages do not say how s and z come from the data; this
oracle uses the min/max asymmetric reading with the zero-point kept as an fp32
offset (z = mn, i.e. the integer-domain zero-point of the page formula is
−mn/s). Each step, in fp32 with correctly rounded operations:
    mn, mx = group minimum, maximum
    s      = (mx − mn) / (2^b − 1)
    code   = clamp(rint((x − mn) / s), 0, 2^b − 1), rint = half to even;
             code = 0 for a constant group (s = 0)
    x̂      = float(code) · s + mn      (two roundings, no fused multiply-add)

Packing (layout of the device buffers; little-endian bit order):
  K: per token, its D channel codes packed along the channel axis; channel
     i of a word (32/b channels per word) at bits [b·i, b·i + b).
  V: per group and channel, the G token codes packed along the token axis,
     32/b tokens per word; token j of a word sits in the low 16 bits when j is
     even and in the high 16 bits when j is odd, at bit b·(j // 2) of its half.
"""
from __future__ import annotations

import numpy as np

F32 = np.float32


def prefill_split(seq_len: int, group: int, residual: int) -> tuple[int, int]:
    """(n_quant, n_resid) after a prefill of seq_len tokens.

    [KIVI-page] §3.2: the newest R tokens stay FP16, older ones form groups of
    G. With seq_len − R not a multiple of G, the split keeps every group whole
    and the window within its capacity: n_quant = G·max(0, min(⌊S/G⌋,
    ⌈(S−R)/G⌉)), so the window holds between R − G + 1 and R tokens (for R = 0:
    the incomplete last group, [KIVI-page] §3.1).
    """
    full = seq_len // group
    need = -((residual - seq_len) // group)  # ceil((S - R) / G)
    n_quant = group * max(0, min(full, need))
    return n_quant, seq_len - n_quant


def window_capacity(group: int, residual: int) -> int:
    """Tokens the FP16 window can hold: R, or G when R = 0."""
    return residual if residual > 0 else group


def _scale(mn: np.ndarray, mx: np.ndarray, bits: int) -> np.ndarray:
    return (mx.astype(F32) - mn.astype(F32)) / F32(2 ** bits - 1)


def _codes(x: np.ndarray, mn: np.ndarray, s: np.ndarray, bits: int) -> np.ndarray:
    qmax = 2 ** bits - 1
    with np.errstate(divide="ignore", invalid="ignore"):
        r = np.rint((x - mn) / s)
    r = np.where(s == 0, F32(0), r)
    return np.clip(r, 0, qmax).astype(np.uint8)


def quantize_k(k: np.ndarray, bits: int, group: int):
    """Per-channel group quantization of K.

    k: fp16 [T, D] with T a multiple of group.
    Returns codes uint8 [T, D], scale fp32 [T/G, D], zero fp32 [T/G, D].
    """
    T, D = k.shape
    assert T % group == 0
    x = k.astype(F32).reshape(T // group, group, D)
    mn = x.min(axis=1)                         # over the group's tokens
    mx = x.max(axis=1)
    s = _scale(mn, mx, bits)
    codes = _codes(x, mn[:, None, :], s[:, None, :], bits)
    return codes.reshape(T, D), s, mn.copy()


def quantize_v(v: np.ndarray, bits: int, channel_group: int | None = None):
    """Per-token quantization of V.

    v: fp16 [T, D]. Returns codes uint8 [T, D], scale fp32 [T], zero fp32 [T];
    with channel_group = Gc, one scale and zero per (token, run of Gc
    channels): scale, zero fp32 [T, D / Gc].
    """
    x = v.astype(F32)
    if channel_group is None:
        mn = x.min(axis=1)                     # over the token's channels
        mx = x.max(axis=1)
        s = _scale(mn, mx, bits)
        codes = _codes(x, mn[:, None], s[:, None], bits)
        return codes, s, mn.copy()
    T, D = x.shape
    xs = x.reshape(T, D // channel_group, channel_group)
    mn = xs.min(axis=2)                        # over each run of Gc channels
    mx = xs.max(axis=2)
    s = _scale(mn, mx, bits)
    codes = _codes(xs, mn[:, :, None], s[:, :, None], bits).reshape(T, D)
    return codes, s, mn.copy()


def dequantize_k(codes: np.ndarray, scale: np.ndarray, zero: np.ndarray,
                 group: int) -> np.ndarray:
    """x̂[t, d] = code[t, d] · s[t/G, d] + z[t/G, d] in fp32."""
    s = np.repeat(scale, group, axis=0)
    z = np.repeat(zero, group, axis=0)
    return codes.astype(F32) * s + z


def dequantize_v(codes: np.ndarray, scale: np.ndarray, zero: np.ndarray) -> np.ndarray:
    """x̂[t, d] = code[t, d] · s[t] + z[t] in fp32 (s[t, d // Gc] and
    z[t, d // Gc] with channel sub-groups)."""
    if scale.ndim == 2:
        gc = codes.shape[1] // scale.shape[1]
        scale = np.repeat(scale, gc, axis=1)
        zero = np.repeat(zero, gc, axis=1)
        return codes.astype(F32) * scale + zero
    return codes.astype(F32) * scale[:, None] + zero[:, None]


# ----------------------------------------------------------------- packing ---

def pack_k(codes: np.ndarray, bits: int) -> np.ndarray:
    """K codes [T, D] → uint32 [T, D·b/32], packed along channels."""
    T, D = codes.shape
    per = 32 // bits
    c = codes.astype(np.uint32).reshape(T, D // per, per)
    words = np.zeros((T, D // per), np.uint32)
    for i in range(per):
        words |= c[:, :, i] << np.uint32(bits * i)
    return words


def unpack_k(words: np.ndarray, bits: int, head_dim: int) -> np.ndarray:
    T = words.shape[0]
    per = 32 // bits
    mask = np.uint32(2 ** bits - 1)
    out = np.empty((T, head_dim // per, per), np.uint8)
    for i in range(per):
        out[:, :, i] = (words >> np.uint32(bits * i)) & mask
    return out.reshape(T, head_dim)


def _v_bit(j: int, bits: int) -> int:
    """Bit offset of token j of a V word: even tokens low half, odd high half."""
    return bits * (j // 2) + 16 * (j % 2)


def pack_v(codes: np.ndarray, bits: int, group: int) -> np.ndarray:
    """V codes [T, D] (T a multiple of G) → uint32 [T/G, D, G·b/32], each
    channel's G token codes of a group packed along tokens."""
    T, D = codes.shape
    per = 32 // bits
    c = codes.astype(np.uint32).reshape(T // group, group, D).transpose(0, 2, 1)
    c = c.reshape(T // group, D, group // per, per)
    words = np.zeros((T // group, D, group // per), np.uint32)
    for j in range(per):
        words |= c[..., j] << np.uint32(_v_bit(j, bits))
    return words


def unpack_v(words: np.ndarray, bits: int, group: int) -> np.ndarray:
    ng, D, _ = words.shape
    per = 32 // bits
    mask = np.uint32(2 ** bits - 1)
    out = np.empty((ng, D, group // per, per), np.uint8)
    for j in range(per):
        out[..., j] = (words >> np.uint32(_v_bit(j, bits))) & mask
    return out.reshape(ng, D, group).transpose(0, 2, 1).reshape(ng * group, D)
