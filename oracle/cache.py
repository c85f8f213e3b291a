"""Cache state machines (oracle side): prefill, append, flush, decode.

KIVI ([KIVI-page] §3.1–3.2; [Tutorial] §九.3): the cache is a grouped region
(whole groups of G tokens, K per channel, V per token, low-bit) followed by an
FP16 residual window holding the newest tokens. New tokens enter the window;
once it has accumulated R tokens they are all quantized, merged into the
grouped region and the window is cleared.

Readings (the pages leave these open):
  * Prefill split: see kivi.prefill_split.
  * Flush timing is lazy: the window is flushed when a token arrives and the
    window is already full, so a full window of R tokens is attended in FP16
    and the flush happens on the next append (decode appends, then attends,
    [Tutorial] §二.1).
  * R = 0: K needs a whole group before it has a scale ([KIVI-page] §3.1), so
    the incomplete group (< G tokens) is the only FP16 part; the window then
    holds up to G tokens.

FP8 ([FP8-page]; [KIVI-page] §6.2 fixes the scale after it is measured): the
per-tensor scales are computed from the prefill K and V and kept for appended
tokens, which saturate at ±448.

Every array is laid out as the device buffers are (see kivi.pack_k/pack_v):
  k_codes uint32 [B][H][CT][D·b/32], v_codes uint32 [B][H][NT][D][32·b/32],
  k_scale/k_zero fp32 [B][H][NG][D], v_scale/v_zero fp32 [B][H][CT],
  k_resid/v_resid fp16 [B][H][Rcap][D], with NG = ceil(C/G), CT = NG·G and
  NT = CT/32. V is quantized per token, so its codes are packed in tiles of
  VT = 32 tokens whatever the group size (G = 32, 64 or 128 sets only how many
  tokens share one K scale and zero-point per channel).
FP8 and FP16 caches use tiles of T = 32 tokens: K [B][H][CT][D] (token rows,
CT = ceil(C/T)·T) and V [B][H][NT][D][T] (per tile, one row of its T tokens per
channel); slots that hold no token are zero.
"""
from __future__ import annotations

import numpy as np

from . import attention, fp8, kivi

VT = 32          # tokens per packed V tile (KIVI)


class KiviCache:
    """bits: K's bit width; v_bits: V's (default: the same). Mixed widths
    (e.g. K 4-bit, V 2-bit) quantize each tensor with its own 2^b − 1 levels.
    v_group_channels: V scales and zero-points per run of that many channels
    of a token (default: one per token); v_scale / v_zero are then
    [B, H, CT, D / Gc]."""

    def __init__(self, batch, num_kv_heads, head_dim, bits, group, residual,
                 capacity, v_bits=None, v_group_channels=None):
        v_bits = bits if v_bits is None else v_bits
        assert bits in (2, 4) and v_bits in (2, 4)
        assert v_group_channels is None or head_dim % v_group_channels == 0
        self.Gc = v_group_channels
        assert residual % group == 0 and group % VT == 0
        self.B, self.H, self.D = batch, num_kv_heads, head_dim
        self.bits, self.G, self.R, self.C = bits, group, residual, capacity
        self.v_bits = v_bits
        self.Rcap = kivi.window_capacity(group, residual)
        self.NG = -(-capacity // group)
        self.CT = self.NG * group
        B, H, D = batch, num_kv_heads, head_dim
        self.k_codes = np.zeros((B, H, self.CT, D * bits // 32), np.uint32)
        self.NT = self.CT // VT
        self.v_codes = np.zeros((B, H, self.NT, D, VT * v_bits // 32), np.uint32)
        self.k_scale = np.zeros((B, H, self.NG, D), np.float32)
        self.k_zero = np.zeros((B, H, self.NG, D), np.float32)
        vshape = (B, H, self.CT) if self.Gc is None else (B, H, self.CT, D // self.Gc)
        self.v_scale = np.zeros(vshape, np.float32)
        self.v_zero = np.zeros(vshape, np.float32)
        self.k_resid = np.zeros((B, H, self.Rcap, D), np.float16)
        self.v_resid = np.zeros((B, H, self.Rcap, D), np.float16)
        self.n_quant = 0
        self.n_resid = 0
        self.flush_steps = []   # append indices (1-based) that flushed
        self.n_appends = 0

    @property
    def n_tokens(self):
        return self.n_quant + self.n_resid

    def _quantize_groups(self, k, v, t0):
        """Quantize fp16 k, v [B, H, T, D] (T a multiple of G) as the groups
        starting at token t0 (a multiple of G)."""
        T = k.shape[2]
        g0 = t0 // self.G
        for b in range(self.B):
            for h in range(self.H):
                kc, ks, kz = kivi.quantize_k(k[b, h], self.bits, self.G)
                vc, vs, vz = kivi.quantize_v(v[b, h], self.v_bits, self.Gc)
                self.k_codes[b, h, t0:t0 + T] = kivi.pack_k(kc, self.bits)
                self.k_scale[b, h, g0:g0 + T // self.G] = ks
                self.k_zero[b, h, g0:g0 + T // self.G] = kz
                self.v_codes[b, h, t0 // VT:(t0 + T) // VT] = kivi.pack_v(vc, self.v_bits, VT)
                self.v_scale[b, h, t0:t0 + T] = vs
                self.v_zero[b, h, t0:t0 + T] = vz

    def prefill(self, k, v):
        k = np.asarray(k, np.float16)
        v = np.asarray(v, np.float16)
        S = k.shape[2]
        assert self.n_tokens == 0 and 1 <= S <= self.C
        nq, nr = kivi.prefill_split(S, self.G, self.R)
        if nq:
            self._quantize_groups(k[:, :, :nq], v[:, :, :nq], 0)
        self.k_resid[:, :, :nr] = k[:, :, nq:]
        self.v_resid[:, :, :nr] = v[:, :, nq:]
        self.n_quant, self.n_resid = nq, nr

    def append(self, k1, v1):
        """k1, v1: fp16 [B, H, D]."""
        assert self.n_tokens < self.C
        self.n_appends += 1
        if self.n_resid == self.Rcap:
            self._quantize_groups(self.k_resid, self.v_resid, self.n_quant)
            self.n_quant += self.Rcap
            self.n_resid = 0
            self.flush_steps.append(self.n_appends)
        self.k_resid[:, :, self.n_resid] = np.asarray(k1, np.float16)
        self.v_resid[:, :, self.n_resid] = np.asarray(v1, np.float16)
        self.n_resid += 1

    def dequantized(self):
        """K̂, V̂ fp32 [B, H, n_tokens, D]: grouped region dequantized from the
        packed buffers, then the fp16 window."""
        nq, ng = self.n_quant, self.n_quant // self.G
        Kh = np.empty((self.B, self.H, self.n_tokens, self.D), np.float32)
        Vh = np.empty_like(Kh)
        for b in range(self.B):
            for h in range(self.H):
                kc = kivi.unpack_k(self.k_codes[b, h, :nq], self.bits, self.D)
                vc = kivi.unpack_v(self.v_codes[b, h, :nq // VT], self.v_bits, VT)
                Kh[b, h, :nq] = kivi.dequantize_k(kc, self.k_scale[b, h, :ng],
                                                  self.k_zero[b, h, :ng], self.G)
                Vh[b, h, :nq] = kivi.dequantize_v(vc, self.v_scale[b, h, :nq],
                                                  self.v_zero[b, h, :nq])
        Kh[:, :, nq:] = self.k_resid[:, :, :self.n_resid].astype(np.float32)
        Vh[:, :, nq:] = self.v_resid[:, :, :self.n_resid].astype(np.float32)
        return Kh, Vh

    def attention(self, q):
        Kh, Vh = self.dequantized()
        return attention.decode_attention(q, Kh, Vh)


class RaggedKiviCache:
    """A ragged batch: B sequences of their own lengths sharing one cache
    layout. Reading (the pages state KIVI per sequence and never mix
    sequences): each sequence is quantized, flushed and attended exactly as a
    batch of one holding only its own tokens — its groups start at its token
    0 and its window holds its own newest tokens — so sequence b of the
    ragged cache is KiviCache(1, ...) run on that sequence alone. The arrays
    below are those per-sequence caches stacked along the batch axis, the
    layout of the device buffers."""

    def __init__(self, batch, num_kv_heads, head_dim, bits, group, residual, capacity,
                 v_bits=None, v_group_channels=None):
        self.B = batch
        self.seqs = [KiviCache(1, num_kv_heads, head_dim, bits, group, residual, capacity,
                               v_bits=v_bits, v_group_channels=v_group_channels)
                     for _ in range(batch)]

    @property
    def seq_n_quant(self):
        return [c.n_quant for c in self.seqs]

    @property
    def seq_n_resid(self):
        return [c.n_resid for c in self.seqs]

    def prefill(self, k, v, seq_lens):
        """k, v: fp16 [B, H, max_len, D]; sequence b is its first seq_lens[b]
        tokens (the rest is padding, never read)."""
        for b, c in enumerate(self.seqs):
            S = int(seq_lens[b])
            c.prefill(k[b:b + 1, :, :S], v[b:b + 1, :, :S])

    def append(self, k1, v1):
        """k1, v1: fp16 [B, H, D], one token per sequence."""
        for b, c in enumerate(self.seqs):
            c.append(k1[b:b + 1], v1[b:b + 1])

    def array(self, name):
        return np.concatenate([getattr(c, name) for c in self.seqs], axis=0)

    def attention(self, q):
        """q: fp32 [B, Hq, D] → fp64 [B, Hq, D], each row over its own sequence."""
        return np.concatenate([c.attention(q[b:b + 1]) for b, c in enumerate(self.seqs)], axis=0)


TILE = 32   # tokens per V tile of the FP8 / FP16 layouts


def tile_rows(x, n_tiles):
    """[..., T_tokens, D] token rows → [..., n_tiles, D, TILE] tiles (zero
    padded): element (t, d) goes to tile t // TILE, row d, column t % TILE."""
    x = np.asarray(x)
    t = x.shape[-2]
    pad = np.zeros(x.shape[:-2] + (n_tiles * TILE - t, x.shape[-1]), x.dtype)
    y = np.concatenate([x, pad], axis=-2)
    y = y.reshape(x.shape[:-2] + (n_tiles, TILE, x.shape[-1]))
    return np.swapaxes(y, -1, -2).copy()


def untile_rows(y, n_tokens):
    """Inverse of tile_rows for the first n_tokens tokens."""
    x = np.swapaxes(np.asarray(y), -1, -2)
    x = x.reshape(y.shape[:-3] + (y.shape[-3] * TILE, y.shape[-2]))
    return x[..., :n_tokens, :]


class Fp8Cache:
    """FP8 cache: codes of the format `fmt` ("e4m3" or "e5m2"), one K and one V
    scale per tensor, or per KV head when per_head ([Tutorial] §十八.6);
    tensor_scale is [2] = (s_K, s_V) or [H, 2]. Scales are measured at
    prefill and then frozen: appended tokens reuse them ([KIVI-page] §6.2)."""

    def __init__(self, batch, num_kv_heads, head_dim, capacity, fmt="e4m3", per_head=False):
        self.B, self.H, self.D, self.C = batch, num_kv_heads, head_dim, capacity
        self.fmt, self.per_head = fmt, per_head
        self.NT = -(-capacity // TILE)
        self.k_codes = np.zeros((batch, num_kv_heads, self.NT * TILE, head_dim), np.uint8)
        self.v_codes = np.zeros((batch, num_kv_heads, self.NT, head_dim, TILE), np.uint8)
        self.tensor_scale = np.zeros((num_kv_heads, 2) if per_head else 2, np.float32)
        self.n_quant = 0
        self.n_resid = 0

    @property
    def n_tokens(self):
        return self.n_quant

    def _scales(self, which):
        """Scale of each KV head, [H] (the one tensor scale repeated if per tensor)."""
        ts = self.tensor_scale
        return ts[:, which] if self.per_head else np.full(self.H, ts[which], np.float32)

    def _quantize(self, x, which):
        """x: [B, H, ...] fp16 → codes, head h with its own scale."""
        s = self._scales(which)
        return np.stack([fp8.quantize(x[:, h], s[h], self.fmt) for h in range(self.H)], axis=1)

    def _dequantize(self, codes, which):
        s = self._scales(which)
        return np.stack([fp8.dequantize(codes[:, h], s[h], self.fmt) for h in range(self.H)],
                        axis=1)

    def prefill(self, k, v):
        k = np.asarray(k, np.float16)
        v = np.asarray(v, np.float16)
        S = k.shape[2]
        assert self.n_quant == 0 and 1 <= S <= self.C
        if self.per_head:
            self.tensor_scale[:, 0] = fp8.head_scales(k, self.fmt)
            self.tensor_scale[:, 1] = fp8.head_scales(v, self.fmt)
        else:
            self.tensor_scale[:] = (fp8.tensor_scale(k, self.fmt), fp8.tensor_scale(v, self.fmt))
        self.k_codes[:, :, :S] = self._quantize(k, 0)
        self.v_codes[:] = tile_rows(self._quantize(v, 1), self.NT)
        self.n_quant = S

    def append(self, k1, v1):
        assert 0 < self.n_quant < self.C
        t = self.n_quant
        self.k_codes[:, :, t] = self._quantize(np.asarray(k1, np.float16), 0)
        self.v_codes[:, :, t // TILE, :, t % TILE] = self._quantize(np.asarray(v1, np.float16), 1)
        self.n_quant += 1

    def dequantized(self):
        n = self.n_quant
        return (self._dequantize(self.k_codes[:, :, :n], 0),
                self._dequantize(untile_rows(self.v_codes, n), 1))

    def attention(self, q, fp8_query=False):
        """Decode attention over the dequantized cache; fp8_query: the query
        itself goes through per-head E4M3 quantization first (attention in the
        FP8 domain, [Tutorial] §十八.7)."""
        Kh, Vh = self.dequantized()
        if fp8_query:
            q = fp8.dequantize_query(*fp8.quantize_query(q))
        return attention.decode_attention(q, Kh, Vh)


class Fp16Cache:
    def __init__(self, batch, num_kv_heads, head_dim, capacity):
        self.B, self.H, self.D, self.C = batch, num_kv_heads, head_dim, capacity
        self.NT = -(-capacity // TILE)
        self.k = np.zeros((batch, num_kv_heads, self.NT * TILE, head_dim), np.float16)
        self.v = np.zeros((batch, num_kv_heads, self.NT, head_dim, TILE), np.float16)
        self.n_quant = 0
        self.n_resid = 0

    @property
    def n_tokens(self):
        return self.n_quant

    def prefill(self, k, v):
        S = k.shape[2]
        assert self.n_quant == 0 and 1 <= S <= self.C
        self.k[:, :, :S] = k
        self.v[:] = tile_rows(np.asarray(v, np.float16), self.NT)
        self.n_quant = S

    def append(self, k1, v1):
        assert self.n_quant < self.C
        t = self.n_quant
        self.k[:, :, t] = k1
        self.v[:, :, t // TILE, :, t % TILE] = v1
        self.n_quant += 1

    def dequantized(self):
        n = self.n_quant
        return (self.k[:, :, :n].astype(np.float32),
                untile_rows(self.v, n).astype(np.float32))

    def attention(self, q):
        Kh, Vh = self.dequantized()
        return attention.decode_attention(q, Kh, Vh)


class PagedKiviCache:
    """A ragged KIVI batch whose grouped region lives in a pool of pages
    ([Tutorial] §十三.1: paged attention maps each sequence's logical token
    blocks onto discrete physical blocks, and quantization and paging
    compose).

    Reading (the pages give no page layout): a page holds P consecutive
    tokens of every KV head of one sequence — P a power of two, a multiple of
    the group size G and of the 32-token V tile, so pages hold whole groups —
    laid out as one sequence's contiguous buffers restricted to those tokens:
      k_codes [NP][H][P][D·b/32],  v_codes [NP][H][P/32][D][32·b_V/32],
      k_scale, k_zero [NP][H][P/G][D],  v_scale, v_zero [NP][H][P] (or
      [NP][H][P][D/Gc] with V channel sub-groups).
    Logical page j of sequence b (its tokens [jP, jP + P)) is physical page
    table[b][j]. Only the grouped region is paged; the FP16 window stays per
    sequence (k_resid, v_resid [B][H][Rcap][D]). Quantization, flushes and
    attention are those of the ragged cache (each sequence alone, as a batch
    of one): paging changes where the grouped data sits, not what it is.
    Pages that no sequence has written stay zero."""

    def __init__(self, batch, num_kv_heads, head_dim, bits, group, residual, capacity,
                 page_tokens, num_pages, table, v_bits=None, v_group_channels=None):
        P = page_tokens
        assert P >= VT and P & (P - 1) == 0 and P % group == 0
        self.ragged = RaggedKiviCache(batch, num_kv_heads, head_dim, bits, group, residual,
                                      capacity, v_bits=v_bits, v_group_channels=v_group_channels)
        self.B, self.H, self.D, self.G, self.P, self.NP = (batch, num_kv_heads, head_dim, group,
                                                           P, num_pages)
        self.max_pages = -(-capacity // P)
        self.table = np.asarray(table, np.int64)
        assert self.table.shape == (batch, self.max_pages)
        c0 = self.ragged.seqs[0]
        H, D = num_kv_heads, head_dim
        self.k_codes = np.zeros((num_pages, H, P) + c0.k_codes.shape[3:], np.uint32)
        self.v_codes = np.zeros((num_pages, H, P // VT) + c0.v_codes.shape[3:], np.uint32)
        self.k_scale = np.zeros((num_pages, H, P // group, D), np.float32)
        self.k_zero = np.zeros_like(self.k_scale)
        self.v_scale = np.zeros((num_pages, H, P) + c0.v_scale.shape[3:], np.float32)
        self.v_zero = np.zeros_like(self.v_scale)

    @property
    def seq_n_quant(self):
        return self.ragged.seq_n_quant

    @property
    def seq_n_resid(self):
        return self.ragged.seq_n_resid

    def _store(self):
        """Writes every sequence's grouped tokens [0, n_quant) into its pages:
        logical page j's tokens go to page table[b][j] at slots t − jP."""
        P, G = self.P, self.G
        for b, c in enumerate(self.ragged.seqs):
            for j in range(-(-c.n_quant // P)):
                p = self.table[b, j]
                t0, t1 = j * P, min(c.n_quant, j * P + P)
                n = t1 - t0
                self.k_codes[p, :, :n] = c.k_codes[0, :, t0:t1]
                self.v_codes[p, :, :n // VT] = c.v_codes[0, :, t0 // VT:t1 // VT]
                self.k_scale[p, :, :n // G] = c.k_scale[0, :, t0 // G:t1 // G]
                self.k_zero[p, :, :n // G] = c.k_zero[0, :, t0 // G:t1 // G]
                self.v_scale[p, :, :n] = c.v_scale[0, :, t0:t1]
                self.v_zero[p, :, :n] = c.v_zero[0, :, t0:t1]

    def prefill(self, k, v, seq_lens):
        self.ragged.prefill(k, v, seq_lens)
        self._store()

    def append(self, k1, v1):
        self.ragged.append(k1, v1)
        self._store()

    def window(self, name):
        """k_resid or v_resid of the whole batch, [B][H][Rcap][D]."""
        return self.ragged.array(name)

    def dequantized_seq(self, b):
        """Sequence b's K̂, V̂ [1, H, n, D] read back from the pool through
        its block table, then its FP16 window."""
        c = self.ragged.seqs[b]
        P, G, nq = self.P, self.G, c.n_quant
        pages = [self.table[b, j] for j in range(-(-nq // P))]
        ntok = [min(P, nq - j * P) for j in range(len(pages))]
        Kh = np.empty((1, self.H, nq + c.n_resid, self.D), np.float32)
        Vh = np.empty_like(Kh)
        for h in range(self.H):
            if nq:
                kc = np.concatenate([self.k_codes[p, h, :n] for p, n in zip(pages, ntok)])
                vc = np.concatenate([self.v_codes[p, h, :n // VT] for p, n in zip(pages, ntok)])
                ks = np.concatenate([self.k_scale[p, h, :n // G] for p, n in zip(pages, ntok)])
                kz = np.concatenate([self.k_zero[p, h, :n // G] for p, n in zip(pages, ntok)])
                vs = np.concatenate([self.v_scale[p, h, :n] for p, n in zip(pages, ntok)])
                vz = np.concatenate([self.v_zero[p, h, :n] for p, n in zip(pages, ntok)])
                Kh[0, h, :nq] = kivi.dequantize_k(kivi.unpack_k(kc, c.bits, self.D), ks, kz, G)
                Vh[0, h, :nq] = kivi.dequantize_v(kivi.unpack_v(vc, c.v_bits, VT), vs, vz)
        Kh[0, :, nq:] = c.k_resid[0, :, :c.n_resid].astype(np.float32)
        Vh[0, :, nq:] = c.v_resid[0, :, :c.n_resid].astype(np.float32)
        return Kh, Vh

    def attention(self, q):
        """q: fp32 [B, Hq, D] → fp64 [B, Hq, D], each row over its own
        sequence as read from the pool."""
        out = []
        for b in range(self.B):
            Kh, Vh = self.dequantized_seq(b)
            out.append(attention.decode_attention(q[b:b + 1], Kh, Vh))
        return np.concatenate(out, axis=0)
