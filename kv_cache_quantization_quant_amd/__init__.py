"""Python binding of libkvq (KIVI / FP8 KV-cache quantization and decode
attention on MI355X).

Argument marshalling only: every function below forwards to the C ABI of the
same name in include/kvq.h, and every step of the path runs in the HIP
kernels of libkvq.so. torch is used for device memory and streams. Importing
this module fails loudly if libkvq.so has not been built
(`python kv_cache_quantization_quant_amd/build.py`).
"""
from __future__ import annotations

import ctypes
import os
from ctypes import POINTER, byref, c_double, c_int32, c_int64, c_size_t, c_void_p, pointer

import torch

# KVQ_LIB names another build of the same library (e.g. one compiled with
# different tuning macros); by default the in-tree libkvq.so is loaded.
_LIB_PATH = os.environ.get("KVQ_LIB") or os.path.join(os.path.dirname(os.path.abspath(__file__)),
                                                      "libkvq.so")

KVQ_OK = 0
KVQ_ERR_INVALID_ARG = 1
KVQ_ERR_UNSUPPORTED = 2
KVQ_ERR_CAPACITY = 3
KVQ_ERR_STATE = 4
KVQ_ERR_DEVICE = 5
KVQ_ERR_WORKSPACE = 6

ABI_VERSION = 11       # KVQ_ABI_VERSION of include/kvq.h
STATIC_WORKSPACE_BYTES = 32 << 20   # KVQ_STATIC_WORKSPACE_BYTES

KVQ_FMT_FP16 = 0
KVQ_FMT_FP8_E4M3 = 1
KVQ_FMT_KIVI = 2
KVQ_FMT_FP8_E5M2 = 3

FORMATS = {"fp16": KVQ_FMT_FP16, "fp8": KVQ_FMT_FP8_E4M3, "kivi": KVQ_FMT_KIVI,
           "fp8_e5m2": KVQ_FMT_FP8_E5M2}
FP8_FORMATS = (KVQ_FMT_FP8_E4M3, KVQ_FMT_FP8_E5M2)


class KvqConfig(ctypes.Structure):
    _fields_ = [("format", c_int32), ("bits", c_int32), ("group_size", c_int32),
                ("residual_length", c_int32), ("batch", c_int32),
                ("num_kv_heads", c_int32), ("head_dim", c_int32), ("capacity", c_int32),
                ("v_bits", c_int32), ("scale_per_head", c_int32), ("fp8_attention", c_int32),
                ("v_group_channels", c_int32), ("deterministic", c_int32),
                ("page_tokens", c_int32), ("num_pages", c_int32)]


class KvqLayout(ctypes.Structure):
    _fields_ = [(n, c_size_t) for n in ("k_codes", "v_codes", "k_scale", "k_zero", "v_scale",
                                         "v_zero", "k_resid", "v_resid", "tensor_scale")]


class KvqCache(ctypes.Structure):
    _fields_ = [("cfg", KvqConfig),
                ("k_codes", c_void_p), ("v_codes", c_void_p),
                ("k_scale", c_void_p), ("k_zero", c_void_p),
                ("v_scale", c_void_p), ("v_zero", c_void_p),
                ("k_resid", c_void_p), ("v_resid", c_void_p),
                ("tensor_scale", c_void_p),
                ("n_quant", c_int64), ("n_resid", c_int32), ("reserved", c_int32),
                ("seq_n_quant", POINTER(c_int64)), ("seq_n_resid", POINTER(c_int32)),
                ("block_table", c_void_p)]


MAX_RAGGED_BATCH = 128   # KVQ_MAX_RAGGED_BATCH


class KvqError(RuntimeError):
    def __init__(self, status: int, what: str):
        super().__init__(f"{what}: {kvq_status_str(status)} (status {status})")
        self.status = status


def _load():
    if not os.path.exists(_LIB_PATH):
        raise ImportError(f"libkvq.so not found at {_LIB_PATH}; build it with "
                          "`python kv_cache_quantization_quant_amd/build.py`")
    lib = ctypes.CDLL(_LIB_PATH)
    sig = {
        "kvq_abi_version": (c_int32, []),
        "kvq_status_str": (ctypes.c_char_p, [c_int32]),
        "kvq_layout_query": (c_int32, [POINTER(KvqConfig), POINTER(KvqLayout)]),
        "kvq_cache_init": (c_int32, [POINTER(KvqCache), POINTER(KvqConfig)]),
        "kvq_cache_reset": (c_int32, [POINTER(KvqCache)]),
        "kvq_prefill_quantize": (c_int32, [POINTER(KvqCache), c_void_p, c_void_p, c_int64,
                                           c_void_p]),
        "kvq_prefill_quantize_ragged": (c_int32, [POINTER(KvqCache), c_void_p, c_void_p, c_int64,
                                                  POINTER(c_int64), c_void_p]),
        "kvq_append_token": (c_int32, [POINTER(KvqCache), c_void_p, c_void_p, c_void_p]),
        "kvq_decode_workspace_bytes": (c_size_t, [POINTER(KvqConfig), c_int32]),
        "kvq_decode_attention": (c_int32, [POINTER(KvqCache), c_void_p, c_int32, c_void_p,
                                           c_void_p, c_size_t, c_void_p]),
        "kvq_decode_attention_static": (c_int32, [POINTER(KvqCache), c_void_p, c_int32,
                                                  c_void_p, c_void_p]),
        "kvq_append_decode": (c_int32, [POINTER(KvqCache), c_void_p, c_void_p, c_void_p, c_int32,
                                        c_void_p, c_void_p, c_size_t, c_void_p]),
        "kvq_decode_attention_layers": (c_int32, [POINTER(POINTER(KvqCache)), c_int32,
                                                  c_void_p, c_int32, c_void_p, c_void_p,
                                                  c_size_t, c_void_p]),
        "kvq_decode_bytes": (c_int64, [POINTER(KvqCache), c_int32]),
        "kvq_quantize_query_fp8": (c_int32, [c_void_p, c_int32, c_int32, c_int32, c_void_p,
                                             c_void_p, c_void_p]),
        "kvq_theoretical_bytes": (c_double, [c_int32, c_int32, c_int64, c_int32, c_int32,
                                             c_double]),
        "kvq_theoretical_bytes_layers": (c_double, [c_int32, c_int32, POINTER(c_int64),
                                                    POINTER(c_int32), POINTER(c_int32),
                                                    c_double]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    # the structs below must match the library's
    if lib.kvq_abi_version() != ABI_VERSION:
        raise ImportError(f"{_LIB_PATH} has ABI version {lib.kvq_abi_version()}, this binding "
                          f"expects {ABI_VERSION}; rebuild it")
    return lib


lib = _load()
ABI_SYMBOLS = ("kvq_abi_version", "kvq_status_str", "kvq_layout_query", "kvq_cache_init",
               "kvq_cache_reset", "kvq_prefill_quantize", "kvq_prefill_quantize_ragged",
               "kvq_append_token",
               "kvq_decode_workspace_bytes", "kvq_decode_attention", "kvq_decode_bytes",
               "kvq_quantize_query_fp8", "kvq_theoretical_bytes",
               "kvq_decode_attention_layers", "kvq_theoretical_bytes_layers",
               "kvq_decode_attention_static", "kvq_append_decode")


# ------------------------------------------------- one-to-one ABI wrappers ---

def kvq_abi_version() -> int:
    return lib.kvq_abi_version()


def kvq_status_str(status: int) -> str:
    return lib.kvq_status_str(status).decode()


def kvq_layout_query(cfg: KvqConfig) -> tuple[int, KvqLayout]:
    out = KvqLayout()
    return lib.kvq_layout_query(byref(cfg), byref(out)), out


def kvq_cache_init(cache: KvqCache, cfg: KvqConfig) -> int:
    return lib.kvq_cache_init(byref(cache), byref(cfg))


def kvq_cache_reset(cache: KvqCache) -> int:
    return lib.kvq_cache_reset(byref(cache))


def kvq_prefill_quantize(cache: KvqCache, k_ptr: int, v_ptr: int, seq_len: int,
                         stream: int | None) -> int:
    return lib.kvq_prefill_quantize(byref(cache), k_ptr, v_ptr, seq_len, stream)


def kvq_prefill_quantize_ragged(cache: KvqCache, k_ptr: int, v_ptr: int, max_len: int,
                                seq_lens, stream: int | None) -> int:
    """seq_lens: a ctypes int64 array of `batch` entries (host)."""
    return lib.kvq_prefill_quantize_ragged(byref(cache), k_ptr, v_ptr, max_len, seq_lens, stream)


def kvq_append_token(cache: KvqCache, k_ptr: int, v_ptr: int, stream: int | None) -> int:
    return lib.kvq_append_token(byref(cache), k_ptr, v_ptr, stream)


def kvq_decode_workspace_bytes(cfg: KvqConfig, num_q_heads: int) -> int:
    return lib.kvq_decode_workspace_bytes(byref(cfg), num_q_heads)


def kvq_decode_attention(cache: KvqCache, q_ptr: int, num_q_heads: int, out_ptr: int,
                         ws_ptr: int, ws_bytes: int, stream: int | None) -> int:
    return lib.kvq_decode_attention(byref(cache), q_ptr, num_q_heads, out_ptr, ws_ptr,
                                    ws_bytes, stream)


def kvq_append_decode(cache: KvqCache, k_ptr: int, v_ptr: int, q_ptr: int, num_q_heads: int,
                      out_ptr: int, ws_ptr: int, ws_bytes: int, stream: int | None) -> int:
    return lib.kvq_append_decode(byref(cache), k_ptr, v_ptr, q_ptr, num_q_heads, out_ptr, ws_ptr,
                                 ws_bytes, stream)


def kvq_decode_attention_static(cache: KvqCache, q_ptr: int, num_q_heads: int, out_ptr: int,
                                stream: int | None) -> int:
    return lib.kvq_decode_attention_static(byref(cache), q_ptr, num_q_heads, out_ptr, stream)


def kvq_decode_attention_layers(caches, q_ptr: int, num_q_heads: int, out_ptr: int,
                                ws_ptr: int, ws_bytes: int, stream: int | None) -> int:
    """caches: a sequence of KvqCache (None entries pass a null pointer)."""
    arr = (POINTER(KvqCache) * max(1, len(caches)))()
    for i, c in enumerate(caches):
        arr[i] = pointer(c) if c is not None else POINTER(KvqCache)()
    return lib.kvq_decode_attention_layers(arr, len(caches), q_ptr, num_q_heads, out_ptr,
                                           ws_ptr, ws_bytes, stream)


def kvq_decode_bytes(cache: KvqCache, num_q_heads: int) -> int:
    return lib.kvq_decode_bytes(byref(cache), num_q_heads)


def kvq_quantize_query_fp8(q_ptr: int, batch: int, num_q_heads: int, head_dim: int,
                           codes_ptr: int, scales_ptr: int, stream: int | None) -> int:
    return lib.kvq_quantize_query_fp8(q_ptr, batch, num_q_heads, head_dim, codes_ptr,
                                      scales_ptr, stream)


def kvq_theoretical_bytes(num_layers, batch, seq_len, num_kv_heads, head_dim,
                          bytes_per_elem) -> float:
    return lib.kvq_theoretical_bytes(num_layers, batch, seq_len, num_kv_heads, head_dim,
                                     bytes_per_elem)


def kvq_theoretical_bytes_layers(batch, seq_lens, num_kv_heads, head_dims,
                                 bytes_per_elem) -> float:
    n = len(seq_lens)
    if not (len(num_kv_heads) == len(head_dims) == n):
        raise ValueError("one seq_len, num_kv_heads and head_dim per layer")
    return lib.kvq_theoretical_bytes_layers(n, batch, (c_int64 * max(1, n))(*seq_lens),
                                            (c_int32 * max(1, n))(*num_kv_heads),
                                            (c_int32 * max(1, n))(*head_dims), bytes_per_elem)


def decode_layers(caches, q: torch.Tensor, out: torch.Tensor | None = None,
                  workspace: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """One decode per layer (kvq_decode_attention_layers). caches: DeviceCache
    per layer; q: contiguous fp32 [L, B, Hq, D] → out fp32 [L, B, Hq, D]."""
    if len(caches) < 1:
        raise ValueError("decode_layers: at least one layer")
    c0 = caches[0]
    if q.dim() != 4:
        raise ValueError(f"q: shape {tuple(q.shape)}, expected [layers, batch, Hq, D]")
    hq = q.shape[2]
    shape = (len(caches), c0.cfg.batch, hq, c0.cfg.head_dim)
    for c in caches:
        if c.cfg.batch != c0.cfg.batch or c.cfg.head_dim != c0.cfg.head_dim:
            raise ValueError("decode_layers: every layer needs the same batch and head_dim")
    _require(q, "q", torch.float32, shape, c0.device)
    if out is None:
        out = torch.empty_like(q)
    _require(out, "out", torch.float32, shape, c0.device)
    if workspace is None:
        n = max(c.workspace_bytes(hq) for c in caches)
        if n == 0:
            raise KvqError(KVQ_ERR_INVALID_ARG, "kvq_decode_workspace_bytes")
        workspace = torch.empty(n, dtype=torch.uint8, device=q.device)
    _require(workspace, "workspace", torch.uint8, (workspace.numel(),), c0.device)
    _check(kvq_decode_attention_layers([c.cache for c in caches], q.data_ptr(), hq,
                                       out.data_ptr(), workspace.data_ptr(), workspace.numel(),
                                       _stream_handle(stream)), "kvq_decode_attention_layers")
    return out


def make_config(fmt: str = "kivi", bits: int | None = None, group_size: int = 32,
                residual_length: int = 128, batch: int = 1, num_kv_heads: int = 1,
                head_dim: int = 128, capacity: int = 256, v_bits: int = 0,
                scale_per_head: int = 0, fp8_attention: int = 0,
                v_group_channels: int = 0, deterministic: int = 0, page_tokens: int = 0,
                num_pages: int = 0) -> KvqConfig:
    """v_bits: KIVI V bit width (0 = same as bits); scale_per_head: FP8 scales
    per KV head (1) or per tensor (0); fp8_attention: FP8 decode with the
    query quantized to E4M3 (1); v_group_channels: KIVI V scales per run of
    32 channels (32) or per token (0); deterministic: KIVI and FP8 decode with
    a fixed tile order per wavefront (1, bitwise reproducible) or tiles shared
    as the wavefronts go (0, fastest); page_tokens, num_pages: KIVI grouped
    region in a pool of num_pages pages of page_tokens tokens (0: contiguous;
    the cache is then ragged and needs a block table)."""
    if bits is None:
        bits = {"kivi": 2, "fp8": 8, "fp8_e5m2": 8, "fp16": 16}[fmt]
    return KvqConfig(FORMATS[fmt], bits, group_size, residual_length, batch, num_kv_heads,
                     head_dim, capacity, v_bits, scale_per_head, fp8_attention,
                     v_group_channels, deterministic, page_tokens, num_pages)


def quantize_query_fp8(q: torch.Tensor, stream=None) -> tuple[torch.Tensor, torch.Tensor]:
    """q: contiguous fp32 [B, Hq, D] on the device → (E4M3 codes uint8
    [B, Hq, D], scales fp32 [B, Hq])."""
    if q.dim() != 3:
        raise ValueError(f"q: shape {tuple(q.shape)}, expected [batch, Hq, D]")
    B, Hq, D = q.shape
    _require(q, "q", torch.float32, (B, Hq, D))
    codes = torch.empty(q.shape, dtype=torch.uint8, device=q.device)
    scales = torch.empty((B, Hq), dtype=torch.float32, device=q.device)
    _check(kvq_quantize_query_fp8(q.data_ptr(), B, Hq, D, codes.data_ptr(), scales.data_ptr(),
                                  _stream_handle(stream)), "kvq_quantize_query_fp8")
    return codes, scales


def _check(status: int, what: str):
    if status != KVQ_OK:
        raise KvqError(status, what)


def _require(t, name: str, dtype: torch.dtype, shape, device: torch.device | None = None):
    """Raises ValueError unless t is a contiguous device tensor of this dtype
    and shape (and on `device`, when given). The C ABI takes bare pointers, so
    a tensor of the wrong shape would let the kernels read or write outside
    it: every tensor is checked here, before its pointer goes to the library."""
    if not isinstance(t, torch.Tensor):
        raise ValueError(f"{name}: expected a torch.Tensor, got {type(t).__name__}")
    if t.dtype != dtype:
        raise ValueError(f"{name}: dtype {t.dtype}, expected {dtype}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name}: shape {tuple(t.shape)}, expected {tuple(shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name}: must be contiguous")
    if t.device.type != "cuda":
        raise ValueError(f"{name}: must be a GPU tensor, got device {t.device}")
    if device is not None and t.device != device:
        raise ValueError(f"{name}: on {t.device}, the cache is on {device}")


_raw_stream = getattr(torch._C, "_cuda_getCurrentRawStream", None)


def _stream_handle(stream) -> int:
    if stream is not None:
        return stream.cuda_stream
    if _raw_stream is not None:          # the current stream's handle, no Stream object
        return _raw_stream(torch.cuda.current_device())
    return torch.cuda.current_stream().cuda_stream


# ------------------------------------------ torch-owned cache (plumbing) ---

class DeviceCache:
    """A cache whose device buffers are torch tensors (memory plumbing only);
    every operation is a call into libkvq on the given (or current) stream."""

    _BUFFERS = ("k_codes", "v_codes", "k_scale", "k_zero", "v_scale", "v_zero",
                "k_resid", "v_resid", "tensor_scale")

    def __init__(self, cfg: KvqConfig, device="cuda", ragged: bool = False,
                 block_table: torch.Tensor | None = None):
        """ragged: per-sequence fill levels (KIVI; prefill with prefill_ragged).
        A paged configuration (page_tokens > 0) is ragged and takes its block
        table: int32 [batch, ceil(capacity / page_tokens)] on the device
        (kept here; the caller may update its entries between calls)."""
        self.cfg = cfg
        st, self.layout = kvq_layout_query(cfg)
        _check(st, "kvq_layout_query")
        self.cache = KvqCache()
        _check(kvq_cache_init(self.cache, cfg), "kvq_cache_init")
        self.paged = cfg.format == KVQ_FMT_KIVI and cfg.page_tokens > 0
        if self.paged:
            ragged = True
            if block_table is None:
                raise ValueError("a paged cache needs its block table")
            max_pages = -(-cfg.capacity // cfg.page_tokens)
            if block_table.device.type != "cuda" and torch.device(device).type == "cuda":
                raise ValueError("block_table: must be a GPU tensor")
            if (block_table.dtype != torch.int32 or tuple(block_table.shape) !=
                    (cfg.batch, max_pages) or not block_table.is_contiguous()):
                raise ValueError(f"block_table: contiguous int32 [{cfg.batch}, {max_pages}] "
                                 f"expected, got {block_table.dtype} {tuple(block_table.shape)}")
            self.block_table = block_table
            self.cache.block_table = block_table.data_ptr()
        elif block_table is not None:
            raise ValueError("block_table given for a cache that is not paged")
        self.ragged = ragged
        if ragged:
            # host arrays the library reads and updates (kept alive here)
            self._seq_nq = (c_int64 * cfg.batch)()
            self._seq_nr = (c_int32 * cfg.batch)()
            self.cache.seq_n_quant = ctypes.cast(self._seq_nq, POINTER(c_int64))
            self.cache.seq_n_resid = ctypes.cast(self._seq_nr, POINTER(c_int32))
        self.buffers = {}
        for name in self._BUFFERS:
            nbytes = getattr(self.layout, name)
            if nbytes:
                t = torch.zeros(nbytes, dtype=torch.uint8, device=device)
                self.buffers[name] = t
                setattr(self.cache, name, t.data_ptr())
        # the device every buffer sits on ("cuda" resolved to its index)
        self.device = next(iter(self.buffers.values())).device

    # fill state
    @property
    def n_quant(self) -> int:
        return self.cache.n_quant

    @property
    def n_resid(self) -> int:
        return self.cache.n_resid

    @property
    def seq_n_quant(self) -> list[int]:
        return list(self._seq_nq)

    @property
    def seq_n_resid(self) -> list[int]:
        return list(self._seq_nr)

    def reset(self):
        _check(kvq_cache_reset(self.cache), "kvq_cache_reset")

    def prefill_ragged(self, k: torch.Tensor, v: torch.Tensor, seq_lens, stream=None):
        """k, v: contiguous fp16 [B, H, max_len, D] on the device, sequence b in
        its first seq_lens[b] tokens."""
        if not self.ragged:
            raise ValueError("prefill_ragged needs a cache made with ragged=True")
        c = self.cfg
        if k.dim() != 4:
            raise ValueError(f"k: shape {tuple(k.shape)}, expected [B, H, max_len, D]")
        if len(seq_lens) != c.batch:
            raise ValueError(f"seq_lens: {len(seq_lens)} entries, expected batch = {c.batch}")
        if tuple(v.shape) != tuple(k.shape):
            raise ValueError(f"v: shape {tuple(v.shape)}, k has {tuple(k.shape)}")
        shape = (c.batch, c.num_kv_heads, k.shape[2], c.head_dim)
        _require(k, "k", torch.float16, shape, self.device)
        _require(v, "v", torch.float16, shape, self.device)
        lens = (c_int64 * len(seq_lens))(*[int(x) for x in seq_lens])
        _check(kvq_prefill_quantize_ragged(self.cache, k.data_ptr(), v.data_ptr(), k.shape[2],
                                           lens, _stream_handle(stream)),
               "kvq_prefill_quantize_ragged")

    def prefill(self, k: torch.Tensor, v: torch.Tensor, stream=None):
        """k, v: contiguous fp16 [B, H, S, D] on the device."""
        c = self.cfg
        if k.dim() != 4:
            raise ValueError(f"k: shape {tuple(k.shape)}, expected [B, H, S, D]")
        if tuple(v.shape) != tuple(k.shape):
            raise ValueError(f"v: shape {tuple(v.shape)}, k has {tuple(k.shape)}")
        shape = (c.batch, c.num_kv_heads, k.shape[2], c.head_dim)
        _require(k, "k", torch.float16, shape, self.device)
        _require(v, "v", torch.float16, shape, self.device)
        _check(kvq_prefill_quantize(self.cache, k.data_ptr(), v.data_ptr(), k.shape[2],
                                    _stream_handle(stream)), "kvq_prefill_quantize")

    def append(self, k1: torch.Tensor, v1: torch.Tensor, stream=None):
        """k1, v1: contiguous fp16 [B, H, D] on the device."""
        c = self.cfg
        shape = (c.batch, c.num_kv_heads, c.head_dim)
        _require(k1, "k1", torch.float16, shape, self.device)
        _require(v1, "v1", torch.float16, shape, self.device)
        _check(kvq_append_token(self.cache, k1.data_ptr(), v1.data_ptr(),
                                _stream_handle(stream)), "kvq_append_token")

    def workspace_bytes(self, num_q_heads: int) -> int:
        return kvq_decode_workspace_bytes(self.cfg, num_q_heads)

    def make_workspace(self, num_q_heads: int) -> torch.Tensor:
        n = self.workspace_bytes(num_q_heads)
        if n == 0:
            raise KvqError(KVQ_ERR_INVALID_ARG, "kvq_decode_workspace_bytes")
        return torch.empty(n, dtype=torch.uint8, device=self.device)

    def decode(self, q: torch.Tensor, out: torch.Tensor | None = None,
               workspace: torch.Tensor | None = None, stream=None) -> torch.Tensor:
        """q: contiguous fp32 [B, Hq, D] → out fp32 [B, Hq, D]."""
        c = self.cfg
        if q.dim() != 3:
            raise ValueError(f"q: shape {tuple(q.shape)}, expected [B, Hq, D]")
        hq = q.shape[1]
        shape = (c.batch, hq, c.head_dim)
        _require(q, "q", torch.float32, shape, self.device)
        if out is None:
            out = torch.empty_like(q)
        _require(out, "out", torch.float32, shape, self.device)
        if workspace is None:
            workspace = self.make_workspace(hq)
        _require(workspace, "workspace", torch.uint8, (workspace.numel(),), self.device)
        _check(kvq_decode_attention(self.cache, q.data_ptr(), hq, out.data_ptr(),
                                    workspace.data_ptr(), workspace.numel(),
                                    _stream_handle(stream)), "kvq_decode_attention")
        return out

    def append_decode(self, k1: torch.Tensor, v1: torch.Tensor, q: torch.Tensor,
                      out: torch.Tensor | None = None, workspace: torch.Tensor | None = None,
                      stream=None) -> torch.Tensor:
        """kvq_append_decode: append(k1, v1) then decode(q) as one call.
        k1, v1: contiguous fp16 [B, H, D]; q: contiguous fp32 [B, Hq, D]."""
        c = self.cfg
        kv_shape = (c.batch, c.num_kv_heads, c.head_dim)
        _require(k1, "k1", torch.float16, kv_shape, self.device)
        _require(v1, "v1", torch.float16, kv_shape, self.device)
        if q.dim() != 3:
            raise ValueError(f"q: shape {tuple(q.shape)}, expected [B, Hq, D]")
        hq = q.shape[1]
        shape = (c.batch, hq, c.head_dim)
        _require(q, "q", torch.float32, shape, self.device)
        if out is None:
            out = torch.empty_like(q)
        _require(out, "out", torch.float32, shape, self.device)
        if workspace is None:
            workspace = self.make_workspace(hq)
        _require(workspace, "workspace", torch.uint8, (workspace.numel(),), self.device)
        _check(kvq_append_decode(self.cache, k1.data_ptr(), v1.data_ptr(), q.data_ptr(), hq,
                                 out.data_ptr(), workspace.data_ptr(), workspace.numel(),
                                 _stream_handle(stream)), "kvq_append_decode")
        return out

    def decode_static(self, q: torch.Tensor, out: torch.Tensor, stream=None) -> torch.Tensor:
        """kvq_decode_attention_static: the decode with the library's own
        per-GPU partials array, allocating nothing (out must be given)."""
        c = self.cfg
        if q.dim() != 3:
            raise ValueError(f"q: shape {tuple(q.shape)}, expected [B, Hq, D]")
        shape = (c.batch, q.shape[1], c.head_dim)
        _require(q, "q", torch.float32, shape, self.device)
        _require(out, "out", torch.float32, shape, self.device)
        _check(kvq_decode_attention_static(self.cache, q.data_ptr(), q.shape[1], out.data_ptr(),
                                           _stream_handle(stream)), "kvq_decode_attention_static")
        return out

    def decode_bytes(self, num_q_heads: int) -> int:
        return kvq_decode_bytes(self.cache, num_q_heads)

    # typed views of the device buffers (for tests and inspection)
    def view(self, name: str) -> torch.Tensor:
        c = self.cfg
        B, H, D, G = c.batch, c.num_kv_heads, c.head_dim, c.group_size
        NG = -(-c.capacity // G)
        CT = NG * G
        Rcap = c.residual_length if c.residual_length > 0 else G
        buf = self.buffers[name]
        if c.format == KVQ_FMT_KIVI:
            b = c.bits
            bv = c.v_bits if c.v_bits > 0 else c.bits
            # blocks of token slots: (b, h) of CT slots, or (page, h) of P slots
            NB, T = (c.num_pages, c.page_tokens) if self.paged else (B, CT)
            vsh = (NB, H, T) if c.v_group_channels == 0 else (NB, H, T, D // c.v_group_channels)
            shapes = {"k_codes": (torch.int32, (NB, H, T, D * b // 32)),
                      "v_codes": (torch.int32, (NB, H, T // 32, D, 32 * bv // 32)),
                      "k_scale": (torch.float32, (NB, H, T // G, D)),
                      "k_zero": (torch.float32, (NB, H, T // G, D)),
                      "v_scale": (torch.float32, vsh),
                      "v_zero": (torch.float32, vsh),
                      "k_resid": (torch.float16, (B, H, Rcap, D)),
                      "v_resid": (torch.float16, (B, H, Rcap, D))}
        elif c.format in FP8_FORMATS:
            NT = -(-c.capacity // 32)
            shapes = {"k_codes": (torch.uint8, (B, H, NT * 32, D)),
                      "v_codes": (torch.uint8, (B, H, NT, D, 32)),
                      "tensor_scale": (torch.float32,
                                       (H, 4) if c.scale_per_head else (4,))}
        else:
            NT = -(-c.capacity // 32)
            shapes = {"k_codes": (torch.float16, (B, H, NT * 32, D)),
                      "v_codes": (torch.float16, (B, H, NT, D, 32))}
        dt, shape = shapes[name]
        return buf.view(dt).view(shape)
