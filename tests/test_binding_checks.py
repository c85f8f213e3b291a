"""The Python binding checks every tensor before its pointer reaches the C
ABI (the library takes bare pointers and sizes, so a tensor of the wrong
shape, dtype or device would let a kernel read or write outside it). Runs on
the CPU: each call below must raise before any library call."""
import pytest
import torch

import kv_cache_quantization_quant_amd as kq

B, H, HQ, D, C = 2, 4, 8, 128, 300


@pytest.fixture
def no_calls(monkeypatch):
    """Every library call that takes a tensor pointer fails the test."""
    def boom(*a, **k):
        raise AssertionError("a C entry point was reached")
    for name in ("kvq_prefill_quantize", "kvq_prefill_quantize_ragged", "kvq_append_token",
                 "kvq_decode_attention", "kvq_decode_attention_layers",
                 "kvq_quantize_query_fp8", "kvq_append_decode", "kvq_decode_attention_static"):
        monkeypatch.setattr(kq, name, boom)


def _cache(ragged=False):
    # buffers on the host: the checks must refuse them for every call
    return kq.DeviceCache(kq.make_config("kivi", batch=B, num_kv_heads=H, capacity=C),
                          device="cpu", ragged=ragged)


def _t(shape, dtype):
    return torch.zeros(shape, dtype=dtype)


@pytest.mark.parametrize("shape,dtype,what", [
    ((B, H, 10, D), torch.float32, "dtype"),
    ((B + 1, H, 10, D), torch.float16, "shape"),
    ((B, H - 1, 10, D), torch.float16, "shape"),
    ((B, H, 10, 64), torch.float16, "shape"),
    ((B, H, 10), torch.float16, "shape"),
    ((B, H, 10, D), torch.float16, "GPU tensor"),
])
def test_prefill_checks(no_calls, shape, dtype, what):
    dc = _cache()
    with pytest.raises(ValueError, match=what):
        dc.prefill(_t(shape, dtype), _t(shape, dtype))


def test_prefill_v_mismatch(no_calls):
    dc = _cache()
    with pytest.raises(ValueError, match="v: shape"):
        dc.prefill(_t((B, H, 10, D), torch.float16), _t((B, H, 11, D), torch.float16))


def test_prefill_noncontiguous(no_calls):
    dc = _cache()
    k = _t((B, H, D, 10), torch.float16).transpose(2, 3)
    with pytest.raises(ValueError, match="contiguous"):
        dc.prefill(k, k)


def test_prefill_ragged_checks(no_calls):
    dc = _cache(ragged=True)
    k = _t((B, H, 64, D), torch.float16)
    with pytest.raises(ValueError, match="seq_lens"):
        dc.prefill_ragged(k, k, [64] * (B - 1))     # the host would read past it
    with pytest.raises(ValueError, match="v: shape"):
        dc.prefill_ragged(k, _t((B, H, 65, D), torch.float16), [64] * B)
    with pytest.raises(ValueError, match="shape"):
        dc.prefill_ragged(_t((B, H, 64, 64), torch.float16), _t((B, H, 64, 64), torch.float16),
                          [64] * B)
    with pytest.raises(ValueError, match="GPU tensor"):
        dc.prefill_ragged(k, k, [64] * B)
    with pytest.raises(ValueError, match="ragged=True"):
        _cache().prefill_ragged(k, k, [64] * B)


@pytest.mark.parametrize("shape,dtype", [
    ((B, H, D), torch.float32), ((B, H + 1, D), torch.float16), ((B * H, D), torch.float16),
    ((B, H, D), torch.float16)])
def test_append_checks(no_calls, shape, dtype):
    dc = _cache()
    with pytest.raises(ValueError):
        dc.append(_t(shape, dtype), _t(shape, dtype))


@pytest.mark.parametrize("shape,dtype", [
    ((B, HQ, D), torch.float16), ((B + 1, HQ, D), torch.float32), ((B, HQ, 64), torch.float32),
    ((B, HQ), torch.float32), ((B, HQ, D), torch.float32)])
def test_decode_checks(no_calls, shape, dtype):
    dc = _cache()
    with pytest.raises(ValueError):
        dc.decode(_t(shape, dtype), out=_t((B, HQ, D), torch.float32),
                  workspace=_t((1 << 20,), torch.uint8))


def test_decode_out_and_workspace_checks(no_calls):
    dc = _cache()
    ok = _t((B, HQ, D), torch.float32)
    for out in (_t((B, HQ, D - 1), torch.float32), _t((B, HQ, D), torch.float16),
                _t((B, D, HQ), torch.float32).transpose(1, 2)):
        with pytest.raises(ValueError, match="out|q"):
            dc.decode(ok, out=out, workspace=_t((1 << 20,), torch.uint8))
    with pytest.raises(ValueError):
        dc.decode(ok, out=ok, workspace=_t((1 << 18,), torch.float32))


def test_append_decode_checks(no_calls):
    """kvq_append_decode takes every check of the append and of the decode."""
    dc = _cache()
    kv_ok = (B, H, D)
    q_ok = _t((B, HQ, D), torch.float32)
    ws = _t((1 << 20,), torch.uint8)
    for kv_shape, kv_dtype in (((B, H, D), torch.float32), ((B, H + 1, D), torch.float16),
                               ((B * H, D), torch.float16), (kv_ok, torch.float16)):
        with pytest.raises(ValueError):
            dc.append_decode(_t(kv_shape, kv_dtype), _t(kv_shape, kv_dtype), q_ok, out=q_ok,
                             workspace=ws)
    for q in (_t((B, HQ, D), torch.float16), _t((B + 1, HQ, D), torch.float32),
              _t((B, HQ), torch.float32), q_ok):
        with pytest.raises(ValueError):
            dc.append_decode(_t(kv_ok, torch.float16), _t(kv_ok, torch.float16), q, out=q_ok,
                             workspace=ws)
    with pytest.raises(ValueError):
        dc.append_decode(_t(kv_ok, torch.float16), _t(kv_ok, torch.float16), q_ok,
                         out=_t((B, HQ, D - 1), torch.float32), workspace=ws)


def test_decode_layers_checks(no_calls):
    caches = [_cache(), _cache()]
    ok = _t((2, B, HQ, D), torch.float32)
    for q in (_t((3, B, HQ, D), torch.float32), _t((2, B + 1, HQ, D), torch.float32),
              _t((2, B, HQ, D), torch.float16), _t((B, HQ, D), torch.float32), ok):
        with pytest.raises(ValueError):
            kq.decode_layers(caches, q, out=ok, workspace=_t((1 << 20,), torch.uint8))
    with pytest.raises(ValueError, match="at least one"):
        kq.decode_layers([], ok)


def test_quantize_query_checks(no_calls):
    for q in (_t((B, HQ, D), torch.float16), _t((B, HQ), torch.float32),
              _t((B, HQ, D), torch.float32)):
        with pytest.raises(ValueError):
            kq.quantize_query_fp8(q)
