"""One decode over several attention layers (kvq_decode_attention_layers)
against one decode per layer and against the oracle. The layers differ the
way a model's may (the KV Cache quantization page's mixed-layer byte formula,
§四.4; the KIVI page's sensitive layers kept unquantized, §7.1): KIVI 2-bit,
a layer kept at FP16, a shorter KIVI 4-bit layer with its own KV-head count and
window, a ragged KIVI layer and an FP8 layer. Bar: bitwise equal to the
single-layer decodes (every layer is deterministic), within 2e-3 of the
oracle; a failing layer leaves the output untouched (nothing enqueued).
"""
import sys

import numpy as np
import pytest
import torch

import synth
from oracle import cache as ocache

pytestmark = pytest.mark.gpu

ATOL = 2e-3
D = 128
B, HQ = 2, 8


@pytest.fixture(scope="module")
def kq():
    assert torch.cuda.is_available(), "GPU tests need a ROCm device"
    import kv_cache_quantization_quant_amd as m
    return m


def _np(t):
    return t.detach().cpu().numpy()


# (format, bits, KV heads, tokens, capacity, window R, ragged lengths)
LAYERS = [("kivi", 2, 2, 3000, 3000, 128, None),
          ("fp16", None, 2, 3000, 3000, 0, None),
          ("kivi", 4, 4, 700, 704, 64, None),
          ("kivi", 2, 1, 2500, 2500, 128, [2500, 1100]),
          ("fp8", None, 1, 2000, 2000, 0, None)]


def _build(kq):
    caches, oracles = [], []
    for fmt, bits, H, S, C, R, lens in LAYERS:
        k = synth.make_k(B, H, 0, S, D, device="cuda")
        v = synth.make_v(B, H, 0, S, D, device="cuda")
        cfg = kq.make_config(fmt, bits=bits, batch=B, num_kv_heads=H, capacity=C,
                             residual_length=R if fmt == "kivi" else 128, deterministic=1)
        dc = kq.DeviceCache(cfg, ragged=lens is not None)
        if lens is not None:
            dc.prefill_ragged(k, v, lens)
            oc = ocache.RaggedKiviCache(B, H, D, bits, 32, R, C)
            oc.prefill(_np(k), _np(v), lens)
        else:
            dc.prefill(k, v)
            if fmt == "kivi":
                oc = ocache.KiviCache(B, H, D, bits, 32, R, C)
            elif fmt == "fp8":
                oc = ocache.Fp8Cache(B, H, D, C, fmt="e4m3")
            else:
                oc = ocache.Fp16Cache(B, H, D, C)
            oc.prefill(_np(k), _np(v))
        caches.append(dc)
        oracles.append(oc)
    return caches, oracles


def test_layers_match_single_layer_decodes_and_oracle(kq):
    print("[layers] mixed KIVI / FP16 / FP8 / ragged layers", file=sys.stderr, flush=True)
    caches, oracles = _build(kq)
    L = len(caches)
    q = synth.make_q(L * B, HQ, D, device="cuda").view(L, B, HQ, D)
    out = kq.decode_layers(caches, q)
    torch.cuda.synchronize()
    for l, (dc, oc) in enumerate(zip(caches, oracles)):
        single = dc.decode(q[l].contiguous())
        torch.cuda.synchronize()
        assert torch.equal(out[l], single), l
        err = float(np.max(np.abs(_np(out[l]).astype(np.float64) - oc.attention(_np(q[l])))))
        print(f"  layer {l} ({LAYERS[l][0]}): max abs err {err:.3e}", file=sys.stderr, flush=True)
        assert err <= ATOL, l


def test_failing_layer_enqueues_nothing(kq):
    caches, _ = _build(kq)
    empty = kq.DeviceCache(kq.make_config("kivi", batch=B, num_kv_heads=2, capacity=256))
    q = synth.make_q(3 * B, HQ, D, device="cuda").view(3, B, HQ, D)
    out = torch.full_like(q, float("nan"))
    with pytest.raises(kq.KvqError) as e:
        kq.decode_layers([caches[0], caches[1], empty], q, out=out)
    assert e.value.status == kq.KVQ_ERR_STATE
    torch.cuda.synchronize()
    assert torch.isnan(out).all()
    # a workspace that fits the short 4-bit layer (first) but not the 3000-token
    # layer after it
    small = caches[2].make_workspace(HQ)
    assert caches[0].workspace_bytes(HQ) > small.numel()
    q2 = q[:2].contiguous()
    out2 = torch.full_like(q2, float("nan"))
    with pytest.raises(kq.KvqError) as e:
        kq.decode_layers([caches[2], caches[0]], q2, out=out2, workspace=small)
    assert e.value.status == kq.KVQ_ERR_WORKSPACE
    torch.cuda.synchronize()
    assert torch.isnan(out2).all()
