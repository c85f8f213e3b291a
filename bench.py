#!/usr/bin/env python
"""Benchmark of the KIVI decode hot path on one MI355X.

Workload (the 70B-style GQA layer at 32K context): B=16, 64 query heads,
8 KV heads, D=128, KIVI 2-bit K and V, G=32, R=128. The 32768-token prefill is
quantized once before timing; a step is one streamed decode step of one layer:
append one token per (b, KV head) — with the lazy window flush when due, every
128 appends — then decode attention of one query per head over the whole
cache. The steps cycle through LAYERS independent layer caches of that shape,
as consecutive layers of a model do, so that no step finds its cache in the
256 MB Infinity Cache. Inputs are seeded synthetic tensors (synth), resident
in HBM before timing.

Printed (one JSON line): value = effective KV GB/s of the timed steps
(Σ algorithmic decode bytes / wall time of the timed region, HIP events on the
launch stream); roofline of the dominant kernel (decode attention, events
around each decode launch); the CPU oracle on a bounded sample of the same
workload; extra per-workload figures for the other configurations.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X published HBM3E bandwidth
D = 128
COUNTERS_FILE = os.path.join(ROOT, "profiles", "decode_gqa70b_32k_counters.json")
LAYERS = 4                     # layer caches the timed steps cycle through (4 × 441 MB)


def _log(*a):
    print(*a, file=sys.stderr, flush=True)


def decode_source_hash() -> str:
    h = hashlib.sha256()
    for f in ("kvq_decode.hip", "kvq_decode_mfma.hip", "kvq_internal.h", "kvq_fp8.h",
              "kvq_api.cpp"):
        with open(os.path.join(ROOT, "kv_cache_quantization_quant_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def traffic_from_counters():
    """HBM bytes per decode launch from committed rocprofv3 PMC runs, scaled by
    the same counters' reading for a copy of known size; None when absent or
    taken on a different decode kernel source."""
    try:
        with open(COUNTERS_FILE) as f:
            c = json.load(f)
    except (OSError, ValueError):
        return None
    if c.get("decode_source_hash") != decode_source_hash():
        return None
    return c.get("traffic_bytes_per_launch")


class Scrub:
    """A 1 GiB buffer read between timed launches where the Infinity Cache
    (256 MB) must not serve the next launch. Reading (not writing) leaves no
    dirty lines whose write-back would be charged to the next launch."""

    def __init__(self, torch):
        self.buf = torch.ones(1 << 28, dtype=torch.float32, device="cuda")
        self.acc = torch.zeros((), dtype=torch.float32, device="cuda")

    def __call__(self):
        self.acc += self.buf.sum()


def time_launches(torch, fn, iters, scrub=None):
    """Durations (µs) of `fn` launches measured with events on the current stream."""
    out = []
    for _ in range(iters):
        if scrub is not None:
            scrub()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record()
        fn()
        e1.record()
        out.append((e0, e1))
    torch.cuda.synchronize()
    return [a.elapsed_time(b) * 1e3 for a, b in out]


def quantize_traffic_bytes(B, H, S, bits, n_quant, n_resid):
    """Bytes a KIVI prefill must move: read fp16 K and V, write codes, fp32
    scale/zero and the fp16 window."""
    read = 2 * B * H * S * D * 2
    ng = n_quant // 32
    write = B * H * (2 * n_quant * D * bits // 8 + ng * D * 8 + n_quant * 8 + 2 * n_resid * D * 2)
    return read + write


def run_main(torch, kq, synth, args):
    cfg = synth.CONFIGS["gqa70b_32k"]
    B, H, Hq, S, bits = (cfg["batch"], cfg["num_kv_heads"], cfg["num_q_heads"],
                         cfg["seq_len"], cfg["bits"])
    n_steps = args.warmup + args.steps
    C = S + -(-n_steps // LAYERS)
    _log(f"[bench] gqa70b_32k: B={B} Hq={Hq} H={H} S={S} KIVI {bits}-bit, "
         f"{LAYERS} layer caches, warmup={args.warmup} steps={args.steps}")
    t0 = time.time()
    k = synth.make_k(B, H, 0, S + n_steps, D, device="cuda")
    v = synth.make_v(B, H, 0, S + n_steps, D, device="cuda")
    kp, vp = k[:, :, :S].contiguous(), v[:, :, :S].contiguous()
    k_new = [k[:, :, S + i].contiguous() for i in range(n_steps)]
    v_new = [v[:, :, S + i].contiguous() for i in range(n_steps)]
    qs = [synth.make_q(B, Hq, D, step=i, device="cuda") for i in range(n_steps)]
    del k, v
    torch.cuda.synchronize()
    _log(f"[bench] inputs generated in {time.time() - t0:.1f}s")

    cfg_c = kq.make_config("kivi", bits=bits, batch=B, num_kv_heads=H, capacity=C)
    layers = [kq.DeviceCache(cfg_c) for _ in range(LAYERS)]
    dc = layers[0]
    ws = dc.make_workspace(Hq)
    out = torch.empty_like(qs[0])

    # prefill quantize throughput (reset + prefill, median of 5)
    def prefill():
        dc.reset()
        dc.prefill(kp, vp)
    prefill()
    pre_us = statistics.median(time_launches(torch, prefill, 5))
    q_bytes = quantize_traffic_bytes(B, H, S, bits, dc.n_quant, dc.n_resid)
    for c in layers[1:]:
        c.prefill(kp, vp)
    del kp, vp

    # step i works on layer i % LAYERS; with every layer prefilled to a full
    # window, the first append of each layer flushes 128 tokens into 4 groups
    warm_flush = []
    for i in range(args.warmup):
        c = layers[i % LAYERS]
        flushes = c.n_resid == c.cfg.residual_length
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record()
        c.append(k_new[i], v_new[i])
        e1.record()
        if flushes:
            warm_flush.append((e0, e1))
        c.decode(qs[i], out=out, workspace=ws)
    torch.cuda.synchronize()
    warm_flush_us = [a.elapsed_time(b) * 1e3 for a, b in warm_flush]

    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(args.steps)]
    ev_app = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    flush_step = []
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    step_bytes = []
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    start.record()
    for j in range(args.steps):
        i = args.warmup + j
        c = layers[i % LAYERS]
        flush_step.append(c.n_resid == c.cfg.residual_length)   # this append flushes
        ev_app[j].record()
        c.append(k_new[i], v_new[i])
        step_bytes.append(c.decode_bytes(Hq))
        ev[j][0].record()
        c.decode(qs[i], out=out, workspace=ws)
        ev[j][1].record()
    end.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    total_ms = start.elapsed_time(end)
    dec_us = [a.elapsed_time(b) * 1e3 for a, b in ev]
    app_us = [a.elapsed_time(b[0]) * 1e3 for a, b in zip(ev_app, ev)]
    plain_app = [u for u, f in zip(app_us, flush_step) if not f]
    flush_app = [u for u, f in zip(app_us, flush_step) if f] + warm_flush_us
    total_bytes = sum(step_bytes)
    value = total_bytes / (total_ms * 1e-3) / 1e9
    mean_dec_us = sum(dec_us) / len(dec_us)
    achieved = (total_bytes / len(step_bytes)) / (mean_dec_us * 1e-6) / 1e9

    # decode launches with the Infinity Cache scrubbed before each one
    cold_med = None
    bytes_now = dc.decode_bytes(Hq)
    if not args.no_cold:
        scrub = Scrub(torch)
        cold = time_launches(torch, lambda: dc.decode(qs[-1], out=out, workspace=ws), 20, scrub)
        cold_med = statistics.median(cold)

    res = {
        "B": B, "Hq": Hq, "H": H, "S": S, "bits": bits,
        "total_ms": total_ms, "wall_s": wall, "ms_per_step": total_ms / args.steps,
        "value": value, "mean_decode_us": mean_dec_us,
        "p50_decode_us": statistics.median(dec_us),
        "p95_decode_us": sorted(dec_us)[int(0.95 * (len(dec_us) - 1))],
        "decode_bytes_per_launch": total_bytes / len(step_bytes),
        "achieved_gbs": achieved,
        "cold_decode_us_p50": cold_med,
        "cold_decode_gbs": None if cold_med is None else bytes_now / (cold_med * 1e-6) / 1e9,
        "append_us_p50": statistics.median(plain_app) if plain_app else None,
        "flush_append_us_mean": statistics.mean(flush_app) if flush_app else None,
        "flush_steps": len(flush_app),
        "append_plus_decode_us_mean": statistics.mean(a + d for a, d in zip(app_us, dec_us)),
        "prefill_quantize_us": pre_us,
        "prefill_quantize_gbs": q_bytes / (pre_us * 1e-6) / 1e9,
        "layers": LAYERS,
        "final_state": [[c.n_quant, c.n_resid] for c in layers],
    }
    return res


def run_extra(torch, kq, synth):
    """Decode (Infinity Cache scrubbed) and prefill figures of the other
    workloads, one decode step each."""
    scrub = Scrub(torch)
    out = {}
    # workload, format and the knobs that differ from the workload's defaults
    # (G = 32, the workload's bit width for K and V, per-tensor FP8 scales)
    plan = [dict(name="llama2_7b_layer", fmt="kivi"),
            dict(name="mha_large_batch_4bit", fmt="kivi"),
            dict(name="gqa70b_32k", fmt="kivi", G=64), dict(name="gqa70b_32k", fmt="kivi", G=128),
            dict(name="gqa70b_32k", fmt="kivi", kbits=4, vbits=2),
            dict(name="gqa70b_32k", fmt="kivi", kbits=2, vbits=4),
            dict(name="gqa70b_32k", fmt="kivi", v_group_channels=32),
            # ragged batch: sequence b holds 32768 - 1920·b tokens (32768 .. 3968)
            dict(name="gqa70b_32k", fmt="kivi", ragged=True),
            dict(name="gqa_128k", fmt="fp16"), dict(name="gqa_128k", fmt="fp8"),
            dict(name="gqa_128k", fmt="fp8", per_head=1), dict(name="gqa_128k", fmt="fp8_e5m2"),
            dict(name="gqa_128k", fmt="fp8", fp8_attention=1),
            dict(name="gqa_128k", fmt="kivi")]
    kv_cache = {}
    outs = {}                      # gqa_128k decode outputs, same K/V and q
    for item in plan:
        name, fmt = item["name"], item["fmt"]
        G, kbits, vbits = item.get("G", 32), item.get("kbits"), item.get("vbits")
        per_head = item.get("per_head", 0)
        qf8 = item.get("fp8_attention", 0)
        gc = item.get("v_group_channels", 0)
        c = synth.CONFIGS[name]
        B, H, Hq, S = c["batch"], c["num_kv_heads"], c["num_q_heads"], c["seq_len"]
        if name not in kv_cache:
            kv_cache.clear()
            torch.cuda.empty_cache()
            kv_cache[name] = (synth.make_k(B, H, 0, S, D, device="cuda"),
                              synth.make_v(B, H, 0, S, D, device="cuda"))
        k, v = kv_cache[name]
        bits = (kbits or c["bits"]) if fmt == "kivi" else None
        ragged = item.get("ragged", False)
        lens = [S - 1920 * b for b in range(B)] if ragged else None
        dc = kq.DeviceCache(kq.make_config(fmt, bits=bits, group_size=G, batch=B,
                                           num_kv_heads=H, capacity=S, v_bits=vbits or 0,
                                           scale_per_head=per_head, fp8_attention=qf8,
                                           v_group_channels=gc), ragged=ragged)

        def prefill():
            dc.reset()
            if ragged:
                dc.prefill_ragged(k, v, lens)
            else:
                dc.prefill(k, v)
        prefill()
        pre = statistics.median(time_launches(torch, prefill, 3, scrub))
        q = synth.make_q(B, Hq, D, device="cuda")
        ws = dc.make_workspace(Hq)
        o = torch.empty_like(q)
        dec = statistics.median(time_launches(
            torch, lambda: dc.decode(q, out=o, workspace=ws), 10, scrub))
        key = (f"{name}/{fmt}" + (f"_g{G}" if G != 32 else "") +
               (f"_k{kbits}v{vbits}" if vbits else "") + ("_per_head" if per_head else "") +
               ("_fp8_attention" if qf8 else "") + (f"_vgc{gc}" if gc else "") +
               ("_ragged" if ragged else ""))
        if name == "gqa_128k":
            outs[key.split("/")[1]] = o.double().cpu()
        nbytes = dc.decode_bytes(Hq)
        out[key] = {
            "decode_us": round(dec, 2), "decode_bytes": nbytes,
            "decode_gbs": round(nbytes / (dec * 1e-6) / 1e9, 1),
            "decode_frac_hbm": round(nbytes / (dec * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
            "prefill_us": round(pre, 1)}
        del dc, ws
        _log(f"[bench] extra {key}: {out[key]}")
    kv_cache.clear()
    torch.cuda.empty_cache()
    # one call over four layers of the 32K GQA shape, three KIVI 2-bit and one
    # left unquantized (FP16), as a model with a sensitive layer kept at full
    # precision would hold them; the same K/V in every layer
    c = synth.CONFIGS["gqa70b_32k"]
    B, H, Hq, S = c["batch"], c["num_kv_heads"], c["num_q_heads"], c["seq_len"]
    k = synth.make_k(B, H, 0, S, D, device="cuda")
    v = synth.make_v(B, H, 0, S, D, device="cuda")
    layers = []
    for fmt in ("kivi", "kivi", "fp16", "kivi"):
        lc = kq.DeviceCache(kq.make_config(fmt, bits=2 if fmt == "kivi" else None, batch=B,
                                           num_kv_heads=H, capacity=S))
        lc.prefill(k, v)
        layers.append(lc)
    del k, v
    ql = synth.make_q(len(layers) * B, Hq, D, device="cuda").view(len(layers), B, Hq, D)
    ol = torch.empty_like(ql)
    wsl = max((lc.make_workspace(Hq) for lc in layers), key=lambda t: t.numel())
    dec = statistics.median(time_launches(
        torch, lambda: kq.decode_layers(layers, ql, out=ol, workspace=wsl), 10, scrub))
    nbytes = sum(lc.decode_bytes(Hq) for lc in layers)
    key = "gqa70b_32k/layers_kivi3_fp16_1"
    out[key] = {"decode_us": round(dec, 2), "decode_bytes": nbytes,
                "decode_gbs": round(nbytes / (dec * 1e-6) / 1e9, 1),
                "decode_frac_hbm": round(nbytes / (dec * 1e-6) / 1e9 / HBM_PEAK_GBS, 4)}
    _log(f"[bench] extra {key}: {out[key]}")
    del layers, ql, ol, wsl
    torch.cuda.empty_cache()
    # accuracy side report: FP8 and KIVI attention against FP16 attention
    ref = outs["fp16"]
    acc = {}
    for fmt in ("fp8", "fp8_per_head", "fp8_e5m2", "fp8_fp8_attention", "kivi"):
        d = outs[fmt] - ref
        acc[fmt] = {"max_abs": float(d.abs().max()),
                    "rel_l2": float(d.norm() / ref.norm())}
    out["gqa_128k/accuracy_vs_fp16"] = acc
    _log(f"[bench] gqa_128k accuracy vs fp16: {acc}")
    return out


def _cuda_ok():
    import torch
    return torch.cuda.is_available()


def run_cpu_baseline(synth):
    """The oracle on a bounded sample of the same workload: 8 of the 128
    (b, KV head) blocks, prefill-quantized, then 8 decode steps each
    (append + dequantize + fp64 attention of the block's 8 query heads), on one
    host thread."""
    import numpy as np
    from threadpoolctl import threadpool_limits

    from oracle import bytes_model, cache as ocache

    cfg = synth.CONFIGS["gqa70b_32k"]
    B, H, Hq, S = cfg["batch"], cfg["num_kv_heads"], cfg["num_q_heads"], cfg["seq_len"]
    nq = Hq // H
    blocks = [(b, h) for b in (0, 5, 10, 15) for h in (0, 7)]
    steps = 8
    with threadpool_limits(limits=1):
        dev = "cuda" if _cuda_ok() else "cpu"
        kb = np.stack([synth.make_k(1, H, 0, S + steps, D, device=dev, b0=b)[0, h].cpu().numpy()
                       for b, h in blocks])
        vb = np.stack([synth.make_v(1, H, 0, S + steps, D, device=dev, b0=b)[0, h].cpu().numpy()
                       for b, h in blocks])
        q = synth.make_q(B, Hq, D, step=0).numpy()
        t0 = time.perf_counter()
        oc = ocache.KiviCache(len(blocks), 1, D, 2, 32, 128, S + steps)
        oc.prefill(kb[:, None, :S], vb[:, None, :S])
        t_pre = time.perf_counter() - t0
        nbytes = 0
        t0 = time.perf_counter()
        for i in range(steps):
            oc.append(kb[:, None, S + i], vb[:, None, S + i])
            qs = np.stack([q[b, h * nq:(h + 1) * nq] for b, h in blocks])   # [8 blocks, nq, D]
            Kh, Vh = oc.dequantized()
            from oracle import attention
            for j in range(len(blocks)):
                attention.decode_attention(qs[j:j + 1], Kh[j:j + 1], Vh[j:j + 1])
            nbytes += bytes_model.decode_bytes_kivi(len(blocks), 1, D, 2, 32, oc.n_quant,
                                                    oc.n_resid)
        t_dec = time.perf_counter() - t0
    return {"value": round(nbytes / t_dec / 1e9, 4), "unit": "GB/s", "cores": 1,
            "kind": "oracle",
            "sample": (f"{len(blocks)} of {B * H} (b, KV head) blocks of the 32K GQA layer, "
                       f"{steps} decode steps each (append + dequantize + fp64 attention of "
                       f"{nq} query heads); prefill quantize of those blocks took "
                       f"{t_pre:.2f}s; decode {t_dec:.2f}s"),
            "decode_s_per_block_step": round(t_dec / (steps * len(blocks)), 4)}


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=256)
    ap.add_argument("--warmup", type=int, default=16)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extra", action="store_true")
    ap.add_argument("--no-cold", action="store_true",
                    help="skip the scrubbed single-launch decode timing (profiling runs)")
    ap.add_argument("--copy-probe-mib", type=int, default=0,
                    help="after the run, copy a device buffer of this many MiB (a known-size "
                         "transfer that calibrates rocprofv3 FETCH_SIZE / WRITE_SIZE)")
    args = ap.parse_args()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(json.dumps({"error": "this benchmark measures one GPU only; the path runs on a "
                          "single MI355X and has no multi-GPU mode (--gpus 1)"}))
        sys.exit(2)
    if args.steps < 1 or args.warmup < 0:
        ap.error("--steps must be ≥ 1 and --warmup ≥ 0")

    import torch

    import kv_cache_quantization_quant_amd as kq
    import synth

    assert torch.cuda.is_available(), "bench.py needs a ROCm GPU"
    torch.cuda.set_device(0)
    main_res = run_main(torch, kq, synth, args)
    extra = None if args.no_extra else run_extra(torch, kq, synth)
    cpu = None if args.no_cpu_baseline else run_cpu_baseline(synth)
    if args.copy_probe_mib > 0:
        n = args.copy_probe_mib << 18                      # float32 elements
        src = torch.full((n,), 1.0, device="cuda")
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    traffic = traffic_from_counters()
    achieved = main_res["achieved_gbs"]
    line = {
        "metric": "decode attention effective KV GB/s (% of HBM peak) and µs/step at B×S",
        "value": round(main_res["value"], 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(main_res["ms_per_step"], 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "u2-codes/fp32",
        "data": "synthetic (seeded Threefry: K channel-lognormal with 2 x10 outlier channels "
                "per KV head, V token-lognormal, q N(0,1))",
        "config": {"workload": "gqa70b_32k: 64 query / 8 KV heads, D=128, B=16, S=32768 "
                               "(+ streamed tokens), KIVI 2-bit K per-channel / V per-token, "
                               "G=32, R=128; step = append (+flush every 128) + decode of one "
                               "layer, steps cycling through 4 layer caches",
                   "global_batch": main_res["B"], "seq_len": main_res["S"],
                   "parallelism": "single GPU"},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": traffic,
                     "kernel": "decode attention (split + merge launches)",
                     "bytes_per_launch": int(main_res["decode_bytes_per_launch"]),
                     "mean_launch_us": round(main_res["mean_decode_us"], 3)},
        "cpu_baseline": cpu,
        "details": {k: (round(v, 3) if isinstance(v, float) else v)
                    for k, v in main_res.items()},
        "extra": extra,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
