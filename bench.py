#!/usr/bin/env python
"""Benchmark of the KIVI decode hot path on one MI355X.

Workload (the 70B-style GQA layer at 32K context): B=16, 64 query heads,
8 KV heads, D=128, KIVI 2-bit K and V, G=32, R=128. The 32768-token prefill is
quantized once before timing; a step is one streamed decode step of one layer:
append one token per (b, KV head) — with the lazy window flush when due, every
128 appends — then decode attention of one query per head over the whole
cache: one kvq_append_decode call in the pass the value is taken from, the two
calls with events around the decode in the roofline pass. The steps cycle through LAYERS independent layer caches of that shape,
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
import gc
import hashlib
import json
import os
import re
import shutil
import statistics
import subprocess
import sys
import threading
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


def _file_hash() -> str:
    with open(os.path.abspath(__file__), "rb") as fh:
        return hashlib.sha256(fh.read()).hexdigest()[:16]


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


def _bytes_at(kq, cache, n_quant, n_resid, hq):
    """kvq_decode_bytes of `cache` at another fill state (a host-side copy of
    its struct; nothing is enqueued)."""
    c = kq.KvqCache.from_buffer_copy(cache)
    c.n_quant, c.n_resid = n_quant, n_resid
    return kq.kvq_decode_bytes(c, hq)


def run_main(torch, kq, synth, args):
    cfg = synth.CONFIGS["gqa70b_32k"]
    B, H, Hq, S, bits = (cfg["batch"], cfg["num_kv_heads"], cfg["num_q_heads"],
                         cfg["seq_len"], cfg["bits"])
    R = cfg["residual_length"]
    # Layer l enters the timed steps with a window of 1 + 32·l tokens (setup
    # appends after the prefill; the first one flushes the full prefill
    # window), so that even a short run decodes over every part of the window
    # cycle and a long one crosses flushes in the timed region.
    stagger = [1 + (R // LAYERS) * l for l in range(LAYERS)]
    # the timed steps run twice: once with events around each decode (the
    # roofline pass), once with only the region's two events (the value)
    per_layer = -(-(args.warmup + 2 * args.steps) // LAYERS)
    n_new = max(stagger) + per_layer
    C = S + n_new
    _log(f"[bench] gqa70b_32k: B={B} Hq={Hq} H={H} S={S} KIVI {bits}-bit, "
         f"{LAYERS} layer caches (windows {stagger}), warmup {args.warmup_s}s + "
         f"{args.warmup} steps, steps={args.steps}")
    t0 = time.time()
    k = synth.make_k(B, H, 0, C, D, device="cuda")
    v = synth.make_v(B, H, 0, C, D, device="cuda")
    kp, vp = k[:, :, :S].contiguous(), v[:, :, :S].contiguous()
    k_new = [k[:, :, S + i].contiguous() for i in range(n_new)]
    v_new = [v[:, :, S + i].contiguous() for i in range(n_new)]
    n_q = args.warmup + 2 * args.steps
    qs = [synth.make_q(B, Hq, D, step=i, device="cuda") for i in range(n_q)]
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

    # setup appends (untimed as steps): the first append of each layer finds
    # the prefill window full and flushes it (timed here on its own), the
    # next ones are plain window writes
    # (each behind a cache scrub, so that the GPU is busy while the host
    # enqueues it and the events time the append's kernels alone)
    pos = [0] * LAYERS                     # next streamed token of each layer
    flush_us, plain_us = [], []
    scrub = Scrub(torch)
    for l, c in enumerate(layers):
        for j in range(stagger[l]):
            flushes = c.n_resid == c.cfg.residual_length
            (flush_us if flushes else plain_us).extend(time_launches(
                torch, lambda: c.append(k_new[pos[l]], v_new[pos[l]]), 1, scrub))
            pos[l] += 1

    # time-based warm-up: decodes cycling through the layers until the clocks
    # have settled under this load, then the requested warm-up steps
    t_w = time.perf_counter()
    n_warm = 0
    while time.perf_counter() - t_w < args.warmup_s:
        for c in layers:
            c.decode(qs[0], out=out, workspace=ws)
        n_warm += LAYERS
        torch.cuda.synchronize()
    qi = 0
    for i in range(args.warmup):
        l = i % LAYERS
        layers[l].append_decode(k_new[pos[l]], v_new[pos[l]], qs[qi], out=out, workspace=ws)
        pos[l] += 1
        qi += 1
    torch.cuda.synchronize()

    def timed(per_decode_events):
        """K steps (append + decode, layer i % LAYERS); returns the region's
        time (us), the fill state each decode saw, the decodes' event times."""
        nonlocal qi
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(args.steps)] if per_decode_events else None
        state = []
        host = []
        start = torch.cuda.Event(enable_timing=True)
        end = torch.cuda.Event(enable_timing=True)
        # no garbage collection pass inside the region (a pass over this
        # process's many tensors and events holds the host for milliseconds)
        gc.collect()
        gc.disable()
        torch.cuda.synchronize()
        wall0 = time.perf_counter()
        start.record()
        for j in range(args.steps):
            host.append(time.perf_counter())
            l = j % LAYERS
            c = layers[l]
            if ev:
                # roofline pass: the append, then events around the decode alone
                c.append(k_new[pos[l]], v_new[pos[l]])
                ev[j][0].record()
                c.decode(qs[qi], out=out, workspace=ws)
                ev[j][1].record()
            else:
                # value pass: the step as one call (one launch unless a flush
                # is due: the decode stores the new token itself)
                c.append_decode(k_new[pos[l]], v_new[pos[l]], qs[qi], out=out, workspace=ws)
            pos[l] += 1
            qi += 1
            state.append((l, c.cache.n_quant, c.cache.n_resid))
        end.record()
        wall_enqueue = time.perf_counter() - wall0
        torch.cuda.synchronize()
        gc.enable()
        total_us = start.elapsed_time(end) * 1e3
        dec = [a.elapsed_time(b) * 1e3 for a, b in ev] if ev else None
        host.append(wall0 + wall_enqueue)
        step_host_max = max(b - a for a, b in zip(host, host[1:])) * 1e6
        return total_us, state, dec, wall_enqueue, step_host_max

    # value: the steps with nothing but the region's two events
    total_us, state, _, wall_enq, host_max = timed(False)
    step_bytes = [_bytes_at(kq, layers[l].cache, nq, nr, Hq) for l, nq, nr in state]
    total_bytes = sum(step_bytes)
    value = total_bytes / (total_us * 1e-6) / 1e9
    # roofline: the same steps with events around each decode
    total_us2, state2, dec_us, _, _ = timed(True)
    bytes2 = [_bytes_at(kq, layers[l].cache, nq, nr, Hq) for l, nq, nr in state2]
    mean_dec_us = sum(dec_us) / len(dec_us)
    mean_bytes = sum(bytes2) / len(bytes2)
    achieved = mean_bytes / (mean_dec_us * 1e-6) / 1e9

    # decode launches with the Infinity Cache scrubbed before each one
    cold_med = None
    bytes_now = dc.decode_bytes(Hq)
    if not args.no_cold:
        cold = time_launches(torch, lambda: dc.decode(qs[-1], out=out, workspace=ws), 20, scrub)
        cold_med = statistics.median(cold)

    # the shader clock while the layers' decodes run back to back (the chip's
    # power limit sets it under this load)
    sclk = None
    if not args.no_clock:
        li = [0]

        def one():
            layers[li[0] % LAYERS].decode(qs[-1], out=out, workspace=ws)
            li[0] += 1
        sclk = sustained_sclk_mhz(torch, one)

    windows = [nr for _, _, nr in state]
    res = {
        "B": B, "Hq": Hq, "H": H, "S": S, "bits": bits,
        "total_ms": total_us * 1e-3, "ms_per_step": total_us * 1e-3 / args.steps,
        "host_enqueue_us_per_step": wall_enq / args.steps * 1e6,
        "host_enqueue_us_max_step": host_max,
        "value": value,
        "decode_bytes_per_step_mean": total_bytes / len(step_bytes),
        "window_tokens_min_max": [min(windows), max(windows)],
        "flushes_in_timed_steps": sum(1 for _, _, nr in state if nr == 1),
        "roofline_pass_ms_per_step": total_us2 * 1e-3 / args.steps,
        "mean_decode_us": mean_dec_us,
        "p50_decode_us": statistics.median(dec_us),
        "p95_decode_us": sorted(dec_us)[int(0.95 * (len(dec_us) - 1))],
        "decode_bytes_per_launch": mean_bytes,
        "achieved_gbs": achieved,
        "cold_decode_us_p50": cold_med,
        "cold_decode_gbs": None if cold_med is None else bytes_now / (cold_med * 1e-6) / 1e9,
        "append_us_p50": statistics.median(plain_us) if plain_us else None,
        # median: the first flushing append is the flush kernel's first launch
        # in this process
        "flush_append_us_p50": statistics.median(flush_us) if flush_us else None,
        "warmup_decodes": n_warm,
        "sclk_mhz_back_to_back_decodes": sclk,
        "prefill_quantize_us": pre_us,
        "prefill_quantize_gbs": q_bytes / (pre_us * 1e-6) / 1e9,
        "layers": LAYERS,
        "final_state": [[c.n_quant, c.n_resid] for c in layers],
    }
    return res


def sustained_sclk_mhz(torch, fn, secs=1.5):
    """Shader clock (MHz) sampled with `rocm-smi --showclocks` from another
    thread while `fn` runs back to back for `secs`; the first and last
    samples, which may fall outside the load, are dropped. None where
    rocm-smi is missing or fails."""
    exe = shutil.which("rocm-smi")
    if exe is None:
        return None
    samples, stop = [], threading.Event()

    def sampler():
        while not stop.is_set():
            try:
                r = subprocess.run([exe, "--showclocks", "--json"], capture_output=True,
                                   text=True, timeout=10)
            except (OSError, subprocess.SubprocessError):
                return
            m = re.search(r'sclk clock speed:": "\((\d+)Mhz\)', r.stdout)
            if m:
                samples.append(int(m.group(1)))
            stop.wait(0.2)

    t = threading.Thread(target=sampler, daemon=True)
    t.start()
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < secs:
        for _ in range(32):
            fn()
        torch.cuda.synchronize()
    stop.set()
    t.join(timeout=15)
    return samples[1:-1] or None


def copy_peak_gbs(torch, mib=1024, iters=10):
    """Device-to-device copy rate on this machine (read + write bytes / time),
    median of `iters` copies of `mib` MiB: a measured peak beside the
    published 8 TB/s."""
    n = mib << 18
    src = torch.ones(n, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    t = time_launches(torch, lambda: dst.copy_(src), iters)
    del src, dst
    torch.cuda.empty_cache()
    return 2 * (mib << 20) / (statistics.median(t) * 1e-6) / 1e9


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
            # the same ragged batch in pages of 256 tokens under a shuffled table
            dict(name="gqa70b_32k", fmt="kivi", ragged=True, paged=256),
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
        P = item.get("paged", 0)
        table, NP = None, 0
        if P:
            import numpy as np
            max_pages = -(-S // P)
            NP = B * max_pages
            perm = np.random.default_rng(0).permutation(NP).astype(np.int32)
            table = torch.from_numpy(perm.reshape(B, max_pages)).cuda()
        dc = kq.DeviceCache(kq.make_config(fmt, bits=bits, group_size=G, batch=B,
                                           num_kv_heads=H, capacity=S, v_bits=vbits or 0,
                                           scale_per_head=per_head, fp8_attention=qf8,
                                           v_group_channels=gc, page_tokens=P, num_pages=NP),
                            ragged=ragged, block_table=table)

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
               ("_ragged" if ragged else "") + (f"_paged{P}" if P else ""))
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


def _cpu_worker(arg):
    """One host process of the CPU baseline: its (b, KV head) blocks of the 32K
    GQA layer, drawn on the CPU, prefill-quantized, then `steps` decode steps
    (append + dequantize + fp64 attention of the block's query heads), on one
    thread. Returns (algorithmic decode bytes, prefill s, decode s)."""
    blocks, steps, in_dir = arg
    import numpy as np
    import torch
    from threadpoolctl import threadpool_limits

    import synth
    from oracle import attention, bytes_model, cache as ocache

    torch.set_num_threads(1)
    cfg = synth.CONFIGS["gqa70b_32k"]
    B, H, Hq, S = cfg["batch"], cfg["num_kv_heads"], cfg["num_q_heads"], cfg["seq_len"]
    nq = Hq // H
    with threadpool_limits(limits=1):
        # each block's K, V (tokens [0, S + steps)) and queries as drawn by the
        # parent (seeded synth; plain .npy arrays)
        kb = np.stack([np.load(os.path.join(in_dir, f"k_{b}_{h}.npy")) for b, h in blocks])
        vb = np.stack([np.load(os.path.join(in_dir, f"v_{b}_{h}.npy")) for b, h in blocks])
        q_all = np.load(os.path.join(in_dir, "q.npy"))                 # [steps, B, Hq, D]
        qs = [np.stack([q_all[i, b, h * nq:(h + 1) * nq] for b, h in blocks])
              for i in range(steps)]
        t0 = time.perf_counter()
        oc = ocache.KiviCache(len(blocks), 1, D, 2, 32, 128, S + steps)
        oc.prefill(kb[:, None, :S], vb[:, None, :S])
        t_pre = time.perf_counter() - t0
        nbytes = 0
        t0 = time.perf_counter()
        for i in range(steps):
            oc.append(kb[:, None, S + i], vb[:, None, S + i])
            Kh, Vh = oc.dequantized()
            for j in range(len(blocks)):
                attention.decode_attention(qs[i][j:j + 1], Kh[j:j + 1], Vh[j:j + 1])
            nbytes += bytes_model.decode_bytes_kivi(len(blocks), 1, D, 2, 32, oc.n_quant,
                                                    oc.n_resid)
        t_dec = time.perf_counter() - t0
    return nbytes, t_pre, t_dec


def _cpu_blocks(n):
    """The (b, KV head) blocks of the CPU baseline sample, spread over batch
    elements and heads."""
    return [((5 * j) % 16, (j + j // 16) % 8) for j in range(n)]


def cpu_baseline_child(workers, per_worker, steps, in_dir):
    """Runs in a child process that never touches the GPU: `workers` host
    processes (one thread each) of _cpu_worker over `per_worker` blocks each,
    started together; prints one JSON line."""
    import multiprocessing as mp

    n = workers * per_worker
    blocks = _cpu_blocks(n)
    chunks = [(blocks[w * per_worker:(w + 1) * per_worker], steps, in_dir)
              for w in range(workers)]
    t0 = time.perf_counter()
    if workers == 1:
        res = [_cpu_worker(chunks[0])]
    else:
        with mp.get_context("fork").Pool(workers) as pool:
            res = pool.map(_cpu_worker, chunks)
    wall = time.perf_counter() - t0
    nbytes = sum(r[0] for r in res)
    t_dec = max(r[2] for r in res)          # the workers decode side by side
    print(json.dumps({"bytes": nbytes, "decode_s": t_dec, "prefill_s": max(r[1] for r in res),
                      "blocks": n, "steps": steps, "workers": workers, "wall_s": wall}),
          flush=True)


def run_cpu_baseline(torch, synth):
    """The oracle, unmodified, on a bounded sample of the same workload, in a
    child process: once on one thread (8 blocks), once on N host cores (N
    processes of one thread, 2 blocks each; N = the cores this process may
    run on, at most 16). The blocks' inputs are drawn here (on the GPU when
    there is one: the same seeded values) and handed over as .npy files."""
    import shutil
    import tempfile

    import numpy as np

    cfg = synth.CONFIGS["gqa70b_32k"]
    B, H, Hq, S = cfg["batch"], cfg["num_kv_heads"], cfg["num_q_heads"], cfg["seq_len"]
    steps = 8
    n_all = min(16, len(os.sched_getaffinity(0)))
    dev = "cuda" if torch.cuda.is_available() else "cpu"
    in_dir = tempfile.mkdtemp(prefix="kvq_cpu_baseline_")
    try:
        for b, h in sorted(set(_cpu_blocks(max(8, 2 * n_all)))):
            np.save(os.path.join(in_dir, f"k_{b}_{h}.npy"),
                    synth.make_k(1, H, 0, S + steps, D, device=dev, b0=b, heads=[h])[0, 0].cpu().numpy())
            np.save(os.path.join(in_dir, f"v_{b}_{h}.npy"),
                    synth.make_v(1, H, 0, S + steps, D, device=dev, b0=b, heads=[h])[0, 0].cpu().numpy())
        np.save(os.path.join(in_dir, "q.npy"), np.stack(
            [synth.make_q(B, Hq, D, step=i, device=dev).cpu().numpy() for i in range(steps)]))
        runs = {}
        for workers, per in ((1, 8), (n_all, 2)):
            r = subprocess.run([sys.executable, os.path.abspath(__file__), "--cpu-baseline-child",
                                str(workers), str(per), str(steps), in_dir], capture_output=True,
                               text=True, timeout=900, cwd=ROOT)
            if r.returncode != 0:
                raise RuntimeError(f"cpu baseline child failed:\n{r.stderr[-2000:]}")
            runs[workers] = json.loads(r.stdout.strip().splitlines()[-1])
            _log(f"[bench] cpu baseline {workers} core(s): {runs[workers]}")
    finally:
        shutil.rmtree(in_dir, ignore_errors=True)
    one, alln = runs[1], runs[n_all]
    gbs = lambda r: r["bytes"] / r["decode_s"] / 1e9
    return {"value": round(gbs(alln), 4), "unit": "GB/s", "cores": n_all, "kind": "oracle",
            "sample": (f"{alln['blocks']} of 128 (b, KV head) blocks of the 32K GQA layer, "
                       f"{alln['steps']} decode steps each (append + dequantize + fp64 "
                       f"attention of 8 query heads), {n_all} host processes of one thread "
                       f"side by side (2 blocks each), decode {alln['decode_s']:.2f}s"),
            "single_thread": {"value": round(gbs(one), 4), "unit": "GB/s", "cores": 1,
                              "sample": f"{one['blocks']} blocks x {one['steps']} steps, "
                                        f"decode {one['decode_s']:.2f}s, prefill quantize "
                                        f"{one['prefill_s']:.2f}s"},
            "decode_s_per_block_step_1_thread": round(one["decode_s"] / (8 * one["blocks"]), 4)}


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=256)
    ap.add_argument("--warmup", type=int, default=16)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extra", action="store_true")
    ap.add_argument("--no-clock", action="store_true",
                    help="skip sampling the shader clock (rocm-smi) during back-to-back decodes")
    ap.add_argument("--no-cold", action="store_true",
                    help="skip the scrubbed single-launch decode timing (profiling runs)")
    ap.add_argument("--copy-probe-mib", type=int, default=0,
                    help="after the run, copy a device buffer of this many MiB (a known-size "
                         "transfer that calibrates rocprofv3 FETCH_SIZE / WRITE_SIZE)")
    ap.add_argument("--warmup-s", type=float, default=0.5,
                    help="seconds of decodes before the warm-up steps (clocks settle under "
                         "the load)")
    ap.add_argument("--cpu-baseline-child", nargs=4, metavar=("WORKERS", "BLOCKS", "STEPS", "DIR"),
                    help=argparse.SUPPRESS)
    args = ap.parse_args()
    if args.cpu_baseline_child:
        w, blk, st, d = args.cpu_baseline_child
        cpu_baseline_child(int(w), int(blk), int(st), d)
        return
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
    copy_gbs = copy_peak_gbs(torch)
    cpu = None if args.no_cpu_baseline else run_cpu_baseline(torch, synth)
    props = torch.cuda.get_device_properties(0)
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
                     "mean_launch_us": round(main_res["mean_decode_us"], 3),
                     "measured_copy_gbs": round(copy_gbs, 1),
                     "frac_of_measured_copy": round(achieved / copy_gbs, 4)},
        "cpu_baseline": cpu,
        "details": {k: (round(v, 3) if isinstance(v, float) else v)
                    for k, v in main_res.items()},
        "env": {"device": props.name, "compute_units": props.multi_processor_count,
                "torch": torch.__version__, "hip": torch.version.hip,
                "decode_source_hash": decode_source_hash(), "bench_sha256_16": _file_hash()},
        "extra": extra,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
