#!/usr/bin/env python
"""rocprofv3 evidence for the decode kernel of bench.py's gqa70b_32k workload.

Profiler runs of a short bench (each its own process, the program right
after `--`), chosen by name on the command line (default: all):
  stats    --kernel-trace --stats: per-kernel launch counts and average
           durations over the bench's default steps;
  traffic  --pmc FETCH_SIZE, then --pmc WRITE_SIZE (KiB per dispatch), both
           with a 1 GiB device-to-device copy at the end
           (--copy-probe-mib 1024), whose known size calibrates the counters;
  sq       three --pmc passes of SQ_* / GRBM_* counters over the split kernel
           (instructions per 32-token group, VALU and MFMA busy, LDS bank
           conflicts, shader clock);
  gaps     --kernel-trace of a short benchmark run
           (--steps 20 --warmup 5): kernel durations and the idle gaps
           between the kernels of its timed steps;
  quant    the prefill quantize kernel of the same short bench (its 32K
           prefills, the dispatches with the largest grid): durations from a
           kernel trace, the SQ / GRBM passes, FETCH_SIZE / WRITE_SIZE
           calibrated by the 1 GiB copy, against the bytes it must move.
Writes decode_gqa70b_32k_kernel_stats.txt, decode_gqa70b_32k_counters.txt,
decode_gqa70b_32k_counters.json (read by bench.py for roofline.traffic, keyed by
a hash of the decode sources), decode_gqa70b_32k_sq_counters.txt,
decode_gqa70b_32k_step_gaps.txt and prefill_quantize_gqa70b_32k_counters.txt
to OUT/profiles/ (OUT below), to be copied
into profiles/; raw profiler output stays under OUT/prof_*.
Run on a machine with the GPU: python profile_counters.py [stats traffic sq gaps quant]
"""
from __future__ import annotations

import csv
import glob
import json
import os
import re
import statistics
import subprocess
import sys

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)
OUT = os.path.join(ROOT, "gpurun_out")
PROF = os.path.join(OUT, "profiles")          # copied into profiles/ afterwards
# the kernel-trace pass times the bench's own default steps (so that its
# average decode duration compares with the bench line); the counter passes,
# which serialize every dispatch they count, use a short run
BENCH_STATS = ["python3", os.path.join(ROOT, "bench.py"), "--steps", "256", "--warmup", "16",
               "--no-cpu-baseline", "--no-extra", "--no-cold", "--no-clock"]
BENCH = ["python3", os.path.join(ROOT, "bench.py"), "--steps", "16", "--warmup", "4",
         "--no-cpu-baseline", "--no-extra", "--no-cold", "--no-clock"]
BENCH_DRIVER = ["python3", os.path.join(ROOT, "bench.py"), "--gpus", "1", "--steps", "20",
                "--warmup", "5", "--no-cpu-baseline", "--no-extra", "--no-clock"]
COPY_MIB = 1024
# SQ / GRBM counter passes (at most 8 SQ and 2 GRBM counters per pass)
SQ_PASSES = [
    ["SQ_WAVES", "SQ_INSTS_VALU", "SQ_INSTS_MFMA", "SQ_INSTS_LDS", "SQ_INSTS_SALU",
     "SQ_INSTS_VMEM_RD", "SQ_BUSY_CYCLES", "SQ_WAVE_CYCLES", "GRBM_GUI_ACTIVE", "GRBM_COUNT"],
    ["SQ_ACTIVE_INST_VALU", "SQ_VALU_MFMA_BUSY_CYCLES", "SQ_ACTIVE_INST_LDS",
     "SQ_LDS_BANK_CONFLICT", "SQ_WAIT_INST_ANY", "SQ_ACTIVE_INST_ANY", "SQ_INST_CYCLES_VMEM_RD",
     "SQ_INSTS_SMEM"],
    ["SQ_INSTS_VALU_CVT", "SQ_INSTS_VALU_INT32", "SQ_INSTS_VALU_FMA_F32", "SQ_INSTS_VALU_MUL_F32",
     "SQ_INSTS_VALU_ADD_F32", "SQ_INSTS_VALU_TRANS_F32", "SQ_INSTS_VALU_MFMA_MOPS_F16",
     "SQ_INSTS_VALU_MFMA_MOPS_BF16"],
]
N_SIMD = 1024          # 256 compute units x 4 SIMDs
N_XCD = 8
DECODE = "kivi_mfma_split_kernel<2, 2, 1, true, false, false>"   # unit-sized workgroups, contiguous, G = 32
MERGE = "decode_merge_kernel"
QUANT = "kivi_quantize_kernel<2, 2, 1>"
# the 32K prefill: B = 16, 8 KV heads, 32768 tokens of which 32640 are grouped
# (R = 128 stay in the window), D = 128, 2-bit K and V, G = 32
PRE_B, PRE_H, PRE_NQ, PRE_D, PRE_BITS, PRE_G = 16, 8, 32640, 128, 2, 32


def run(tag, prof_args, extra=(), bench=BENCH):
    d = os.path.join(OUT, f"prof_{tag}")
    cmd = ["rocprofv3", *prof_args, "--output-format", "csv", "-d", d, "-o", "run", "--",
           *bench, *extra]
    print("[profile] " + " ".join(cmd), flush=True)
    with open(os.path.join(OUT, f"prof_{tag}.log"), "w") as log:
        r = subprocess.run(cmd, stdout=log, stderr=subprocess.STDOUT, timeout=300,
                           cwd="/tmp", env={**os.environ, "TMPDIR": "/tmp"})
    print(f"[profile] {tag}: exit {r.returncode}", flush=True)
    if r.returncode != 0:
        sys.exit(r.returncode)
    return d, cmd


def short(name):
    name = re.sub(r"\(anonymous namespace\)::", "", name)
    name = name[5:] if name.startswith("void ") else name
    return name.split("(")[0]


def rel(cmd):
    return " ".join(c.replace(ROOT + "/", "").replace(OUT, "gpurun_out") for c in cmd)


def write_stats_summary(csv_path, cmd, out_path):
    """Every kvq kernel, then the five longest others (the input generator)."""
    with open(csv_path) as fh:
        srows = list(csv.DictReader(fh))
    srows.sort(key=lambda r: -float(r["TotalDurationNs"]))
    ours = [r for r in srows if "kvq::" in r["Name"]]
    rest = [r for r in srows if "kvq::" not in r["Name"]][:5]
    lines = ["# rocprofv3 kernel stats, gqa70b_32k decode (bench.py, 256 timed + 16 warmup steps, "
             "4 layer caches)",
             f"# command: {cmd}",
             f"# {'kernel':62s} {'calls':>6s} {'avg_us':>10s} {'min_us':>10s} {'max_us':>10s}"]
    for r in ours + rest:
        lines.append(f"  {short(r['Name'])[:62]:62s} {int(r['Calls']):6d} "
                     f"{float(r['AverageNs']) / 1e3:10.2f} {float(r['MinNs']) / 1e3:10.2f} "
                     f"{float(r['MaxNs']) / 1e3:10.2f}")
    with open(out_path, "w") as fh:
        fh.write("\n".join(lines) + "\n")


def counter_rows(d):
    f = glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True)
    assert f, f"no counter csv under {d}"
    with open(f[0]) as fh:
        return list(csv.DictReader(fh))


def per_kernel(rows, counter):
    by = {}
    for r in rows:
        if r["Counter_Name"] == counter:
            by.setdefault(r["Kernel_Name"], []).append(float(r["Counter_Value"]))
    return by


def pick(by, needle):
    keys = [k for k in by if needle in k]
    assert keys, f"{needle} not found"
    return [v for k in keys for v in by[k]]


def copy_reading(by):
    """The 1 GiB copy: the dispatch with the largest counter value among the
    blit / copy kernels."""
    vals = [max(v) for k, v in by.items() if "copy" in k.lower()]
    return max(vals)


def split_stats_avg_us():
    """The split kernel's average duration from the stats pass (written by it)."""
    f = glob.glob(os.path.join(OUT, "prof_stats", "**", "*kernel_stats.csv"), recursive=True)
    if not f:
        return None
    with open(f[0]) as fh:
        for r in csv.DictReader(fh):
            if DECODE in short(r["Name"]):
                return float(r["AverageNs"]) / 1e3
    return None


def sq_pass():
    """Counters of the split kernel, median per dispatch, and what they give
    per 32-token group; the group count of a dispatch is the bench's grouped
    tiles (16·8 (b, KV head) blocks × 1024 tiles after the first flush)."""
    vals, cmds = {}, []
    for i, ctrs in enumerate(SQ_PASSES):
        d, c = run(f"sq{i}", ["--pmc", *ctrs, "--kernel-include-regex", "kivi_mfma_split_kernel"])
        cmds.append(rel(c))
        rows = counter_rows(d)
        for ctr in ctrs:
            v = pick(per_kernel(rows, ctr), DECODE)
            vals[ctr] = statistics.median(v)
        if i == 0:   # the pass that counts GRBM_GUI_ACTIVE: its own dispatch time
            ctr_us = dispatch_us(rows, DECODE)
    tiles = 16 * 8 * 1024
    waves = vals["SQ_WAVES"]
    dur_us = split_stats_avg_us()
    lines = ["# rocprofv3 SQ / GRBM counters of the split kernel, gqa70b_32k decode "
             "(bench.py --steps 16 --warmup 4, 4 layer caches); median per dispatch"]
    lines += [f"# command (pass {i}): {c}" for i, c in enumerate(cmds)]
    lines += [f"{k:32s} {v:16.0f}" for k, v in vals.items()]
    per = lambda k: vals[k] / tiles
    lines.append(f"groups (32-token tiles) per dispatch: {tiles}; wavefronts: {waves:.0f}")
    for k in ("SQ_INSTS_VALU", "SQ_INSTS_MFMA", "SQ_INSTS_LDS", "SQ_INSTS_SALU", "SQ_INSTS_VMEM_RD",
              "SQ_INSTS_SMEM", "SQ_INSTS_VALU_CVT", "SQ_INSTS_VALU_INT32", "SQ_INSTS_VALU_FMA_F32",
              "SQ_INSTS_VALU_MUL_F32", "SQ_INSTS_VALU_ADD_F32", "SQ_INSTS_VALU_TRANS_F32"):
        lines.append(f"{k} per group: {per(k):8.1f}")
    cyc = vals["GRBM_GUI_ACTIVE"] / N_XCD
    clk = cyc / (ctr_us * 1e-6) / 1e9
    if dur_us:
        lines.append(f"split kernel average duration (stats pass): {dur_us:.2f} us")
    lines.append(f"split kernel in the counter pass: {ctr_us:.2f} us (median), "
                 f"GRBM_GUI_ACTIVE / {N_XCD} XCDs = {cyc:.0f} cycles -> shader clock "
                 f"{clk:.2f} GHz")
    # SQ_ACTIVE_INST_VALU counts quad-cycles per wave; one VALU issue per SIMD per cycle
    lines.append(f"VALU busy = 4*SQ_ACTIVE_INST_VALU / (SIMDs * GUI cycles) = "
                 f"{4 * vals['SQ_ACTIVE_INST_VALU'] / (N_SIMD * cyc):.3f}")
    lines.append(f"MFMA busy = SQ_VALU_MFMA_BUSY_CYCLES / (SIMDs * GUI cycles) = "
                 f"{vals['SQ_VALU_MFMA_BUSY_CYCLES'] / (N_SIMD * cyc):.3f}")
    lines.append(f"VALU issue time at that clock: 4 cycles x SQ_INSTS_VALU / SIMDs = "
                 f"{4 * vals['SQ_INSTS_VALU'] / N_SIMD / (clk * 1e3):.1f} us of {ctr_us:.1f} us")
    lines.append(f"LDS bank conflict cycles per LDS instruction: "
                 f"{vals['SQ_LDS_BANK_CONFLICT'] / max(1.0, vals['SQ_INSTS_LDS']):.3f}")
    with open(os.path.join(PROF, "decode_gqa70b_32k_sq_counters.txt"), "w") as fh:
        fh.write("\n".join(lines) + "\n")
    print("\n".join(lines), flush=True)


def gaps_pass():
    """Kernel durations and idle gaps of the timed steps of the short bench
    run. The bench runs 5 warm-up steps, then the 20 steps its value is
    taken from (one kvq_append_decode call each: the split and merge
    launches, after the flush's quantize launch when one is due), then the
    same 20 steps as an append's copy launch followed by the decode, with
    events around each decode (its roofline pass)."""
    d, c = run("gaps", ["--kernel-trace"], bench=BENCH_DRIVER)
    f = glob.glob(os.path.join(d, "**", "*kernel_trace.csv"), recursive=True)[0]
    with open(f) as fh:
        rows = list(csv.DictReader(fh))
    rows.sort(key=lambda r: int(r["Start_Timestamp"]))
    names = [short(r["Kernel_Name"]) for r in rows]
    t0 = [int(r["Start_Timestamp"]) for r in rows]
    t1 = [int(r["End_Timestamp"]) for r in rows]
    splits = [i for i in range(1, len(rows)) if DECODE in names[i]]
    # the roofline pass: the 20 splits right after an append's copy launch
    roof = [i for i in splits if "copy_tokens_kernel" in names[i - 1]][-20:]
    # the value pass: the 20 splits before the roofline pass's first step
    value = [i for i in splits if i < roof[0] - 1][-20:]
    lines = ["# rocprofv3 kernel trace of a short benchmark run: per timed step, "
             "the append's kernels (none in a fused step without a flush), the decode's "
             "split and merge, and the idle time on the GPU between them",
             f"# command: {rel(c)}"]
    # the first step of each pass follows a host synchronization: left out
    for tag, sel in (("value pass (kvq_append_decode, region events only)", value[1:]),
                     ("roofline pass (append, then events around each decode)", roof[1:])):
        step_us, idle_us, split_us, merge_us, app_us = [], [], [], [], []
        for i in sel:
            first = i
            while first > 0 and ("copy_tokens_kernel" in names[first - 1] or
                                 "kivi_quantize_kernel" in names[first - 1]):
                first -= 1
            last = i + 1 if i + 1 < len(rows) and MERGE in names[i + 1] else i
            busy = sum(t1[k] - t0[k] for k in range(first, last + 1))
            # the step runs from the end of the previous kernel to its last kernel's end
            span = t1[last] - t1[first - 1]
            step_us.append(span / 1e3)
            idle_us.append((span - busy) / 1e3)
            split_us.append((t1[i] - t0[i]) / 1e3)
            if last != i:
                merge_us.append((t1[last] - t0[last]) / 1e3)
            app_us.append(sum(t1[k] - t0[k] for k in range(first, i)) / 1e3)
        m = statistics.mean
        lines.append(f"{tag}: {len(sel)} steps; step {m(step_us):.2f} us = append kernels "
                     f"{m(app_us):.2f} + split {m(split_us):.2f} + merge "
                     f"{m(merge_us) if merge_us else 0:.2f} + idle {m(idle_us):.2f}")
    lines.append("idle: the GPU waiting for the host, which under --kernel-trace pays the "
                 "tracer's work on every launch; the bench's own host_enqueue_us_max_step (no "
                 "tracer) is the host time of the untraced command. The kernel durations are "
                 "the figures to set against the bench line's per-decode events.")
    with open(os.path.join(PROF, "decode_gqa70b_32k_step_gaps.txt"), "w") as fh:
        fh.write("\n".join(lines) + "\n")
    print("\n".join(lines), flush=True)


def dispatch_us(rows, needle, grid=None):
    """Median duration (us) of the counted dispatches of a kernel, from the
    counter pass's own timestamps (one row per counter: deduplicated by
    dispatch); `grid`: only dispatches of that grid size."""
    seen = {}
    for r in rows:
        if needle in short(r["Kernel_Name"]) and (grid is None or int(r["Grid_Size"]) == grid):
            seen[r["Dispatch_Id"]] = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3
    return statistics.median(seen.values())


def prefill_values(rows, counter):
    """`counter` of the prefill quantize dispatches: the quantize dispatches
    with the largest grid (the flushes of a full window have 4 groups per
    (b, h) block, the 32K prefills 1020)."""
    q = [r for r in rows if QUANT in short(r["Kernel_Name"]) and r["Counter_Name"] == counter]
    assert q, f"no {QUANT} dispatch with {counter}"
    g = max(int(r["Grid_Size"]) for r in q)
    return [float(r["Counter_Value"]) for r in q if int(r["Grid_Size"]) == g]


def quant_pass():
    """Evidence for the prefill quantize kernel: what it moves and how busy
    its units are."""
    d, c_trace = run("qtrace", ["--kernel-trace"])
    f = glob.glob(os.path.join(d, "**", "*kernel_trace.csv"), recursive=True)[0]
    with open(f) as fh:
        rows = [r for r in csv.DictReader(fh) if QUANT in short(r["Kernel_Name"])]
    durs = sorted((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3 for r in rows)
    pre = [x for x in durs if x > 20 * durs[0]]          # the prefills, not the flushes
    dur_us = statistics.median(pre)
    cmds = {"trace": rel(c_trace)}
    vals = {}
    for i, ctrs in enumerate(SQ_PASSES):
        d, c = run(f"qsq{i}", ["--pmc", *ctrs, "--kernel-include-regex", "kivi_quantize_kernel"])
        cmds[f"sq{i}"] = rel(c)
        rows = counter_rows(d)
        for ctr in ctrs:
            vals[ctr] = statistics.median(prefill_values(rows, ctr))
        if i == 0:   # the pass that counts GRBM_GUI_ACTIVE: its own dispatch time
            g = max(int(r["Grid_Size"]) for r in rows if QUANT in short(r["Kernel_Name"]))
            ctr_us = dispatch_us(rows, QUANT, g)
    traffic = {}
    for ctr in ("FETCH_SIZE", "WRITE_SIZE"):
        d, c = run(f"q{ctr.lower()}", ["--pmc", ctr, "--kernel-include-regex",
                                       "kivi_quantize_kernel|[Cc]opy"],
                   ["--copy-probe-mib", str(COPY_MIB)])
        cmds[ctr] = rel(c)
        rows = counter_rows(d)
        kib = statistics.median(prefill_values(rows, ctr))
        scale = COPY_MIB * 1024.0 / copy_reading(per_kernel(rows, ctr))
        traffic[ctr] = (kib, scale, kib * scale * 1024)
    bh = PRE_B * PRE_H
    read = 2 * bh * PRE_NQ * PRE_D * 2
    write = bh * (2 * PRE_NQ * PRE_D * PRE_BITS // 8 + (PRE_NQ // PRE_G) * PRE_D * 8 + PRE_NQ * 8)
    groups = bh * (PRE_NQ // PRE_G)
    cyc = vals["GRBM_GUI_ACTIVE"] / N_XCD
    lines = ["# prefill quantize kernel (KIVI 2-bit, G = 32) of the 32K GQA layer: "
             "B = 16, 8 KV heads, 32640 grouped tokens per (b, h) block",
             *[f"# command ({k}): {v}" for k, v in cmds.items()],
             f"prefill dispatches timed: {len(pre)}; median duration {dur_us:.1f} us "
             f"(kernel trace, no counters)",
             f"bytes it must move: read {read / 1e6:.1f} MB (fp16 K and V), write "
             f"{write / 1e6:.1f} MB (codes, K scale / zero per group and channel, V scale / "
             f"zero per token); {(read + write) / 1e6:.1f} MB",
             f"achieved: {(read + write) / (dur_us * 1e-6) / 1e9:.0f} GB/s = "
             f"{(read + write) / (dur_us * 1e-6) / 8e12:.3f} of 8 TB/s"]
    for ctr, (kib, scale, b) in traffic.items():
        lines.append(f"{ctr}: {kib:.0f} KiB per prefill dispatch x copy scale {scale:.4f} = "
                     f"{b / 1e6:.1f} MB")
    lines.append(f"HBM traffic / bytes it must move: "
                 f"{(traffic['FETCH_SIZE'][2] + traffic['WRITE_SIZE'][2]) / (read + write):.3f}")
    lines += [f"{k:32s} {v:16.0f}" for k, v in vals.items()]
    lines.append(f"groups (32 tokens of one (b, h) block) per dispatch: {groups}; "
                 f"wavefronts: {vals['SQ_WAVES']:.0f}")
    for k in ("SQ_INSTS_VALU", "SQ_INSTS_LDS", "SQ_INSTS_SALU", "SQ_INSTS_VMEM_RD",
              "SQ_INSTS_VALU_CVT", "SQ_INSTS_VALU_FMA_F32", "SQ_INSTS_VALU_MUL_F32",
              "SQ_INSTS_VALU_ADD_F32"):
        lines.append(f"{k} per group: {vals[k] / groups:8.1f}")
    clk = cyc / (ctr_us * 1e-6) / 1e9
    lines.append(f"GRBM_GUI_ACTIVE / {N_XCD} XCDs = {cyc:.0f} cycles over the counter pass's "
                 f"own dispatch time {ctr_us:.1f} us (dispatches serialized) -> {clk:.2f} GHz")
    lines.append(f"VALU busy = 4*SQ_ACTIVE_INST_VALU / (SIMDs * GUI cycles) = "
                 f"{4 * vals['SQ_ACTIVE_INST_VALU'] / (N_SIMD * cyc):.3f}")
    lines.append(f"VALU issue time: 4 cycles x SQ_INSTS_VALU / SIMDs at that clock = "
                 f"{4 * vals['SQ_INSTS_VALU'] / N_SIMD / (clk * 1e3):.1f} us of {ctr_us:.1f} us")
    lines.append(f"LDS bank conflict cycles per LDS instruction: "
                 f"{vals['SQ_LDS_BANK_CONFLICT'] / max(1.0, vals['SQ_INSTS_LDS']):.3f}")
    with open(os.path.join(PROF, "prefill_quantize_gqa70b_32k_counters.txt"), "w") as fh:
        fh.write("\n".join(lines) + "\n")
    print("\n".join(lines), flush=True)


def main():
    os.makedirs(PROF, exist_ok=True)
    from bench import decode_source_hash
    passes = sys.argv[1:] or ["stats", "traffic", "sq", "gaps", "quant"]

    if "stats" in passes:
        d1, c1 = run("stats", ["--kernel-trace", "--stats"], bench=BENCH_STATS)
        stats = glob.glob(os.path.join(d1, "**", "*kernel_stats.csv"), recursive=True)[0]
        write_stats_summary(stats, rel(c1),
                            os.path.join(PROF, "decode_gqa70b_32k_kernel_stats.txt"))
    if "sq" in passes:
        sq_pass()
    if "gaps" in passes:
        gaps_pass()
    if "quant" in passes:
        quant_pass()
    if "traffic" not in passes:
        return

    res = {}
    cmds = {}
    for ctr in ("FETCH_SIZE", "WRITE_SIZE"):
        # counters only on the decode kernels and the copy: the input generator's
        # thousands of small dispatches would each be serialized otherwise
        d, c = run(ctr.lower(), ["--pmc", ctr, "--kernel-include-regex",
                                 "kivi_mfma_split_kernel|decode_merge_kernel|[Cc]opy"],
                   ["--copy-probe-mib", str(COPY_MIB)])
        cmds[ctr] = rel(c)
        by = per_kernel(counter_rows(d), ctr)
        dec = pick(by, DECODE)
        mrg = pick(by, MERGE)
        cp = copy_reading(by)
        factor = COPY_MIB * 1024.0 / cp          # true KiB per counted KiB
        res[ctr] = {"decode_kib_median": statistics.median(dec), "merge_kib_median":
                    statistics.median(mrg), "copy_kib": cp, "copy_true_kib": COPY_MIB * 1024,
                    "scale": factor, "decode_dispatches": len(dec)}
    fetch = res["FETCH_SIZE"]["decode_kib_median"] * res["FETCH_SIZE"]["scale"] * 1024
    write = res["WRITE_SIZE"]["decode_kib_median"] * res["WRITE_SIZE"]["scale"] * 1024
    merge = (res["FETCH_SIZE"]["merge_kib_median"] * res["FETCH_SIZE"]["scale"] +
             res["WRITE_SIZE"]["merge_kib_median"] * res["WRITE_SIZE"]["scale"]) * 1024
    out = {"decode_source_hash": decode_source_hash(),
           "traffic_bytes_per_launch": int(round(fetch + write + merge)),
           "split_kernel_fetch_bytes": int(round(fetch)),
           "split_kernel_write_bytes": int(round(write)),
           "merge_kernel_bytes": int(round(merge)),
           "counters": res, "commands": cmds}
    with open(os.path.join(PROF, "decode_gqa70b_32k_counters.json"), "w") as fh:
        json.dump(out, fh, indent=1)
    txt = [f"# rocprofv3 FETCH_SIZE / WRITE_SIZE, gqa70b_32k decode, calibrated by a "
           f"{COPY_MIB} MiB device copy in the same run",
           f"# command (fetch): {cmds['FETCH_SIZE']}",
           f"# command (write): {cmds['WRITE_SIZE']}"]
    for ctr, r in res.items():
        txt.append(f"{ctr}: decode split median {r['decode_kib_median']:.1f} KiB over "
                   f"{r['decode_dispatches']} dispatches; merge {r['merge_kib_median']:.1f} KiB; "
                   f"copy reads {r['copy_kib']:.1f} KiB for {r['copy_true_kib']} KiB "
                   f"(scale {r['scale']:.4f})")
    txt.append(f"HBM traffic per decode (split + merge), scaled: "
               f"{out['traffic_bytes_per_launch'] / 1e6:.2f} MB "
               f"(split fetch {fetch / 1e6:.2f} MB, split write {write / 1e6:.2f} MB, "
               f"merge {merge / 1e6:.2f} MB)")
    with open(os.path.join(PROF, "decode_gqa70b_32k_counters.txt"), "w") as fh:
        fh.write("\n".join(txt) + "\n")
    print("\n".join(txt), flush=True)


if __name__ == "__main__":
    main()
