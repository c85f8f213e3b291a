#!/usr/bin/env python
"""rocprofv3 evidence for the decode kernel of bench.py's gqa70b_32k workload.

Three profiler runs of a short bench (each its own process, the program right
after `--`):
  1. --kernel-trace --stats: per-kernel launch counts and average durations;
  2. --pmc FETCH_SIZE and 3. --pmc WRITE_SIZE (KiB per dispatch), both with a
     1 GiB device-to-device copy at the end (--copy-probe-mib 1024), whose
     known size calibrates the two counters.
Writes decode_gqa70b_32k_kernel_stats.txt, decode_gqa70b_32k_counters.txt and
decode_gqa70b_32k_counters.json (read by bench.py for roofline.traffic, keyed by
a hash of the decode sources) to OUT/profiles/ (OUT below), to be copied into
profiles/; raw profiler output stays under OUT/prof_*.
Run on a machine with the GPU: python profile_counters.py
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
               "--no-cpu-baseline", "--no-extra", "--no-cold"]
BENCH = ["python3", os.path.join(ROOT, "bench.py"), "--steps", "16", "--warmup", "4",
         "--no-cpu-baseline", "--no-extra", "--no-cold"]
COPY_MIB = 1024
DECODE = "kivi_mfma_split_kernel<2, 2, 1, true>"   # the unit-sized workgroup shape
MERGE = "decode_merge_kernel"


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


def main():
    os.makedirs(PROF, exist_ok=True)
    from bench import decode_source_hash

    d1, c1 = run("stats", ["--kernel-trace", "--stats"], bench=BENCH_STATS)
    stats = glob.glob(os.path.join(d1, "**", "*kernel_stats.csv"), recursive=True)[0]
    write_stats_summary(stats, rel(c1), os.path.join(PROF, "decode_gqa70b_32k_kernel_stats.txt"))

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
