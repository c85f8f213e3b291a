"""Builds libkvq.so (the HIP kernels and the C ABI) for gfx950 with hipcc.

Usage: python kv_cache_quantization_quant_amd/build.py   (or build.build()); it does not
import the package, so a stale library never blocks a rebuild.
Always recompiles every source; objects go to _build/ next to this file.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import re
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
OUT = os.path.join(PKG, "libkvq.so")
BUILD_DIR = os.path.join(PKG, "_build")

SOURCES = ["kvq_api.cpp", "kvq_quant.hip", "kvq_quant_kivi.hip", "kvq_decode.hip",
           "kvq_decode_mfma.hip"]

HIPCC = os.environ.get("HIPCC", shutil.which("hipcc") or "/opt/rocm/bin/hipcc")

COMMON = [
    "-O3", "-std=c++17", "-fPIC", "--offload-arch=gfx950",
    # IEEE fp32: no contraction into FMA unless written as fmaf; correctly
    # rounded division (the HIP default, stated explicitly).
    "-ffp-contract=off", "-fhip-fp32-correctly-rounded-divide-sqrt",
    # no packed-FP32 VALU instructions
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # MFMA accumulators in ordinary VGPRs (no AGPR copies around VALU work)
    "-mllvm", "-amdgpu-mfma-vgpr-form",
    "-Wall", "-Wno-unused-function",
    "-I", os.path.join(ROOT, "include"),
]


def _scratch_kernels(remarks: str) -> list[str]:
    """Kernels whose resource-usage remark reports scratch (spilled registers
    or stack): such a kernel issues vector-memory instructions the decode
    kernels' hand-counted `s_waitcnt vmcnt` waits do not expect."""
    bad, name = [], None
    for line in remarks.splitlines():
        m = re.search(r"Function Name: (\S+)", line)
        if m:
            name = m.group(1)
        m = re.search(r"ScratchSize \[bytes/lane\]: (\d+)", line)
        if m and name and int(m.group(1)) > 0:
            bad.append(f"{name} ({m.group(1)} bytes/lane)")
    return bad


# Per-source flags. The decode kernels' only atomics are the LDS tile counters,
# taken by one lane per wavefront: the atomic optimizer's wave-wide
# reduction around them (lane counts, prefix, broadcast) is pure overhead in
# the steady-state loop.
EXTRA = {
    "kvq_decode_mfma.hip": ["-mllvm", "-amdgpu-atomic-optimizer-strategy=None"],
    # IEEE mode off for the KIVI quantizer: its fp16 min / max need no quieting
    # of every loaded value first (the flag requires relaxed NaN handling)
    "kvq_quant_kivi.hip": ["-mno-amdgpu-ieee", "-fno-honor-nans"],
}


def _compile(src: str) -> str:
    obj = os.path.join(BUILD_DIR, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC, *COMMON, *EXTRA.get(src, []), "-x", "hip", "-c", os.path.join(CSRC, src),
           "-o", obj]
    if src.endswith(".hip"):
        cmd.append("-Rpass-analysis=kernel-resource-usage")
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stdout}\n{r.stderr}")
    bad = _scratch_kernels(r.stderr)
    if bad:
        raise RuntimeError(f"{src}: kernels using scratch memory: {', '.join(bad)}")
    return obj


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD_DIR, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=len(SOURCES)) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = OUT + ".tmp"
    cmd = [HIPCC, "-shared", "-fPIC", "--offload-arch=gfx950", *objs, "-o", tmp,
           "-Wl,-rpath,/opt/rocm/lib"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, OUT)
    if verbose:
        print(f"built {OUT}")
    return OUT


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
