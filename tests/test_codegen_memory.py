"""Generated-code checks of the memory instructions the kernels' speed rests on
(compiles only; no GPU).

- The KIVI quantizer writes every code, scale and zero-point with a
  non-temporal store (`global_store_* … nt`): its outputs are read much later
  by the decode, and stores that stay dirty in the Infinity Cache are written
  back during the next kernel's reads. The optimizer once merged the code
  stores with their copies on the exact-division path and dropped the
  non-temporal mark (the back-to-back 32K prefill then took 459 µs instead
  of 423).
- The paged KIVI decode reads its block-table entries with scalar loads. A
  vector load there makes the compiler wait for it with `s_waitcnt vmcnt(0)`,
  which also waits for every copy the ring has in flight, once per tile
  (76 µs instead of 67.5 for the paged 32K batch).
"""
import os
import re
import subprocess

import pytest

from kv_cache_quantization_quant_amd import build as kbuild


def _compile(src_name):
    src = os.path.join(kbuild.CSRC, src_name)
    cmd = [kbuild.HIPCC, *[f for f in kbuild.COMMON if f != "-fPIC"],
           *kbuild.EXTRA.get(src_name, []), "--cuda-device-only", "-S", "-x", "hip", src,
           "-o", "-"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    return r.stdout


def _kernels(asm, pattern):
    lines = asm.splitlines()
    out = {}
    for i, line in enumerate(lines):
        m = re.match(r"^(_Z\w+):", line)
        if m and re.search(pattern, m.group(1)):
            end = next(j for j in range(i, len(lines)) if lines[j].startswith(".Lfunc_end"))
            out[m.group(1)] = [x.strip() for x in lines[i + 1:end]]
    return out


@pytest.fixture(scope="module")
def quant_asm():
    return _compile("kvq_quant_kivi.hip")


@pytest.fixture(scope="module")
def decode_asm():
    return _compile("kvq_decode_mfma.hip")


def test_kivi_quantizer_stores_are_non_temporal(quant_asm):
    """Every global store of the KIVI quantize kernels is non-temporal, except
    the 16-byte copies of an appended token into the FP16 window (read by the
    next decode)."""
    kernels = _kernels(quant_asm, r"kivi_quantize_kernel")
    assert len(kernels) >= 12
    for name, body in kernels.items():
        stores = [x for x in body if x.startswith("global_store")]
        plain = [x for x in stores if not x.endswith(" nt")]
        assert all(x.startswith("global_store_dwordx4") for x in plain), (name[:60], plain)
        assert len(stores) - len(plain) >= 5, (name[:60], stores)


def test_paged_decode_reads_its_table_with_scalar_loads(decode_asm):
    """In the paged KIVI decode kernels no vector load feeds the per-tile
    source computation: every `global_load_dword` (the only width a table
    entry would take) belongs to the window or the query, before the ring's
    steady-state loop, and the loop waits on `vmcnt` only with the ring's own
    counts (never `vmcnt(0)`) while copies are in flight."""
    kernels = _kernels(decode_asm, r"kivi_mfma_split_kernelILi\dELi\dELi\dELb\dELb1E")
    assert kernels, "paged decode instances"
    for name, body in kernels.items():
        loops = _loop_bodies(body)
        ring = [b for b in loops.values() if any(x.startswith("global_load_lds") for x in b)]
        assert ring, name[:60]
        for loop in ring:
            assert not any(re.match(r"global_load_dword\b", x) for x in loop), name[:60]
            assert "s_waitcnt vmcnt(0)" not in loop, name[:60]


def _loop_bodies(body):
    """Instructions of each loop, keyed by its header block: the blocks the
    compiler's comments place in that loop (rotated loops put some of them
    before the header)."""
    loops, cur = {}, None
    for x in body:
        m = re.match(r"^(\.LBB\w+):", x)
        if m:
            h = re.search(r"Header=(BB\w+)", x)
            cur = ("." + "L" + h.group(1)) if h else (m.group(1) if "Loop Header" in x else None)
            continue
        if cur is not None and x and not x.startswith((";", ".")):
            loops.setdefault(cur, []).append(x)
    return loops
