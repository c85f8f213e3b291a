"""Generated-code check of the decode kernels (compiles only; no GPU).

A matrix-core instruction (v_mfma_*) must not read a VGPR within two wait
states of the VALU instruction that wrote it. The compiler pads its own
instructions, but not instructions hidden in inline asm, and a violation
feeds the MFMA the register's previous contents (one accumulator tile of the
KIVI decode came out as garbage that way). This test compiles
kvq_decode_mfma.hip for gfx950 with the library's flags and checks, in every
kernel, that each MFMA's A and B operands were written at least two wait
states (instructions or s_nop slots) earlier, and likewise the DPP-read
operand of every DPP instruction.
"""
import os
import re
import subprocess

import pytest

from kv_cache_quantization_quant_amd import build as kbuild

SRC = os.path.join(kbuild.CSRC, "kvq_decode_mfma.hip")


def _regs(tok):
    m = re.match(r"v\[(\d+):(\d+)\]", tok)
    if m:
        return set(range(int(m.group(1)), int(m.group(2)) + 1))
    m = re.match(r"v(\d+)$", tok)
    return {int(m.group(1))} if m else set()


def _kernels(asm):
    lines = asm.splitlines()
    out = {}
    for i, line in enumerate(lines):
        m = re.match(r"^(_Z\w+_kernel\w*):", line)
        if m:
            end = next(j for j in range(i, len(lines)) if lines[j].startswith(".Lfunc_end"))
            out[m.group(1)] = [x.strip() for x in lines[i + 1:end]]
    return out


def _operand_gaps(body):
    """(gap, mfma, producer) for each MFMA whose A/B operand a VALU wrote
    fewer than 4 slots earlier (straight-line look-back)."""
    found = []
    for i, t in enumerate(body):
        if not t.startswith("v_mfma"):
            continue
        ops = [o.strip(",") for o in t.split()[1:5]]
        src = _regs(ops[1]) | _regs(ops[2])
        k, slots = i - 1, 0
        while k >= 0 and slots < 4:
            u = body[k]
            if u.startswith(".LBB") or u.startswith("s_cbranch") or u.startswith("s_branch"):
                break                                   # block boundary: stop looking
            if u and not u.startswith((".", ";")):
                if u.startswith("s_nop"):
                    slots += int(u.split()[1]) + 1
                else:
                    if u.startswith("v_") and not u.startswith("v_mfma"):
                        if _regs(u.split()[1].strip(",")) & src:
                            found.append((slots, t, u))
                            break
                    slots += 1
            k -= 1
    return found


@pytest.fixture(scope="module")
def decode_asm(tmp_path_factory):
    out = tmp_path_factory.mktemp("asm") / "dec.s"
    cmd = [kbuild.HIPCC, *[f for f in kbuild.COMMON if f != "-fPIC"],
           *kbuild.EXTRA.get(os.path.basename(SRC), []), "--cuda-device-only", "-S",
           "-x", "hip", SRC, "-o", str(out)]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    return out.read_text()


def test_every_mfma_operand_has_two_wait_states(decode_asm):
    kernels = _kernels(decode_asm)
    assert any("kivi_mfma_split_kernel" in k for k in kernels)
    assert any("dense_mfma_split_kernel" in k for k in kernels)
    bad = []
    for name, body in kernels.items():
        for gap, mfma, producer in _operand_gaps(body):
            if gap < 2:
                bad.append(f"{name[:60]}: {producer} -> {mfma} ({gap} wait states)")
    assert not bad, "\n".join(bad[:10])


def _dpp_gaps(body):
    """(gap, dpp, producer) for each DPP instruction whose DPP-read source
    (src0) a VALU instruction wrote fewer than 2 slots earlier."""
    found = []
    for i, t in enumerate(body):
        if not (t.startswith("v_") and "_dpp" in t.split()[0]):
            continue
        ops = [o.strip(",") for o in t.split()[1:3]]
        src = _regs(ops[1])
        k, slots = i - 1, 0
        while k >= 0 and slots < 2:
            u = body[k]
            if u.startswith(".LBB") or u.startswith("s_cbranch") or u.startswith("s_branch"):
                break
            if u and not u.startswith((".", ";")):
                if u.startswith("s_nop"):
                    slots += int(u.split()[1]) + 1
                else:
                    if u.startswith("v_") and _regs(u.split()[1].strip(",")) & src:
                        found.append((slots, t, u))
                        break
                    slots += 1
            k -= 1
    return found


def test_every_dpp_read_has_two_wait_states(decode_asm):
    """A DPP operand read of a VGPR needs two wait states after the VALU
    write of it; the compiler pads only its own instructions."""
    bad = []
    for name, body in _kernels(decode_asm).items():
        for gap, dpp, producer in _dpp_gaps(body):
            bad.append(f"{name[:60]}: {producer} -> {dpp} ({gap} wait states)")
    assert not bad, "\n".join(bad[:10])


def test_inline_asm_valu_is_padded_in_decode_source():
    """Inline asm in the decode kernels that holds VALU instructions (the
    DPP half swaps) opens and closes with two wait states (s_nop 1), since the
    compiler does not pad around instructions it did not emit."""
    src = open(SRC).read()
    bodies = re.findall(r'asm(?:\s+volatile)?\s*\((.*?)\)\s*;', src, re.S)
    valu = [b for b in bodies if re.search(r'"\s*v_', b)]
    assert valu, "the half swaps are inline asm"
    for b in valu:
        lits = []
        for lit in re.findall(r'"((?:[^"\\]|\\.)*)"', b):
            if re.fullmatch(r"[=&+]*[a-z]", lit):     # first operand constraint
                break
            lits.append(lit)
        text = "".join(lits).replace("\\n", "\n").replace("\\t", "")
        instrs = [x.strip() for x in text.split("\n") if x.strip()]
        assert instrs[0] == "s_nop 1" and instrs[-1] == "s_nop 1", instrs


def test_inline_asm_keeps_scc_in_decode_source():
    """The scalar instructions in the decode kernels' inline asm are moves,
    nops and waits only: the compiler may keep a branch condition in SCC
    across an asm block, and SALU arithmetic or logic (s_not, s_and, s_add...)
    would overwrite it."""
    src = open(SRC).read()
    bodies = re.findall(r'asm(?:\s+volatile)?\s*\((.*?)\)\s*;', src, re.S)
    allowed = {"s_mov_b32", "s_mov_b64", "s_nop", "s_waitcnt"}
    for b in bodies:
        for lit in re.findall(r'"((?:[^"\\]|\\.)*)"', b):
            for ins in lit.replace("\\n", "\n").replace("\\t", "").split("\n"):
                op = ins.strip().split(" ")[0] if ins.strip() else ""
                if op.startswith("s_"):
                    assert op in allowed, f"SCC-writing scalar instruction in inline asm: {ins}"
    # the KVQ_COPY_* macros hold the copy instructions
    for m in re.findall(r'#define KVQ_\w+\s+(.*)', src):
        for op in re.findall(r'\b(s_[a-z0-9_]+)', m):
            assert op in allowed, op
