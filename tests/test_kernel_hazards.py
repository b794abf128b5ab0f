"""Static check of the gfx950 device code for MFMA data hazards around
inline asm.

The compiler inserts the wait states that matrix instructions need between
instructions it generated itself, but not around inline asm: an MFMA written
as asm can read an operand that a VALU instruction has just written, or have
its result read before the matrix core has written it, with no error and wrong
numbers. The scan compiles each kernel source to device assembly and checks
every pair in which an MFMA and an inline-asm instruction meet, against the
wait states the compiler itself emits for builtin MFMAs on gfx950:
  R1  a VALU write of a VGPR/AGPR that an asm MFMA reads (A, B or C) is
      followed by at least 2 wait states before that MFMA issues;
  R2  the result registers of an MFMA are not read or written by another
      instruction (VALU, LDS, memory, an MFMA's A or B operand), where one of
      the two is asm, within 12 wait states of a 32x32 MFMA (8 passes) or 8 of
      a 16x16 one (4 passes);
  R3  the result of a transcendental VALU instruction (exp, log, rcp, rsq,
      sqrt, sin, cos) is not read by an inline-asm instruction before one
      wait state has passed (gfx950 needs one before any VALU consumer; the
      compiler inserts it only in front of its own instructions).
Wait states: one per instruction in between, n + 1 for `s_nop n`. An MFMA
taking the previous one's result as its accumulator is forwarded by the
hardware and exempt. The scan follows the text of the assembly (a straight-line
approximation of each basic block's predecessor); it is a guard against the
register allocator moving an asm operand, not a proof.
"""

import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "mla_latent_kv_amd", "csrc")

R1_WAIT = 2


def _r2_wait(op):
    return 12 if "32x32" in op else 8


_REG = re.compile(r"^([va])(?:\[(\d+):(\d+)\]|(\d+))$")


def _regs(tok):
    m = _REG.match(tok.strip())
    if not m:
        return set()
    base = 0 if m.group(1) == "v" else 1 << 16
    if m.group(4) is not None:
        return {base + int(m.group(4))}
    return {base + i for i in range(int(m.group(2)), int(m.group(3)) + 1)}


def _instructions(text):
    """(opcode, operands, line, from inline asm) per instruction."""
    out = []
    in_asm = False
    for line in text.splitlines():
        if ";;#ASMSTART" in line:
            in_asm = True
            continue
        if ";;#ASMEND" in line:
            in_asm = False
            continue
        s = line.split(";")[0].strip()
        if not s or s.startswith(".") or s.endswith(":"):
            continue
        op, _, rest = s.partition(" ")
        operands = [o for o in (x.strip() for x in rest.split(",")) if o]
        out.append((op, operands, s, in_asm))
    return out


def _waits(op, operands):
    if op == "s_nop":
        return int(operands[0], 0) + 1
    return 1


def _is_mfma(op):
    return op.startswith("v_mfma") or op.startswith("v_smfmac")


def _is_valu(op):
    return op.startswith("v_") and not _is_mfma(op)


_TRANS = re.compile(r"^v_(exp|log|rcp|rcp_iflag|rsq|sqrt|sin|cos)_(f32|f16)")


def scan(text):
    """List of hazard descriptions for the device assembly `text`."""
    ins = _instructions(text)
    found = []
    for k, (op, ops, line, asm) in enumerate(ins):
        # R3: a transcendental's result read by the next instruction, in asm
        if _TRANS.match(op) and ops and k + 1 < len(ins):
            nop_, nops, nline, nasm = ins[k + 1]
            if nasm and _is_valu(nop_) and any(_regs(o) & _regs(ops[0]) for o in nops[1:]):
                found.append(f"R3: '{line}' then '{nline}' after 0 wait states")
        if not _is_mfma(op) or len(ops) < 4:
            continue
        dst = _regs(ops[0])
        src = _regs(ops[1]) | _regs(ops[2]) | _regs(ops[3])
        # R1: look back over the last R1_WAIT wait states
        ws = 0
        for j in range(k - 1, -1, -1) if asm else ():
            pop, pops, pline, _ = ins[j]
            if _is_valu(pop) and pops and (_regs(pops[0]) & src):
                found.append(f"R1: '{pline}' then '{line}' after {ws} wait states")
                break
            ws += _waits(pop, pops)
            if ws >= R1_WAIT or pop == "s_endpgm":
                break
        # R2: look ahead over the result's latency
        ws, need = 0, _r2_wait(op)
        for j in range(k + 1, len(ins)):
            nop_, nops, nline, nasm = ins[j]
            if nop_ == "s_endpgm":
                break
            if _is_mfma(nop_):
                if len(nops) >= 4 and _regs(nops[0]) == dst and _regs(nops[3]) == dst:
                    break   # accumulation chain: the next MFMA takes over the result
                if (asm or nasm) and any(_regs(o) & dst for o in nops[1:3]):
                    found.append(f"R2: '{line}' then MFMA operand '{nline}' after {ws}")
                    break
                ws += 1
            else:
                if not nop_.startswith("s_") and any(_regs(o) & dst for o in nops):
                    if asm or nasm:
                        found.append(f"R2: '{line}' then '{nline}' after {ws} wait states")
                    break
                ws += _waits(nop_, nops)
            if ws >= need:
                break
    return found


def _device_asm(src, tmp_path):
    from mla_latent_kv_amd import build
    out = tmp_path / (os.path.splitext(src)[0] + ".s")
    flags = [f for f in build.FLAGS if f != "-fPIC"]
    cmd = [build.hipcc(), *flags, "--cuda-device-only", "-S", os.path.join(CSRC, src), "-o", str(out)]
    res = subprocess.run(cmd, capture_output=True, text=True)
    assert res.returncode == 0, res.stderr[-2000:]
    return out.read_text()


def test_scan_finds_planted_hazards():
    # an asm MFMA reading a VALU result one instruction old, and its own result
    # read 4 wait states later; the same code from the compiler is its own
    # responsibility
    bad = """
        v_mov_b32_e32 v5, v0
        ;;#ASMSTART
        v_mfma_f32_32x32x16_f16 v[8:23], v[2:5], v[24:27], v[8:23]
        ;;#ASMEND
        s_nop 3
        v_add_f32_e32 v0, v9, v1
        s_endpgm
    """
    hz = scan(bad)
    assert any(h.startswith("R1") for h in hz) and any(h.startswith("R2") for h in hz)
    assert len(scan(bad.replace(";;#ASMSTART", "").replace(";;#ASMEND", ""))) == 0
    ok = """
        v_mov_b32_e32 v5, v0
        s_nop 1
        ;;#ASMSTART
        v_mfma_f32_32x32x16_f16 v[8:23], v[2:5], v[24:27], v[8:23]
        ;;#ASMEND
        ;;#ASMSTART
        v_mfma_f32_32x32x16_bf16 v[8:23], v[2:5], v[24:27], v[8:23]
        ;;#ASMEND
        s_nop 11
        v_add_f32_e32 v0, v9, v1
        s_endpgm
    """
    assert scan(ok) == []
    # a builtin MFMA result read by an asm accumulator move too early
    late = """
        v_mfma_f32_32x32x16_f16 a[0:15], v[2:5], v[24:27], a[0:15]
        s_nop 7
        ;;#ASMSTART
        v_accvgpr_read_b32 v1, a3
        ;;#ASMEND
        s_endpgm
    """
    assert any(h.startswith("R2") for h in scan(late))
    # a transcendental's result read at once by an asm conversion (wrong
    # values on the GPU); one instruction in between is enough
    trans = """
        v_exp_f32_e32 v9, v9
        ;;#ASMSTART
        v_cvt_pk_f16_f32 v6, v6, v9
        ;;#ASMEND
        s_endpgm
    """
    assert any(h.startswith("R3") for h in scan(trans))
    assert scan(trans.replace(";;#ASMSTART", "s_nop 0\n        ;;#ASMSTART")) == []


@pytest.mark.parametrize("src", ["attn.hip", "prep.hip", "prep_wide.hip", "merge.hip", "naive.hip"])
def test_no_mfma_hazards(src, tmp_path):
    hz = scan(_device_asm(src, tmp_path))
    assert hz == [], "\n".join(hz[:20])
