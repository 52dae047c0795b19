"""Wait-state check of the MFMA-bound kernel's generated gfx950 assembly.

The kernel's accumulate step is an inline-asm MFMA (its accumulators stay in
AGPRs) and its global -> LDS copies are inline asm too, so the compiler's
hazard recognizer does not see them and inserts no wait states around them.
The CDNA3/CDNA4 ISA requires:

* two wait states between a VALU instruction that writes a VGPR/AGPR and an
  MFMA that reads that register as a source (A, B or C);
* more wait states than the MFMA's pipeline depth between the MFMA writing its
  accumulators and any non-MFMA instruction reading them (16x16x32 bf16/f16:
  8 passes; 18 is taken here as the bound, above the 8-pass figure plus the
  extra issue cycles);
* five wait states between a VALU write of an SGPR (v_readfirstlane, a
  compare into an SGPR pair, v_readlane restoring a spilled scalar) and a copy
  reading that SGPR as its base address, unless a scalar instruction writes
  the SGPR again in between (the copy then reads that value).

Whether the scheduler leaves enough independent instructions in between
depends on the instantiation, so the build compiles each form of the kernel's
unit to assembly as well and refuses to link a library in which any of these
is violated; the test suite runs the same walk.
"""
from __future__ import annotations

import re

VALU_TO_MFMA = 2
MFMA_TO_READ = 18
VALU_SGPR_TO_VMEM = 5


def _regs(tok: str):
    tok = tok.strip()
    m = re.match(r"([va])\[(\d+):(\d+)\]$", tok)
    if m:
        return m.group(1), set(range(int(m.group(2)), int(m.group(3)) + 1))
    m = re.match(r"([va])(\d+)$", tok)
    if m:
        return m.group(1), {int(m.group(2))}
    return None, set()


def _kernels(text: str):
    cur, body = None, []
    for line in text.splitlines():
        m = re.match(r"^(_Z\S+):\s*(;.*)?$", line)
        if m:
            cur, body = m.group(1), []
            continue
        if cur is not None and line.startswith(".Lfunc_end"):
            yield cur, body
            cur = None
        elif cur is not None:
            body.append(line)


def _stream(body):
    """Instructions in order as (kind, text, inside_asm); labels kept."""
    out, inasm = [], False
    for ln in body:
        s = ln.strip()
        if s.startswith(";;#ASMSTART"):
            inasm = True
        elif s.startswith(";;#ASMEND"):
            inasm = False
        elif s.startswith(".LBB"):
            out.append(("label", s, inasm))
        elif s and not s.startswith(";") and not s.startswith("."):
            out.append(("inst", s.split(";")[0].strip(), inasm))
    return out


def _sregs(tok: str):
    tok = tok.strip()
    m = re.match(r"s\[(\d+):(\d+)\]$", tok)
    if m:
        return set(range(int(m.group(1)), int(m.group(2)) + 1))
    m = re.match(r"s(\d+)$", tok)
    return {int(m.group(1))} if m else set()


def _wait_states(inst: str) -> int:
    op = inst.split()[0]
    return int(inst.split()[1], 0) + 1 if op == "s_nop" else 1


def _operands(inst: str):
    parts = inst.split(None, 1)
    return [p.strip() for p in parts[1].split(",")] if len(parts) > 1 else []


def _is_valu(op: str) -> bool:
    return op.startswith("v_") and not op.startswith("v_mfma")


# scalar instructions whose first operand is a source, not a destination
_NO_SCALAR_DEST = ("s_cmp", "s_bitcmp", "s_cbranch", "s_branch", "s_waitcnt", "s_nop", "s_barrier", "s_set",
                   "s_sleep", "s_endpgm", "s_sendmsg")


def _sgpr_dest(inst: str):
    """SGPRs the instruction writes (its first operand, where that is a destination)."""
    op, ops = inst.split()[0], _operands(inst)
    if not ops or op.startswith(_NO_SCALAR_DEST):
        return set()
    return _sregs(ops[0])


def hazards(text: str):
    """Every violation of the rules above in the MFMA-bound kernels of one
    assembly listing, as readable strings (empty: none)."""
    found = []
    for name, body in _kernels(text):
        if "k_gemm_mfma" not in name:
            continue
        L = _stream(body)
        for i, (kind, s, inasm) in enumerate(L):
            if kind != "inst":
                continue
            op = s.split()[0]
            if op.startswith("v_mfma") and inasm:
                srcs = [_regs(t) for t in _operands(s)[1:4]]
                ws, j = 0, i - 1
                while j >= 0 and ws < VALU_TO_MFMA:
                    k2, s2, _ = L[j]
                    if k2 == "label":
                        found.append(f"{name}: branch target within {VALU_TO_MFMA} wait states of '{s}'")
                        break
                    if _is_valu(s2.split()[0]):
                        dst = _regs(_operands(s2)[0]) if _operands(s2) else (None, set())
                        if any(f == dst[0] and r & dst[1] for f, r in srcs):
                            found.append(f"{name}: '{s2}' {ws} wait states before '{s}'")
                    ws += _wait_states(s2)
                    j -= 1
            elif op.startswith("global_load_lds") and inasm:
                used = set().union(*[_sregs(t) for t in _operands(s)])
                ws, j = 0, i - 1
                while j >= 0 and ws < VALU_SGPR_TO_VMEM and used:
                    k2, s2, _ = L[j]
                    if k2 == "label":
                        found.append(f"{name}: branch target within {VALU_SGPR_TO_VMEM} wait states of '{s}'")
                        break
                    dst = _sgpr_dest(s2)
                    if _is_valu(s2.split()[0]) and dst & used:
                        found.append(f"{name}: '{s2}' {ws} wait states before '{s}'")
                    used -= dst   # an earlier write of these no longer reaches the copy
                    ws += _wait_states(s2)
                    j -= 1
            elif not op.startswith("v_mfma") and any(_regs(t)[0] == "a" for t in _operands(s)):
                reads = [_regs(t) for t in _operands(s)[1:] if _regs(t)[0] == "a"]
                if op.startswith("v_accvgpr_write") or not reads:
                    continue
                ws, j = 0, i - 1
                while j >= 0 and ws < MFMA_TO_READ:
                    k2, s2, in2 = L[j]
                    if k2 == "inst" and s2.startswith("v_mfma"):
                        dst = _regs(_operands(s2)[0])
                        if any(r & dst[1] for _, r in reads):
                            found.append(f"{name}: '{s}' {ws} wait states after '{s2}'")
                            break
                    if k2 == "inst":
                        ws += _wait_states(s2)
                    j -= 1
    return found


def inline_ops(text: str):
    """Opcodes of the inline-asm instructions of the MFMA-bound kernels."""
    return [s.split()[0] for name, body in _kernels(text) if "k_gemm_mfma" in name
            for k, s, a in _stream(body) if k == "inst" and a]
