"""Wait states the hardware does not interlock, checked in disassembled gfx950 code.

Some instructions must be separated from a later one that uses their result by
a number of other instructions (wait states); the compiler inserts s_nop where
too few are left, but its search can miss a path through a branch.  This module
checks the code of the library itself: for every producer below it follows every
control-flow path forward and reports a consumer that comes too early.  A path
ends at the consumer, once the wait states are met, or where another
instruction overwrites the producer's result.

Wait states: s_nop N counts N + 1, any other instruction 1 (a branch too).  The
required counts are the ones the compiler itself leaves in straight-line code
(small kernels of each shape, built for gfx950):

  producer                               consumer                                   wait states
  v_mfma_f32_16x16x32_bf16 (its result)  any instruction touching it, except a       8
  v_mfma_f32_32x32x16_bf16               later MFMA that only accumulates into it    12
  transcendental VALU (v_exp_f32, ...)   a VALU instruction reading the result       1
  VALU writing a VGPR                    a DPP instruction reading it                2
  VALU writing a VGPR                    v_permlane16/32_swap reading it             2
  v_readlane / v_readfirstlane (SGPR)    a VALU instruction reading that SGPR        2
  v_readlane / v_readfirstlane (SGPR)    v_readlane / v_writelane lane select        4

Input: llvm-objdump -d text, whose lines carry each instruction's address
(`// 0000000021A8: ...`) and, for a branch, the target as `<symbol+0xOFF>`.
"""
from __future__ import annotations

import re

MFMA_WAITS = {
    "v_mfma_f32_16x16x32_bf16": 8,
    "v_mfma_f32_32x32x16_bf16": 12,
}
TRANS = ("v_exp_", "v_log_", "v_rcp_", "v_rsq_", "v_sqrt_", "v_sin_", "v_cos_")

_REG = re.compile(r"\b([vas])(?:\[(\d+):(\d+)\]|(\d+)(?!\w))")
_FUNC = re.compile(r"^([0-9a-fA-F]+) <([^>]+)>:")
_ADDR = re.compile(r"//\s*([0-9a-fA-F]+):")
_TARGET = re.compile(r"<([^>+]+)\+0x([0-9a-fA-F]+)>")
_DPP = re.compile(r"\b(row_\w+|quad_perm|wave_\w+)\b")


def registers(operands: str):
    """(kind, first, last) of every VGPR / AGPR / SGPR operand, in order."""
    out = []
    for m in _REG.finditer(operands):
        first = int(m.group(4) if m.group(4) is not None else m.group(2))
        last = int(m.group(4) if m.group(4) is not None else m.group(3))
        out.append((m.group(1), first, last))
    return out


def _overlap(a, b) -> bool:
    return a[0] == b[0] and a[1] <= b[2] and b[1] <= a[2]


def functions(text: str):
    """[(name, [(address, opcode, operands, branch target address or None)])]."""
    funcs, cur, base = [], None, 0
    for line in text.splitlines():
        m = _FUNC.match(line)
        if m:
            base = int(m.group(1), 16)
            cur = (m.group(2), [])
            funcs.append(cur)
            continue
        if cur is None or "//" not in line:
            continue
        code, _, comment = line.partition("//")
        code = code.strip()
        a = _ADDR.search(line)
        if not code or not a:
            continue
        op, _, rest = code.partition(" ")
        target = None
        if op == "s_branch" or op.startswith("s_cbranch"):
            t = _TARGET.search(comment)
            if t and t.group(1) == cur[0]:
                target = base + int(t.group(2), 16)
        cur[1].append((int(a.group(1), 16), op, rest.strip(), target))
    return funcs


def _valu_sources(op: str, regs):
    """Registers a VALU instruction reads (all but the destination; a VOPC
    compare in its 32-bit form has no register destination)."""
    if op.startswith("v_cmp") and op.endswith("_e32"):
        return regs
    return regs[1:]


def _rules(op: str, arg: str):
    """(name, hazard register, wait states, consumer test) for each hazard the
    instruction opens; the test takes (opcode, operands, registers) and says
    whether that instruction consumes the register too early."""
    regs = registers(arg)
    if not regs or not op.startswith("v_"):
        return []
    dst = regs[0]
    if op.startswith("v_mfma"):
        if op not in MFMA_WAITS:
            raise ValueError(f"no wait-state count for {op}")

        def mfma_use(op2, arg2, regs2):
            touched = regs2[1:3] if op2.startswith("v_mfma") else regs2
            return any(_overlap(dst, r) for r in touched)
        return [("mfma", dst, MFMA_WAITS[op], mfma_use)]
    out = []
    if op.startswith(("v_readlane", "v_readfirstlane")) and dst[0] == "s":
        def sgpr_valu(op2, arg2, regs2):
            return op2.startswith("v_") and any(_overlap(dst, r) for r in _valu_sources(op2, regs2))

        def sgpr_lane(op2, arg2, regs2):
            return op2.startswith(("v_readlane", "v_writelane")) and len(regs2) >= 3 and _overlap(dst, regs2[-1])
        out += [("readlane sgpr -> valu", dst, 2, sgpr_valu), ("readlane sgpr -> lane select", dst, 4, sgpr_lane)]
    if dst[0] == "v":
        if op.startswith(TRANS):
            def trans_use(op2, arg2, regs2):
                return op2.startswith("v_") and any(_overlap(dst, r) for r in _valu_sources(op2, regs2))
            out.append(("trans -> valu", dst, 1, trans_use))

        def dpp_use(op2, arg2, regs2):
            return (op2.startswith("v_") and (op2.endswith("_dpp") or _DPP.search(arg2) is not None)
                    and len(regs2) >= 2 and _overlap(dst, regs2[1]))

        def swap_use(op2, arg2, regs2):
            return op2.startswith(("v_permlane16_swap", "v_permlane32_swap")) and any(_overlap(dst, r) for r in regs2)
        out += [("valu -> dpp", dst, 2, dpp_use), ("valu -> permlane swap", dst, 2, swap_use)]
    return out


def short_waits(text: str, only: str | None = None):
    """Every (function, rule, producer text, consumer text, wait states, required)
    where a consumer comes too early on some path (rules whose name starts with
    `only`, if given)."""
    found = []
    for name, ins in functions(text):
        at = {addr: i for i, (addr, _, _, _) in enumerate(ins)}

        def successors(i):
            _, op, _, target = ins[i]
            nxt = [i + 1] if i + 1 < len(ins) else []
            if op == "s_branch":
                return [at[target]] if target in at else []
            if op.startswith("s_cbranch"):
                return ([at[target]] if target in at else []) + nxt
            if op in ("s_endpgm", "s_setpc_b64"):
                return []
            return nxt

        for i, (_, op, arg, _) in enumerate(ins):
            for rule, reg, need, consumes in _rules(op, arg):
                if only is not None and not rule.startswith(only):
                    continue
                best = {}  # instruction -> the most wait states still needed when reached
                todo = [(k, 0) for k in successors(i)]
                while todo:
                    j, w = todo.pop()
                    if w >= need or best.get(j, -1) >= need - w:
                        continue
                    best[j] = need - w
                    _, op2, arg2, _ = ins[j]
                    regs2 = registers(arg2)
                    if consumes(op2, arg2, regs2):
                        found.append((name, rule, f"{op} {arg}", f"{op2} {arg2}", w, need))
                        continue
                    if rule != "mfma" and op2.startswith("v_") and regs2 and _overlap(reg, regs2[0]) \
                            and not (op2.startswith("v_cmp") and op2.endswith("_e32")):
                        continue  # overwritten: later readers see the new value
                    cost = int(arg2, 0) + 1 if op2 == "s_nop" else 1
                    todo.extend((k, w + cost) for k in successors(j))
    return found
