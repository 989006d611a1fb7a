"""Wait states after MFMA instructions in disassembled gfx950 code.

The matrix unit does not interlock a later instruction that touches an MFMA's
result registers: the program has to leave a number of other instructions (wait
states) between them, and the compiler puts in s_nop where too few are left.
Its search can miss a path through a branch, so this module checks the code of
the library itself: for every MFMA it follows every control-flow path forward
and reports any instruction that reads or writes the MFMA's destination
registers before the required number of wait states has passed.  A later MFMA
that takes the result as its accumulator (or writes the same registers) is fed
by the unit itself and is not reported; one that takes it as its A or B operand
is.

Wait states: s_nop N counts N + 1, any other instruction 1 (a branch too).  The
required counts are the ones the compiler itself leaves after these MFMAs in
straight-line code before a vector-ALU read of the result.

Input: llvm-objdump -d text, whose lines carry each instruction's address
(`// 0000000021A8: ...`) and, for a branch, the target as `<symbol+0xOFF>`.
"""
from __future__ import annotations

import re

REQUIRED = {
    "v_mfma_f32_16x16x32_bf16": 8,
    "v_mfma_f32_32x32x16_bf16": 12,
}

_REG = re.compile(r"\b([va])(?:\[(\d+):(\d+)\]|(\d+)(?!\w))")
_FUNC = re.compile(r"^([0-9a-fA-F]+) <([^>]+)>:")
_ADDR = re.compile(r"//\s*([0-9a-fA-F]+):")
_TARGET = re.compile(r"<([^>+]+)\+0x([0-9a-fA-F]+)>")


def registers(operands: str):
    """(kind, first, last) of every VGPR / AGPR operand, in order."""
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


def short_waits(text: str):
    """Every (function, MFMA text, consumer text, wait states left, required) where
    an instruction touches an MFMA's result too early on some path."""
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
            if not op.startswith("v_mfma"):
                continue
            if op not in REQUIRED:
                raise ValueError(f"no wait-state count for {op}")
            need = REQUIRED[op]
            dst = registers(arg)[0]
            best = {}  # instruction -> the most wait states still needed when it was reached
            todo = [(k, 0) for k in successors(i)]
            while todo:
                j, w = todo.pop()
                if w >= need or best.get(j, -1) >= need - w:
                    continue
                best[j] = need - w
                _, op2, arg2, _ = ins[j]
                regs2 = registers(arg2)
                touched = regs2[1:3] if op2.startswith("v_mfma") else regs2
                if any(_overlap(dst, r) for r in touched):
                    found.append((name, f"{op} {arg}", f"{op2} {arg2}", w, need))
                    continue
                cost = int(arg2, 0) + 1 if op2 == "s_nop" else 1
                todo.extend((k, w + cost) for k in successors(j))
    return found
