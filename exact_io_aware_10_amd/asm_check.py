"""Build-time check of the kernels' inline-assembly MFMAs.

Some MFMAs in the kernels are written as inline assembly (accumulators kept
in VGPRs or AGPRs against the compiler's own choice).  The compiler's hazard
recognizer does not look inside inline assembly, so nothing stops the
register allocator from placing a copy of such an MFMA's result right after
it, before the matrix core has written the result; nor does anything stop it
from overwriting the registers such an MFMA reads as its accumulator input
(srcC) while the matrix core is still reading them.  The kernels bracket those
MFMAs with fences; this check verifies the generated code: no instruction may
read or overwrite the destination registers of an inline-assembly MFMA, nor
write its srcC registers, within MIN_WAIT wait states of it (an 8-pass 32x32
MFMA needs about 11 for the first and fewer for the second).

A second rule covers loads written as inline assembly: the compiler does not
know such an instruction is a load whose data arrives later, so it inserts no
wait before the destination registers are used, and it may copy them (a
spill into AGPRs, say) the moment the statement ends.  A load into registers
(as opposed to an LDS-direct load, which names no destination register) must
therefore be an ordinary, compiler-visible load.

Usage: python -m exact_io_aware_10_amd.asm_check FILE.s ...
"""
from __future__ import annotations

import re
import sys

MIN_WAIT = 12

_RANGE = re.compile(r"([av])\[(\d+):(\d+)\]")
_SINGLE = re.compile(r"([av])(\d+)$")


def _regs(tok: str) -> set:
    m = _RANGE.fullmatch(tok)
    if m:
        return {(m.group(1), i) for i in range(int(m.group(2)), int(m.group(3)) + 1)}
    m = _SINGLE.fullmatch(tok)
    if m:
        return {(m.group(1), int(m.group(2)))}
    return set()


def _parse(text: str):
    insts, in_asm = [], False
    for ln, line in enumerate(text.split("\n"), 1):
        if ";;#ASMSTART" in line:
            in_asm = True
        elif ";;#ASMEND" in line:
            in_asm = False
        body = line.split(";")[0].strip()
        if not body or body.startswith(".") or body.endswith(":"):
            continue
        parts = body.replace(",", " ").split()
        insts.append((ln, parts[0], parts[1:], in_asm))
    return insts


def _written(op: str, ops: list) -> set:
    """VGPRs / AGPRs an instruction writes (its first operand, where that is a
    destination: VALU and MFMA results, LDS and buffer loads into registers)."""
    if not ops:
        return set()
    if op.startswith("v_") or op.startswith(("ds_read", "ds_load")) or (
            op.startswith(("buffer_load", "global_load", "flat_load", "scratch_load"))
            and "lds" not in ops):
        return _regs(ops[0])
    return set()


def check(text: str, min_wait: int = MIN_WAIT) -> list[str]:
    """Return one message per early access to an inline-asm MFMA's result,
    early overwrite of its srcC registers, or inline-asm load into registers."""
    insts = _parse(text)
    problems = []
    for idx, (ln, op, ops, in_asm) in enumerate(insts):
        if in_asm and op.startswith(("buffer_load", "global_load", "flat_load", "scratch_load",
                                     "ds_read", "ds_load")) and _written(op, ops):
            problems.append(f"line {ln}: {op} {' '.join(ops)} loads into registers from inline "
                            f"assembly (the compiler cannot wait for it)")
            continue
        if not (in_asm and op.startswith("v_mfma")):
            continue
        dst = _regs(ops[0])
        srcc = _regs(ops[3]) - dst if len(ops) > 3 else set()
        waited = 0
        for ln2, op2, ops2, _ in insts[idx + 1:]:
            waited += int(ops2[0], 0) + 1 if op2 == "s_nop" else 1
            if waited > min_wait or op2.startswith(("s_branch", "s_cbranch", "s_endpgm", "s_setpc")):
                break
            touched = set()
            for tok in ops2:
                touched |= _regs(tok)
            if srcc & _written(op2, ops2):
                problems.append(f"line {ln}: {op} srcC {ops[3]} is overwritten {waited} wait states "
                                f"later at line {ln2}: {op2} {' '.join(ops2)}")
                break
            if op2.startswith("v_mfma") and _regs(ops2[0]) == dst and ops2[3:4] == [ops[0]]:
                continue  # accumulation chain into the same registers: forwarded
            if dst & touched:
                problems.append(f"line {ln}: {op} {ops[0]} is accessed {waited} wait states "
                                f"later at line {ln2}: {op2} {' '.join(ops2)}")
                break
    return problems


def main(argv: list[str]) -> int:
    bad = 0
    for path in argv:
        with open(path) as f:
            for msg in check(f.read()):
                print(f"{path}: {msg}")
                bad += 1
    return 1 if bad else 0


if __name__ == "__main__":
    sys.exit(main(sys.argv[1:]))
