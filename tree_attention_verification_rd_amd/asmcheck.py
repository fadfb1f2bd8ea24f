"""Build-time check of the explicitly scheduled load rings in the gfx950 assembly.

Stream loads that the kernels issue through inline asm (invisible to the
compiler's wait tracking) write their destination VGPRs some time after
issue.  If the compiler hands one of those registers to other code before
the explicit wait, the landing load corrupts it.  This walks each kernel's
assembly, keeps the set of VGPRs with an inline-asm buffer load in flight
(retired by s_waitcnt vmcnt(N), in issue order), visits every loop body
twice so back-edges are covered, and reports any instruction that reads or
writes such a register.  Loads the compiler schedules itself are ignored:
it inserts their waits.
"""
from __future__ import annotations

import re
import subprocess
import sys

_VREG = re.compile(r"\bv\[(\d+):(\d+)\]|\bv(\d+)\b")


def _regs(text: str) -> set:
    out = set()
    for m in _VREG.finditer(text):
        if m.group(3) is not None:
            out.add(int(m.group(3)))
        else:
            out.update(range(int(m.group(1)), int(m.group(2)) + 1))
    return out


def _visit_order(code: list) -> list:
    labels = {c.strip()[:-1]: i for i, c in enumerate(code) if re.match(r"^\.LBB\w+:$", c.strip())}
    order, taken, i = [], set(), 0
    while i < len(code):
        order.append(i)
        m = re.match(r"\s*s_cbranch_\w+\s+(\.LBB\w+)", code[i])
        if m and m.group(1) in labels and labels[m.group(1)] < i and i not in taken:
            taken.add(i)  # walk the loop body a second time
            i = labels[m.group(1)]
            continue
        i += 1
    return order


def check_kernel(lines: list) -> list:
    code, in_asm = [], []
    inside = False
    for raw in lines:
        s = raw.strip()
        if s.startswith(";;#ASMSTART"):
            inside = True
        elif s.startswith(";;#ASMEND"):
            inside = False
        code.append(raw.split(";")[0].rstrip())
        in_asm.append(inside)
    inflight, problems = [], []
    for i in _visit_order(code):
        ins = code[i].strip()
        if not ins or ins.startswith(".") or ins.endswith(":"):
            continue
        op = ins.split()[0]
        operands = ins[len(op):]
        if op == "s_waitcnt" and "vmcnt" in ins:
            n = int(re.search(r"vmcnt\((\d+)\)", ins).group(1))
            inflight = inflight[len(inflight) - n:] if 0 < n < len(inflight) else ([] if n == 0 else inflight)
            continue
        touched = _regs(operands)
        hits = [ln for ln, rs in inflight if rs & touched]
        if hits:
            problems.append(f"line {i + 1}: '{ins}' touches a register loaded at line {hits[0] + 1}")
        if op.startswith("buffer_load") and in_asm[i]:
            inflight.append((i, _regs(operands.split(",")[0])))
    return problems


def check_assembly(text: str) -> dict:
    lines = text.splitlines()
    out = {}
    for s, line in enumerate(lines):
        m = re.match(r"^(_Z\w+):", line)
        if not m:
            continue
        e = next(j for j in range(s, len(lines)) if "s_endpgm" in lines[j])
        probs = check_kernel(lines[s:e + 1])
        if probs:
            out[m.group(1)] = probs
    return out


def check_source(hipcc: str, flags: list, src: str) -> dict:
    res = subprocess.run([hipcc, *flags, "-S", "--cuda-device-only", src, "-o", "-"], capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"assembly generation failed for {src}:\n{res.stderr}")
    return check_assembly(res.stdout)


if __name__ == "__main__":
    text = open(sys.argv[1]).read()
    found = check_assembly(text)
    for k, v in found.items():
        print(k, *v[:5], sep="\n  ")
    sys.exit(1 if found else 0)
