"""Static check of the library's gfx950 device assembly for MFMA results read
too early.

A matrix instruction writes its destination registers several cycles after it
issues, and the hardware does not hold back a later vector, memory or LDS
instruction that reads them: the compiler pads such reads with independent
instructions or s_nop.  It does so along straight-line code, but a read at
the head of a block reached by a branch straight from the MFMA has been left
unpadded (a store read the old register contents, intermittently).  This
module follows every control-flow path forward from each MFMA and reports a
read of its destination that comes fewer wait states after it than the
compiler itself inserts in straight-line code for that instruction.

Wait states along a path: 1 per instruction, N + 1 for s_nop N, and for a
later MFMA its pass count (it cannot issue before the matrix pipe has taken
the earlier one).  A path stops following a register once an instruction
rewrites it.  Usage: python -m mamba_ssd_selective_amd.isa_check [FILE.s ...]
(no argument: compile every kernel source to device assembly and check it).
"""
from __future__ import annotations

import os
import re
import subprocess
import sys
import tempfile
from typing import Dict, List, Set, Tuple

# passes of each matrix instruction the kernels use, and the wait states the
# compiler puts between it and a non-MFMA read of its result in straight-line
# code on gfx950
PASSES = {"v_mfma_f32_16x16x32_bf16": 4, "v_mfma_f32_16x16x4_f32": 8}
NEED = {"v_mfma_f32_16x16x32_bf16": 8, "v_mfma_f32_16x16x4_f32": 10}

_REG = re.compile(r"\b([va])\[(\d+):(\d+)\]|\b([va])(\d+)\b")
# instructions whose operands are all read (no destination register)
_STORES = ("global_store", "buffer_store", "flat_store", "ds_write", "ds_store")

Reg = Tuple[str, int]


def _regs(text: str) -> Set[Reg]:
    out: Set[Reg] = set()
    for m in _REG.finditer(text):
        if m.group(5):
            out.add((m.group(4), int(m.group(5))))
        else:
            out.update((m.group(1), r) for r in range(int(m.group(2)), int(m.group(3)) + 1))
    return out


def _functions(lines: List[str]) -> Dict[str, List[Tuple[int, str]]]:
    """function symbol -> [(line number, instruction or label)]"""
    funcs: Dict[str, List[Tuple[int, str]]] = {}
    cur = None
    for no, raw in enumerate(lines, 1):
        m = re.match(r"^(_Z\w+):", raw)
        if m:
            cur = m.group(1)
            funcs[cur] = []
            continue
        if cur is None:
            continue
        s = raw.split(";")[0].strip()
        if not s:
            continue
        if s.startswith(".Lfunc_end"):
            cur = None
            continue
        if s.startswith(".") and not s.startswith(".LBB"):
            continue
        funcs[cur].append((no, s))
    return funcs


def check_asm(text: str) -> List[str]:
    """Findings (one line each) for the assembly text of one object."""
    found: List[str] = []
    for fn, ins in _functions(text.splitlines()).items():
        label = {s[:-1]: k for k, (_, s) in enumerate(ins) if s.endswith(":")}
        for k, (no, s) in enumerate(ins):
            op = s.split()[0]
            if not op.startswith("v_mfma"):
                continue
            need = NEED.get(op)
            if need is None:
                found.append("%s: line %d: no wait-state figure for %s" % (fn, no, op))
                continue
            start = frozenset(_regs(s[len(op):].split(",")[0]))
            stack = [(k + 1, 0, start)]
            seen = set()
            while stack:
                j, ws, live = stack.pop()
                if not live or ws >= need or j >= len(ins) or (j, ws, live) in seen:
                    continue
                seen.add((j, ws, live))
                no2, s2 = ins[j]
                if s2.endswith(":"):
                    stack.append((j + 1, ws, live))
                    continue
                op2 = s2.split()[0]
                if op2 == "s_endpgm":
                    continue
                args = s2[len(op2):]
                parts = [p.strip() for p in args.split(",")]
                if op2.startswith("v_mfma"):
                    # A / B operands must wait; C is forwarded to a dependent MFMA
                    if _regs(",".join(parts[1:3])) & live:
                        found.append("%s: line %d %s -> line %d %s (%d wait states, needs %d)"
                                     % (fn, no, s, no2, s2, ws, need))
                        continue
                    live = frozenset(live - _regs(parts[0]))
                    step = PASSES.get(op2, 1)
                else:
                    is_store = op2.startswith(_STORES)
                    reads = _regs(args) if is_store else _regs(",".join(parts[1:]))
                    if reads & live:
                        found.append("%s: line %d %s -> line %d %s (%d wait states, needs %d)"
                                     % (fn, no, s, no2, s2, ws, need))
                        continue
                    if not is_store and parts and parts[0]:
                        live = frozenset(live - _regs(parts[0]))
                    step = int(args.strip(), 0) + 1 if op2 == "s_nop" else 1
                if op2 == "s_branch" or op2.startswith("s_cbranch"):
                    target = args.strip()
                    if target in label:
                        stack.append((label[target], ws + step, live))
                    if op2 == "s_branch":
                        continue
                stack.append((j + 1, ws + step, live))
    return found


def device_asm(out_dir: str) -> List[str]:
    """Compile every kernel source of the library to gfx950 device assembly
    with the build's flags; returns the .s paths."""
    from . import _build
    csrc = os.path.join(_build.HERE, "csrc")
    procs, outs = [], []
    for name in sorted(os.listdir(csrc)):
        if not name.endswith(".hip"):
            continue
        out = os.path.join(out_dir, name[:-4] + ".s")
        cmd = [_build.HIPCC, *_build.FLAGS, "-I", os.path.join(_build.HERE, "..", "include"),
               "-c", os.path.join(csrc, name), "-o", out, "--offload-device-only", "-S"]
        procs.append((name, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT)))
        outs.append(out)
    for name, p in procs:
        log = p.communicate()[0].decode(errors="replace")
        if p.returncode != 0:
            raise RuntimeError("device assembly of %s failed:\n%s" % (name, log[-4000:]))
    return outs


def main(argv: List[str]) -> int:
    paths = argv
    tmp = None
    if not paths:
        tmp = tempfile.TemporaryDirectory()
        paths = device_asm(tmp.name)
    n = 0
    for path in paths:
        with open(path) as f:
            for line in check_asm(f.read()):
                print("%s: %s" % (os.path.basename(path), line))
                n += 1
    print("%d finding(s)" % n)
    return 1 if n else 0


if __name__ == "__main__":
    sys.exit(main(sys.argv[1:]))
