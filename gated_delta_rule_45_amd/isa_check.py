"""Static check of the generated gfx950 assembly: wait states after matrix-core (MFMA) results.

A VALU instruction (or v_accvgpr_read / write, a memory instruction) that reads or overwrites the
destination registers of an MFMA must come a number of wait states after it (8 after a 16x16x32
bf16 product, 10 after a 16x16x4 f32 one: the counts the compiler itself leaves inside a basic
block).  The compiler inserts them inside a block, but it has been seen to leave none where the read
sits in another block reached through a join (wrong values, no fault).  This module
walks every path of the control-flow graph from each MFMA, counting wait states (one per issued
instruction, N + 1 for s_nop N), and reports any access to the MFMA's destination registers before
the count is reached.  Feeding the registers back as the accumulator (src C) of the next MFMA of the
same shape is allowed without wait states, and so is overwriting them with another MFMA.

Usage: python -m gated_delta_rule_45_amd.isa_check [file.s ...]   (default: compile every source)
"""
from __future__ import annotations

import os
import re
import subprocess
import sys
import tempfile
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field

HERE = os.path.dirname(os.path.abspath(__file__))

# Wait states an MFMA result needs before another instruction reads or overwrites it: the counts the
# compiler itself leaves inside a basic block for the shapes used here (the 16x16x32 bf16 product is
# a 4-pass instruction on gfx950, the 16x16x4 f32 one an 8-pass one); unknown shapes get the 16-pass
# count.
def required_wait_states(op: str) -> int:
    if re.search(r"16x16x32_(bf16|f16)", op):
        return 8
    if "16x16x4" in op:
        return 10
    return 18


_REG = re.compile(r"\b([av])\[(\d+):(\d+)\]|\b([av])(\d+)\b")


def regs_of(text: str):
    out = set()
    for m in _REG.finditer(text):
        if m.group(1):
            k, a, b = m.group(1), int(m.group(2)), int(m.group(3))
            out.update((k, i) for i in range(a, b + 1))
        else:
            out.add((m.group(4), int(m.group(5))))
    return out


@dataclass
class Insn:
    op: str
    args: str
    line: int


@dataclass
class Block:
    name: str
    insns: list = field(default_factory=list)
    succ: list = field(default_factory=list)


def parse_function(lines, start):
    """Basic blocks of the function whose body starts at lines[start]; stops at .Lfunc_end."""
    blocks = []
    cur = Block("entry")
    i = start
    while i < len(lines):
        raw = lines[i]
        s = raw.strip()
        if s.startswith(".Lfunc_end"):
            break
        if re.match(r"^\.LBB\d+_\d+:", s) or re.match(r"^; %bb\.\d+:", s):
            name = s.split(":")[0].lstrip("; ")
            if cur.insns or cur.name != "entry" or blocks:
                blocks.append(cur)
            cur = Block(name)
        elif s and not s.startswith((";", ".", "//")) and not s.endswith(":"):
            parts = s.split(None, 1)
            cur.insns.append(Insn(parts[0], parts[1].split(";")[0] if len(parts) > 1 else "", i + 1))
        i += 1
    blocks.append(cur)
    index = {b.name: k for k, b in enumerate(blocks)}
    for k, b in enumerate(blocks):
        last = b.insns[-1] if b.insns else None
        ends = False
        if last is not None:
            if last.op == "s_branch":
                t = last.args.strip()
                if t in index:
                    b.succ.append(index[t])
                ends = True
            elif last.op.startswith("s_cbranch"):
                t = last.args.strip()
                if t in index:
                    b.succ.append(index[t])
            elif last.op in ("s_endpgm", "s_setpc_b64", "s_trap"):
                ends = True
        # a conditional branch may also sit before the last instruction (s_cbranch then s_branch)
        for ins in b.insns[:-1]:
            if ins.op.startswith("s_cbranch") or ins.op == "s_branch":
                t = ins.args.strip()
                if t in index and index[t] not in b.succ:
                    b.succ.append(index[t])
        if not ends and k + 1 < len(blocks):
            b.succ.append(k + 1)
    return blocks


def wait_states(ins: Insn) -> int:
    if ins.op == "s_nop":
        try:
            return int(ins.args.strip(), 0) + 1
        except ValueError:
            return 1
    return 1


def check_function(name, blocks):
    """List of (mfma line, access line, wait states seen, required) violations."""
    bad = []
    for bi, b in enumerate(blocks):
        for ii, ins in enumerate(b.insns):
            if not ins.op.startswith("v_mfma"):
                continue
            ops = [o.strip() for o in ins.args.split(",")]
            dst = regs_of(ops[0])
            need = required_wait_states(ins.op)
            # DFS over (block, index, wait states so far)
            stack = [(bi, ii + 1, 0)]
            seen = set()
            while stack:
                cb, ci, ws = stack.pop()
                if (cb, ci, ws) in seen:
                    continue
                seen.add((cb, ci, ws))
                blk = blocks[cb]
                stop = False
                while ci < len(blk.insns):
                    nx = blk.insns[ci]
                    if ws >= need:
                        stop = True
                        break
                    if nx.op.startswith("v_mfma"):
                        nops = [o.strip() for o in nx.args.split(",")]
                        src_ab = regs_of(",".join(nops[1:3]))
                        if src_ab & dst:
                            bad.append((name, ins.line, nx.line, ws, need))
                        # srcC chain or overwrite by another product: no wait needed; the chain's last
                        # product is checked on its own
                        if regs_of(nops[0]) & dst:
                            stop = True
                            break
                    else:
                        used = regs_of(nx.args)
                        if used & dst:
                            bad.append((name, ins.line, nx.line, ws, need))
                            stop = True
                            break
                    ws += wait_states(nx)
                    ci += 1
                if stop:
                    continue
                for s in blk.succ:
                    stack.append((s, 0, ws))
    return bad


def check_asm(path: str):
    lines = open(path).read().splitlines()
    out = []
    for i, l in enumerate(lines):
        m = re.match(r"^(_Z\w+):\s*(;.*)?$", l)
        if m and ".Lfunc_end" not in l:
            blocks = parse_function(lines, i + 1)
            out += check_function(m.group(1), blocks)
    return out


def compile_asm(src: str, outdir: str) -> str:
    from gated_delta_rule_45_amd import build as kbuild
    out = os.path.join(outdir, os.path.splitext(os.path.basename(src))[0] + ".s")
    cmd = [kbuild._hipcc(), *kbuild.COMMON, *kbuild.DEVICE_FLAGS, "--cuda-device-only", "-S", src, "-o", out]
    cmd = [c for c in cmd if c != "-fPIC"]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc -S failed for {src}:\n{res.stderr[-2000:]}")
    return out


def check_sources(jobs: int = 4):
    """Compile every .hip source of the library to assembly and check it; returns violations."""
    from gated_delta_rule_45_amd import build as kbuild
    srcs = [os.path.join(kbuild.CSRC, s) for s in kbuild.SOURCES if s.endswith(".hip")]
    with tempfile.TemporaryDirectory() as d:
        with ThreadPoolExecutor(max_workers=jobs) as ex:
            asms = list(ex.map(lambda s: compile_asm(s, d), srcs))
        bad = []
        for a in asms:
            bad += [(os.path.basename(a),) + v for v in check_asm(a)]
    return bad


if __name__ == "__main__":
    if len(sys.argv) > 1:
        viol = []
        for p in sys.argv[1:]:
            viol += [(os.path.basename(p),) + v for v in check_asm(p)]
    else:
        viol = check_sources()
    for v in viol:
        print(f"{v[0]}: {v[1][:80]}: mfma at line {v[2]}, access at line {v[3]} after {v[4]} wait states (needs {v[5]})")
    print(f"{len(viol)} violation(s)")
    sys.exit(1 if viol else 0)
