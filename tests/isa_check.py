"""Checks of the generated gfx950 assembly around the inline-asm MFMAs.

The output MFMAs that keep O in AGPRs are written as inline asm, and the
compiler's hazard recognizer does not look inside inline asm: it inserts no
wait states between an instruction it issues and an inline-asm MFMA that
reads what that instruction wrote, or between an inline-asm MFMA and a later
instruction that reads its result.  The kernels keep those distances by
construction (the packing of P is pinned well before the output MFMAs; an
explicit `s_nop 7; s_nop 7; s_nop 3` precedes every compiler-issued read of
the AGPR accumulators).  This module finds violations in the assembly text:

* `valu_write_before_asm_mfma`: a VALU instruction (compiler-issued or
  inline asm) writes a VGPR that an inline-asm MFMA reads as its A or B
  operand within the few instructions before it, and no load into that
  register comes in between (a load's result, which the MFMA then reads,
  is awaited by a memory-counter wait, not by wait states);
* `agpr_read_after_asm_mfma`: an instruction the compiler issued (VALU,
  `v_accvgpr_read/mov`, an MFMA reading its C operand, a store) reads an AGPR
  that an inline-asm MFMA writes, with fewer than `required` wait states in
  between on some path of the control-flow graph (each instruction counts
  one wait state, `s_nop n` counts n + 1);
* `agpr_write_before_asm_mfma`: the compiler writes an AGPR that an
  inline-asm MFMA then reads as its C operand within a few wait states.

The control-flow graph is built from the labels and branches of each kernel.
"""
from __future__ import annotations

import re

KERNEL_RE = re.compile(r"^(_ZN3fa2\S*_kernel\S*):", re.M)
MFMA_RE = re.compile(r"^v_(?:mfma|smfmac)\w*\s+(\S+),\s*(\S+),\s*(\S+),\s*(\S+)")
REG_RE = re.compile(r"(?<![\w.])([av])(?:\[(\d+):(\d+)\]|(\d+)\b)")
# A wait-state count that covers the result latency of a 32x32x16 MFMA
# (16 passes) for any reader, on gfx950.
REQUIRED_AFTER_MFMA = 19
# Wait states between a VALU write and an MFMA that reads the written
# register as an operand.
REQUIRED_BEFORE_MFMA = 4
STORE_PREFIXES = ("buffer_store", "scratch_store")
LOAD_PREFIXES = ("ds_read", "ds_load", "buffer_load", "global_load", "flat_load", "scratch_load")


def regs(operand: str, kind: str) -> set:
    """Register numbers of `kind` ('a' or 'v') named by one operand."""
    out = set()
    for m in REG_RE.finditer(operand):
        if m.group(1) != kind:
            continue
        if m.group(4) is not None:
            out.add(int(m.group(4)))
        else:
            out.update(range(int(m.group(2)), int(m.group(3)) + 1))
    return out


def split_operands(line: str):
    parts = line.split(None, 1)
    mnem = parts[0]
    ops = [o.strip() for o in re.split(r",(?![^\[]*\])", parts[1])] if len(parts) > 1 else []
    return mnem, ops


class Instr:
    __slots__ = ("text", "mnem", "ops", "asm", "waits")

    def __init__(self, text: str, asm: bool):
        self.text = text
        self.asm = asm
        self.mnem, self.ops = split_operands(text)
        m = re.match(r"s_nop\s+(\d+)", text)
        self.waits = int(m.group(1)) + 1 if m else 1

    def agpr_reads(self) -> set:
        if self.mnem.startswith(STORE_PREFIXES):
            srcs = self.ops
        else:
            srcs = self.ops[1:]
        out = set()
        for o in srcs:
            out |= regs(o, "a")
        return out

    def agpr_writes(self) -> set:
        if not self.ops or self.mnem.startswith(STORE_PREFIXES) or self.mnem.startswith("s_"):
            return set()
        return regs(self.ops[0], "a")

    def vgpr_writes(self) -> set:
        if not self.mnem.startswith("v_") or not self.ops:
            return set()
        return regs(self.ops[0], "v")

    def load_writes(self) -> set:
        """VGPRs a memory load writes (none for loads straight into LDS,
        whose first operand is an address)."""
        if not self.mnem.startswith(LOAD_PREFIXES) or not self.ops or re.search(r"\blds\s*$", self.text):
            return set()
        return regs(self.ops[0], "v")


def kernel_bodies(text: str) -> dict:
    """{kernel symbol: list of Instr and label strings} for every kernel."""
    out = {}
    for m in KERNEL_RE.finditer(text):
        name = m.group(1)
        start = m.end()
        end = text.index(".Lfunc_end", start)
        items = []
        in_asm = False
        for raw in text[start:end].splitlines():
            line = raw.strip()
            if line.startswith(";;#ASMSTART"):
                in_asm = True
                continue
            if line.startswith(";;#ASMEND"):
                in_asm = False
                continue
            line = line.split(";")[0].strip()
            if not line:
                continue
            if line.endswith(":"):
                items.append(line[:-1])
                continue
            if line.startswith("."):
                continue
            for piece in line.split("\n"):
                items.append(Instr(piece.strip(), in_asm))
        out[name] = items
    return out


def cfg(items):
    """Basic blocks (lists of Instr) and each block's predecessors."""
    blocks, labels = [[]], {}
    for it in items:
        if isinstance(it, str):
            if blocks[-1]:
                blocks.append([])
            labels[it] = len(blocks) - 1
            continue
        blocks[-1].append(it)
        if it.mnem.startswith(("s_branch", "s_cbranch", "s_endpgm", "s_setpc")):
            blocks.append([])
    preds = [set() for _ in blocks]
    for b, blk in enumerate(blocks):
        last = blk[-1] if blk else None
        falls = last is None or not last.mnem.startswith(("s_branch", "s_endpgm", "s_setpc"))
        if falls and b + 1 < len(blocks):
            preds[b + 1].add(b)
        if last is not None and last.mnem.startswith(("s_branch", "s_cbranch")) and last.ops:
            target = labels.get(last.ops[0])
            if target is not None:
                preds[target].add(b)
    return blocks, preds


def walk_back(blocks, preds, b, i, limit, hit):
    """Paths backwards from instruction i of block b (exclusive): returns the
    smallest wait-state distance to an instruction for which hit(instr) is
    true, or None when every path reaches `limit` first."""
    best = None
    stack = [(b, i, 0)]
    seen = {}
    while stack:
        blk, idx, acc = stack.pop()
        while idx > 0:
            idx -= 1
            ins = blocks[blk][idx]
            if hit(ins):
                best = acc if best is None else min(best, acc)
                break
            acc += ins.waits
            if acc >= limit:
                break
        else:
            for p in preds[blk]:
                if seen.get(p, limit + 1) > acc:
                    seen[p] = acc
                    stack.append((p, len(blocks[p]), acc))
    return best


def valu_write_distance(blocks, preds, b, i, srcs, limit):
    """Smallest wait-state distance, over the paths backwards from
    instruction i of block b, to a VALU write of one of the registers `srcs`
    that no later load on the path overwrites; None when there is none
    within `limit`."""
    best = None
    stack = [(b, i, 0, frozenset(srcs))]
    seen = {}
    while stack:
        blk, idx, acc, live = stack.pop()
        while idx > 0 and live:
            idx -= 1
            ins = blocks[blk][idx]
            if ins.mnem.startswith("v_") and not ins.mnem.startswith(("v_mfma", "v_smfmac")) and \
                    ins.vgpr_writes() & live:
                best = acc if best is None else min(best, acc)
                break
            live = live - ins.load_writes()
            acc += ins.waits
            if acc >= limit:
                break
        else:
            if live:
                for p in preds[blk]:
                    if seen.get((p, live), limit + 1) > acc:
                        seen[(p, live)] = acc
                        stack.append((p, len(blocks[p]), acc, live))
    return best


def check_kernel(items):
    """List of (kind, message) violations in one kernel."""
    blocks, preds = cfg(items)
    found = []
    for b, blk in enumerate(blocks):
        for i, ins in enumerate(blk):
            mf = MFMA_RE.match(ins.text)
            if ins.asm and mf:
                # Operands A and B of an inline-asm MFMA: no VALU write shortly before.
                srcs = regs(mf.group(2), "v") | regs(mf.group(3), "v")
                src_c = regs(mf.group(4), "a")

                d = valu_write_distance(blocks, preds, b, i, srcs, REQUIRED_BEFORE_MFMA)
                if d is not None:
                    found.append(("valu_write_before_asm_mfma", f"{ins.text} ({d} wait states after a VALU write)"))

                # Operand C (the accumulator) written by a compiler-issued instruction.
                def agpr_hit(x, src_c=src_c):
                    return not x.asm and bool(x.agpr_writes() & src_c)
                d = walk_back(blocks, preds, b, i, REQUIRED_BEFORE_MFMA, agpr_hit)
                if d is not None:
                    found.append(("agpr_write_before_asm_mfma", f"{ins.text} ({d} wait states after a write)"))
                continue
            if ins.asm:
                continue
            reads = ins.agpr_reads()
            if not reads:
                continue

            def mfma_hit(x, reads=reads):
                m = MFMA_RE.match(x.text)
                return x.asm and m is not None and bool(regs(m.group(1), "a") & reads)
            d = walk_back(blocks, preds, b, i, REQUIRED_AFTER_MFMA, mfma_hit)
            if d is not None:
                found.append(("agpr_read_after_asm_mfma", f"{ins.text} ({d} wait states after an asm MFMA)"))
    return found


def check_text(text: str) -> dict:
    """{kernel: violations} over every kernel of an assembly listing."""
    return {name: check_kernel(items) for name, items in kernel_bodies(text).items()}
