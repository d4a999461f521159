"""Static check of MFMA result reads in gfx950 assembly.

An MFMA writes its result some cycles after it issues; an instruction other
than an MFMA that reads those registers sooner sees a partly accumulated
value.  The hardware does not wait: the program must put enough independent
instructions (wait states, `s_nop n` counting n + 1) between the two.  The
compiler pads straight-line code; a read reached through a branch is where a
short gap can slip through.  This module finds, for every MFMA in a kernel,
the fewest wait states on any control-flow path (fall-through and branch
targets) to the first non-MFMA instruction that reads one of its result
registers, and reports paths shorter than the requirement.

Requirement per opcode (gfx950): passes + 4 for the f16 MFMAs, passes + 2
for the float32 ones, with passes 8 (32x32x16 f16), 4 (16x16x32 and
16x16x16 f16), 16 (32x32x2 f32) and 8 (16x16x4 f32).  These are the gaps the
compiler itself leaves in straight-line code for each opcode.
"""

import re

PASSES = {
    "v_mfma_f32_32x32x16_f16": (8, 4),
    "v_mfma_f32_16x16x32_f16": (4, 4),
    "v_mfma_f32_16x16x16_f16": (4, 4),
    "v_mfma_f32_16x16x16f16": (4, 4),
    "v_mfma_f32_32x32x2_f32": (16, 2),
    "v_mfma_f32_16x16x4_f32": (8, 2),
}


def required_wait_states(op):
    passes, extra = PASSES[op]
    return passes + extra


def _regs(tok):
    """Vector / accumulation register ranges named in one operand."""
    out = []
    for m in re.finditer(r"\b([va])\[(\d+):(\d+)\]|\b([va])(\d+)\b", tok):
        if m.group(1):
            out.append((m.group(1), int(m.group(2)), int(m.group(3))))
        else:
            out.append((m.group(4), int(m.group(5)), int(m.group(5))))
    return out


def parse(text):
    """Kernels of an assembly listing: name -> (instructions, labels)."""
    kernels = {}
    cur = None
    for line in text.splitlines():
        m = re.match(r"^(_Z\w+):", line)
        if m:
            cur = ([], {})
            kernels[m.group(1)] = cur
            continue
        if cur is None:
            continue
        if line.startswith(".Lfunc_end"):
            cur = None
            continue
        m = re.match(r"^(\.LBB\d+_\d+):", line)
        if m:
            cur[1][m.group(1)] = len(cur[0])
            continue
        t = line.split(";")[0].strip()
        if not t or t.startswith("."):
            continue
        parts = t.split(None, 1)
        ops = [a.strip() for a in parts[1].split(",")] if len(parts) > 1 else []
        cur[0].append((parts[0], ops))
    return kernels


def _reads(op, ops, dst):
    if op.startswith("v_mfma") or op.startswith("s_"):
        return False
    stores = ("global_store", "buffer_store", "ds_write", "flat_store", "scratch_store")
    if op.startswith(stores) or op.startswith("v_cmp"):
        srcs = ops
    else:
        srcs = ops[1:]
    for tok in srcs:
        for kind, lo, hi in _regs(tok):
            if kind == dst[0] and not (hi < dst[1] or lo > dst[2]):
                return True
    return False


def _wait_states(op, ops):
    return int(ops[0], 0) + 1 if op == "s_nop" else 1


def violations(text):
    """(kernel, instruction index, opcode, wait states found, required) for
    every MFMA result read that comes too soon on some path."""
    found = []
    for name, (ins, labels) in parse(text).items():
        for i, (op, ops) in enumerate(ins):
            if op not in PASSES:
                continue
            d = _regs(ops[0])
            if not d:
                continue
            dst, need = d[0], required_wait_states(op)
            stack, seen, short = [(i + 1, 0)], set(), None
            while stack:
                pos, w = stack.pop()
                while pos < len(ins) and w < need:
                    if (pos, w) in seen:
                        break
                    seen.add((pos, w))
                    o, a = ins[pos]
                    if _reads(o, a, dst):
                        short = w if short is None else min(short, w)
                        break
                    if o.startswith("v_mfma"):
                        d2 = _regs(a[0])
                        if d2 and d2[0][0] == dst[0] and not (d2[0][2] < dst[1] or d2[0][1] > dst[2]):
                            break  # the registers now belong to another MFMA chain
                    w += _wait_states(o, a)
                    if o == "s_endpgm" or o.startswith("s_setpc"):
                        break
                    if o == "s_branch":
                        pos = labels[a[0]]
                        continue
                    if o.startswith("s_cbranch"):
                        stack.append((labels[a[0]], w))
                    pos += 1
            if short is not None:
                found.append((name, i, op, short, need))
    return found
