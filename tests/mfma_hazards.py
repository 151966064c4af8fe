"""Static check of MFMA data hazards in gfx950 assembly (.s text from hipcc -S).

Kernels that issue MFMAs from inline asm take over from the compiler the job of
spacing dependent instructions: the matrix core writes its result registers
several cycles after issue and the hardware does not interlock vector reads of
them.  This checker walks the control-flow graph of every function in the
assembly and reports:

  * a non-MFMA instruction that reads or writes a register of an MFMA result
    (VGPR or AGPR) fewer than ``result_window(passes)`` wait states after the MFMA issued
    (an MFMA that accumulates into exactly the same registers is allowed: the
    hardware forwards back-to-back accumulations);
  * a non-MFMA instruction that writes a register an MFMA reads as its
    accumulator input (srcC) fewer than ``passes - 1`` wait states after the
    MFMA issued (the matrix core reads srcC over several passes);
  * an MFMA that reads a register written by a VALU instruction fewer than
    ``valu_window`` wait states earlier.

``passes`` is the MFMA's number of 4-cycle passes on gfx950 (``mfma_passes``):
4 for the 16x16x32 bf16/f16 forms, 8 for 32x32x16, 16 for the 32x32x64 fp8
form.  The windows are the figures the compiler schedules for gfx950's XDL ops:
a result may be read 8, 12 and 19 wait states after a 4-, 8- and 16-pass MFMA
issued (one more than gfx940's passes + 3 for 4 and 8 passes, not for 16), and
its accumulator input overwritten passes - 1 after.  ``mfma_window`` /
``srcc_window`` override them for every MFMA.

Wait states are counted as the compiler does: one per instruction, N + 1 for
``s_nop N``.  Along control flow the count is the minimum over all paths
(loops included), so the check is conservative."""

import re

_REG = re.compile(r"\b([va])(?:\[(\d+):(\d+)\]|(\d+)(?!\w))")
_BRANCH = re.compile(r"^s_(c?branch\w*)\s+(\.?L\w+)")


def _regs(text):
    out = []
    for m in _REG.finditer(text):
        base = 0 if m.group(1) == "v" else 256
        if m.group(4) is not None:
            out.append((base + int(m.group(4)),))
        else:
            out.append(tuple(range(base + int(m.group(2)), base + int(m.group(3)) + 1)))
    return out


def _operands(ins):
    parts = ins.split(None, 1)
    if len(parts) < 2:
        return parts[0], []
    ops = []
    depth = 0
    cur = ""
    for ch in parts[1]:
        if ch == "[":
            depth += 1
        elif ch == "]":
            depth -= 1
        if ch == "," and depth == 0:
            ops.append(cur.strip())
            cur = ""
        else:
            cur += ch
    if cur.strip():
        ops.append(cur.strip())
    return parts[0], ops


def classify(ins):
    """(opcode, kind, defs, uses); defs/uses are lists of register tuples."""
    op, ops = _operands(ins)
    regs = [_regs(o) for o in ops]
    flat = lambda lst: [r for x in lst for r in x]
    if op.startswith("v_mfma") or op.startswith("v_smfmac"):
        return op, "mfma", regs[0] if regs else [], flat(regs[1:])
    if op.startswith("v_"):
        if op.startswith("v_permlane") and "swap" in op:
            return op, "valu", flat(regs), flat(regs)
        if op.startswith("v_cmp") or op.startswith("v_readlane") or op.startswith("v_readfirstlane"):
            return op, "valu", [], flat(regs[1:]) if op.startswith("v_cmp") else flat(regs)
        # VOP2 accumulate forms (v_dot2c, v_fmac, v_mac) read their destination too
        acc = "c_" in op or op.startswith("v_fmac") or op.startswith("v_mac")
        return op, "valu", regs[0] if regs else [], flat(regs[1:]) + (regs[0] if acc and regs else [])
    if op.startswith(("ds_", "global_", "buffer_", "flat_", "scratch_")):
        store = any(k in op for k in ("write", "store", "atomic", "add_", "or_"))
        if store and not ("read" in op or "load" in op):
            return op, "mem", [], flat(regs)
        return op, "mem", regs[0] if regs else [], flat(regs[1:])
    return op, "other", [], []


def _functions(text):
    """Yield (name, [lines]) for each function body in the assembly."""
    lines = text.split("\n")
    i = 0
    while i < len(lines):
        m = re.match(r"^([A-Za-z_][\w.$]*):\s*(;.*)?$", lines[i])
        if m and i > 0 and ".type" in "".join(lines[max(0, i - 4):i]):
            name = m.group(1)
            body = []
            i += 1
            while i < len(lines) and not lines[i].startswith(".Lfunc_end"):
                body.append(lines[i])
                i += 1
            yield name, body
        i += 1


def _blocks(body):
    """Split a function body into basic blocks of instructions."""
    blocks, labels = [], {}
    cur = {"label": None, "ins": [], "succ": [], "fall": True}
    blocks.append(cur)
    for raw in body:
        line = raw.split(";", 1)[0].strip()
        if not line or line.startswith("."):
            m = re.match(r"^(\.L\w+):", raw.strip())
            if m:
                if cur["ins"] or cur["label"] is not None:
                    cur = {"label": m.group(1), "ins": [], "succ": [], "fall": True}
                    blocks.append(cur)
                else:
                    cur["label"] = m.group(1)
                labels[m.group(1)] = len(blocks) - 1
            continue
        cur["ins"].append(line)
        b = _BRANCH.match(line)
        if b or line.startswith("s_endpgm") or line.startswith("s_setpc"):
            if b:
                cur["succ"].append(b.group(2))
            cur["fall"] = not (line.startswith("s_branch") or line.startswith("s_endpgm")
                               or line.startswith("s_setpc"))
            cur = {"label": None, "ins": [], "succ": [], "fall": True}
            blocks.append(cur)
    succ = []
    for k, blk in enumerate(blocks):
        s = [labels[x] for x in blk["succ"] if x in labels]
        if blk["fall"] and k + 1 < len(blocks):
            s.append(k + 1)
        succ.append(s)
    return blocks, succ


_PASSES = [
    (re.compile(r"v_mfma_f32_16x16x32_(bf16|f16)\b"), 4),
    (re.compile(r"v_mfma_f32_32x32x16_(bf16|f16)\b"), 8),
    (re.compile(r"v_mfma_(scale_)?f32_16x16x128_f8f6f4\b"), 8),
    (re.compile(r"v_mfma_(scale_)?f32_32x32x64_f8f6f4\b"), 16),
]
_RESULT_WINDOW = {4: 8, 8: 12, 16: 19}


def mfma_passes(op):
    """Passes of an MFMA opcode on gfx950 (16, the longest, for forms not listed)."""
    for pat, n in _PASSES:
        if pat.match(op):
            return n
    return 16


def check(text, mfma_window=None, valu_window=2, srcc_window=None):
    """Return a list of violation strings for every function in ``text``."""
    found = []
    for fname, body in _functions(text):
        blocks, succ = _blocks(body)
        # state: reg -> (wait states still needed, exact MFMA dst range), reg -> VALU wait,
        # reg -> srcC read wait
        entry = [None] * len(blocks)
        entry[0] = ({}, {}, {})
        work = [0]
        reported = set()
        while work:
            k = work.pop()
            mf, va, sc = dict(entry[k][0]), dict(entry[k][1]), dict(entry[k][2])
            for ins in blocks[k]["ins"]:
                op, kind, defs, uses = classify(ins)
                n = 1
                m = re.match(r"s_nop\s+(\d+)", ins)
                if m:
                    n = int(m.group(1)) + 1
                if kind == "mfma":
                    dst = defs[0] if defs else ()
                    for r in uses:
                        for reg in r:
                            if reg in va and va[reg] > 0:
                                found_key = (fname, ins, "valu->mfma")
                                if found_key not in reported:
                                    reported.add(found_key)
                                    found.append(f"{fname}: '{ins}' reads a VALU result "
                                                 f"{valu_window - va[reg]} wait states after it")
                            if reg in mf and mf[reg][0] > 0 and r != mf[reg][1]:
                                found_key = (fname, ins, "mfma->mfma")
                                if found_key not in reported:
                                    reported.add(found_key)
                                    found.append(f"{fname}: '{ins}' reads part of an MFMA result "
                                                 "before it is written")
                else:
                    for reg in (reg for r in defs for reg in r):
                        if reg in sc and sc[reg] > 0:
                            found_key = (fname, ins, "srcc-war")
                            if found_key not in reported:
                                reported.add(found_key)
                                found.append(f"{fname}: '{ins}' overwrites an MFMA accumulator input "
                                             f"{sc[reg]} wait states too early")
                    touched = [reg for r in defs + uses for reg in r]
                    for reg in touched:
                        if reg in mf and mf[reg][0] > 0:
                            found_key = (fname, ins, "mfma->other")
                            if found_key not in reported:
                                reported.add(found_key)
                                found.append(f"{fname}: '{ins}' touches an MFMA result "
                                             f"{mf[reg][0]} wait states too early")
                # advance time, then record this instruction's own effects
                for d in (mf, va, sc):
                    for reg in list(d):
                        if d is mf:
                            left = d[reg][0] - n
                            if left <= 0:
                                del d[reg]
                            else:
                                d[reg] = (left, d[reg][1])
                        else:
                            d[reg] -= n
                            if d[reg] <= 0:
                                del d[reg]
                if kind == "mfma" and defs:
                    p = mfma_passes(op)
                    mw = mfma_window if mfma_window is not None else _RESULT_WINDOW.get(p, p + 4)
                    cw = srcc_window if srcc_window is not None else p - 1
                    for reg in defs[0]:
                        mf[reg] = (mw, defs[0])
                    if len(uses) >= 3:
                        for reg in uses[2]:
                            sc[reg] = cw
                if kind == "valu":
                    for r in defs:
                        for reg in r:
                            va[reg] = valu_window
            for s in succ[k]:
                if entry[s] is None:
                    entry[s] = (dict(mf), dict(va), dict(sc))
                    work.append(s)
                    continue
                old_mf, old_va, old_sc = entry[s]
                changed = False
                for reg, (w, rng) in mf.items():
                    if reg not in old_mf or old_mf[reg][0] < w:
                        old_mf[reg] = (w, rng)
                        changed = True
                for reg, w in va.items():
                    if old_va.get(reg, 0) < w:
                        old_va[reg] = w
                        changed = True
                for reg, w in sc.items():
                    if old_sc.get(reg, 0) < w:
                        old_sc[reg] = w
                        changed = True
                if changed:
                    work.append(s)
    return found
