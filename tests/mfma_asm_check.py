"""Static checks of gfx950 assembly for the hazards the compiler does not guard around
inline-asm MFMAs, and for the fixed accumulator registers of the head-size-128 prefill kernel.

The compiler inserts wait states around the MFMAs it emits itself; an MFMA written as inline
asm is opaque to it.  The rules checked here are the ones its hazard recognizer applies on
gfx950 (observed in its own output): after a 32x32x16 MFMA writes a register, 12 wait states
pass before a non-MFMA instruction reads or overwrites it (13 are required here); a vector
instruction's result reaches an MFMA source after 2 wait states; an MFMA may take the same
accumulator it has just written as its C operand at once, but never an MFMA result as its A
or B operand.  Wait states are counted per instruction (``s_nop N`` counts N + 1).  The scan
follows forward branches; a loop's back edge needs 13 wait states behind the last MFMA.

Inline asm appears between ``;;#ASMSTART`` and ``;;#ASMEND`` in the compiler's assembly.
An asm block that reads the accumulators with ``.rept`` (the rescale) counts as reading all
of a0..a127 where it starts.
"""
import re

MFMA_WS = 13     # wait states between an MFMA and a vector access of its result
VALU_WS = 2      # wait states between a vector write and an MFMA reading it
N_FIXED = 128    # a0 .. a127 hold the O^T accumulators


def regs(tok):
    """Register set named by one operand: v5, a[0:15], v[2:5] -> {('v', 5)}, ..."""
    tok = tok.strip()
    m = re.match(r"^([va])\[(\d+):(\d+)\]$", tok)
    if m:
        return {(m.group(1), r) for r in range(int(m.group(2)), int(m.group(3)) + 1)}
    m = re.match(r"^([va])(\d+)$", tok)
    if m:
        return {(m.group(1), int(m.group(2)))}
    return set()


def split_ops(text):
    return [o.strip() for o in re.split(r",(?![^\[]*\])", text)] if text else []


def kernel_body(asm, name_prefix):
    m = re.search(r"^(" + re.escape(name_prefix) + r"[^:\s]*):", asm, re.M)
    if not m:
        raise KeyError(name_prefix)
    end = asm.find(".Lfunc_end", m.end())
    return asm[m.end():end].splitlines()


def check(lines):
    """Findings (line index, message) for one kernel's assembly lines."""
    findings = []
    pending = []      # [regs written by an MFMA, wait states since]
    valu = []         # [regs written by a vector instruction, wait states since]
    since_mfma = 99
    saved = {}        # forward-branch target -> state at the branch
    in_asm = False
    labels_after = {}
    for i, l in enumerate(lines):
        s = l.split(";")[0].strip()
        if s.endswith(":"):
            labels_after.setdefault(s[:-1], i)
    for i, l in enumerate(lines):
        s = l.strip()
        if s.startswith(";;#ASMSTART"):
            in_asm = True
            block = []
            for t in lines[i + 1:]:
                if t.strip().startswith(";;#ASMEND"):
                    break
                block.append(t)
            text = "\n".join(block)
            if ".rept" in text and "v_accvgpr_read" in text:
                for dd, ws in pending:
                    if any(r[0] == "a" and r[1] < N_FIXED for r in dd) and ws < MFMA_WS:
                        findings.append((i, f"accumulator rescale {ws} wait states after an MFMA"))
            continue
        if s.startswith(";;#ASMEND"):
            in_asm = False
            continue
        s = s.split(";")[0].strip()
        if not s or (s.startswith(".") and not s.endswith(":")):
            continue              # empty line, comment or directive
        if s.endswith(":"):
            lab = s[:-1]
            if lab in saved:
                pm, vm, lw = saved.pop(lab)
                pending = pending + pm
                valu = valu + vm
                since_mfma = min(since_mfma, lw)
            elif since_mfma < MFMA_WS:
                findings.append((i, f"label {lab} reached {since_mfma} wait states after an MFMA"))
            continue
        parts = s.split(None, 1)
        op = parts[0]
        ops = split_ops(parts[1]) if len(parts) > 1 else []
        w = int(ops[0], 0) + 1 if op == "s_nop" else 1
        if op.startswith("s_cbranch") or op == "s_branch":
            tgt = ops[0]
            if labels_after.get(tgt, -1) > i:
                pm, vm, lw = saved.get(tgt, ([], [], 99))
                saved[tgt] = (pm + [list(e) for e in pending], vm + [list(e) for e in valu],
                              min(lw, since_mfma))
            elif since_mfma < MFMA_WS:
                findings.append((i, f"back edge {since_mfma} wait states after an MFMA"))
        if op.startswith("v_mfma"):
            dst = regs(ops[0])
            a, b = regs(ops[1]), regs(ops[2])
            c = regs(ops[3]) if len(ops) > 3 else set()
            for rr, ws in valu:
                if rr & (a | b | c) and ws < VALU_WS:
                    findings.append((i, f"MFMA reads a vector result after {ws} wait states: {s}"))
            for dd, ws in pending:
                if dd & (a | b):
                    findings.append((i, f"MFMA takes an MFMA result as A/B operand: {s}"))
                if (dd & (c | dst)) and dd != c and dd != dst and ws < MFMA_WS:
                    findings.append((i, f"MFMA overlaps another's accumulator partially: {s}"))
            if not in_asm and any(r[0] == "a" and r[1] < N_FIXED for r in dst):
                findings.append((i, f"compiler MFMA writes a fixed accumulator: {s}"))
            for e in pending + valu:
                e[1] += w
            pending.append([dst, 0])
            since_mfma = 0
            continue
        read, written = set(), set()
        if ops:
            stores = op.startswith(("ds_write", "buffer_store", "global_store", "scratch_store"))
            if op.startswith("v_cmp") or stores:
                for o in ops:
                    read |= regs(o)
            else:
                written = regs(ops[0])
                for o in ops[1:]:
                    read |= regs(o)
        for dd, ws in pending:
            if (dd & (read | written)) and ws < MFMA_WS:
                findings.append((i, f"access of an MFMA result after {ws} wait states: {s}"))
        if not in_asm and any(r[0] == "a" and r[1] < N_FIXED for r in written):
            findings.append((i, f"compiler writes a fixed accumulator: {s}"))
        for e in pending + valu:
            e[1] += w
        pending = [e for e in pending if e[1] < MFMA_WS + 8]
        valu = [e for e in valu if e[1] < VALU_WS + 2]
        if op.startswith("v_") and written:
            valu.append([written, 0])
        since_mfma += w
    return findings
