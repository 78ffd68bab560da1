"""Data-hazard check for matrix instructions written as inline asm in the GEMM kernels.

The compiler pads the wait states a matrix instruction needs only around products it generated
itself; a product written as inline asm (between the ;;#ASMSTART / ;;#ASMEND markers of the
assembly listing) is opaque to it.  This scan flags, for each such product:

  * a non-matrix vector instruction writing one of its source registers fewer than WRITE_BEFORE
    wait states before it (two are required for a vector write read by a product);
  * a non-matrix vector, LDS or buffer instruction touching its result registers fewer than
    READ_AFTER wait states after it (a 16 x 16 x 32 bf16 product has 8 passes; the compiler's own
    padding for it is 8, so 11 leaves a margin).

Each instruction counts as one wait state and s_nop N as N + 1.  The scan runs over each kernel's
straight-line listing and over every backward branch (the loop's tail followed by its head)."""

import re

WRITE_BEFORE = 2
READ_AFTER = 11


def _regs(tok):
    m = re.match(r"([va])\[(\d+):(\d+)\]", tok)
    if m:
        return {(m.group(1), i) for i in range(int(m.group(2)), int(m.group(3)) + 1)}
    m = re.match(r"([va])(\d+)$", tok)
    if m:
        return {(m.group(1), int(m.group(2)))}
    return set()


def _wait_states(op, ops):
    return int(ops[0], 0) + 1 if op == "s_nop" else 1


def _check(instrs, name, report):
    for i, (op, ops, asm) in enumerate(instrs):
        if not (asm and op.startswith("v_mfma")):
            continue
        dst = _regs(ops[0])
        srcs = set().union(*(_regs(o) for o in ops[1:4]))
        w = 0
        for j in range(i - 1, -1, -1):
            pop, pops, _ = instrs[j]
            if pop.startswith("v_") and not pop.startswith("v_mfma") and pops and _regs(pops[0]) & srcs:
                if w < WRITE_BEFORE:
                    report.append(f"{name}: {pop} {pops[0]} {w} wait states before {op} {' '.join(ops)}")
                break
            w += _wait_states(pop, pops)
            if w >= WRITE_BEFORE:
                break
        w = 0
        for j in range(i + 1, len(instrs)):
            pop, pops, _ = instrs[j]
            if pop.startswith("v_mfma"):
                w += 1
                continue
            touched = set().union(*(_regs(o) for o in pops)) if pops else set()
            if pop.startswith(("v_", "ds_", "buffer_", "global_")) and touched & dst:
                if w < READ_AFTER:
                    report.append(f"{name}: {pop} {' '.join(pops)} {w} wait states after {op} {ops[0]}")
                break
            w += _wait_states(pop, pops)
            if w >= READ_AFTER:
                break


def scan(listing: str):
    """Hazard reports (empty if none) and the number of inline-asm products seen, over every kernel
    of an AMDGPU assembly listing."""
    report, products = [], 0
    for m in re.finditer(r"^(_Z\S+):", listing, re.M):
        name = m.group(1)
        body = listing[m.end():].split(".Lfunc_end")[0]
        instrs, labels, in_asm = [], {}, False
        for line in body.split("\n"):
            if ";;#ASMSTART" in line:
                in_asm = True
                continue
            if ";;#ASMEND" in line:
                in_asm = False
                continue
            lm = re.match(r"^(\.LBB\S+):", line)
            if lm:
                labels[lm.group(1)] = len(instrs)
                continue
            text = line.split(";")[0].strip()
            if not text or text.startswith(".") or text.endswith(":"):
                continue
            parts = text.split(None, 1)
            if not re.match(r"^[a-z_0-9]+$", parts[0]):
                continue
            ops = [o.strip() for o in parts[1].split(",")] if len(parts) > 1 else []
            instrs.append((parts[0], ops, in_asm))
            if in_asm and parts[0].startswith("v_mfma"):
                products += 1
        _check(instrs, name, report)
        for k, (op, ops, _) in enumerate(instrs):
            if (op.startswith("s_cbranch") or op == "s_branch") and ops and ops[0] in labels and labels[ops[0]] <= k:
                head = labels[ops[0]]
                _check(instrs[max(head, k - 64):k + 1] + instrs[head:head + 64], name + " (back edge)", report)
    return report, products
