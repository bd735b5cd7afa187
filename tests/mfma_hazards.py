"""Matrix-core hazards the compiler cannot see: a scan of gfx950 assembly.

The forward kernel issues its products as inline assembly, so the compiler's
hazard recognizer does not know that an instruction is a matrix-core op and
inserts no wait states around it. This scan re-checks the emitted assembly
along every control-flow path (fall-through and branch targets, so loop
back-edges and joins too) for the two rules that matter here:

* a VALU instruction (v_accvgpr_* included) that writes a register a product
  reads, fewer than 2 wait states before the product;
* any non-matrix-core instruction that reads or writes a product's result
  registers, or a product that takes them as its A/B operand (or overlaps
  them only partly as C), fewer than ``window`` wait states after it. An
  8-pass 32x32x16 product needs 11; the default 19 is the 16-pass figure.

A wait state is one issued instruction; ``s_nop n`` counts n + 1.
"""

import re

_REG = re.compile(r"([va])\[(\d+):(\d+)\]|([va])(\d+)$")


def _regs(tok):
    m = _REG.match(tok)
    if not m:
        return set()
    if m.group(1):
        return {(m.group(1), r) for r in range(int(m.group(2)), int(m.group(3)) + 1)}
    return {(m.group(4), int(m.group(5)))}


def _parse(text):
    ins, labels = [], {}
    for ln, line in enumerate(text.split("\n"), 1):
        s = line.split(";")[0].strip()
        if not s:
            continue
        if s.endswith(":"):
            labels[s[:-1]] = len(ins)
            continue
        if s.startswith("."):
            continue
        parts = s.split(None, 1)
        ops = [o.strip() for o in parts[1].split(",")] if len(parts) > 1 else []
        ins.append((ln, parts[0], ops))
    return ins, labels


def _writes(op, ops):
    if not ops or op.startswith(("v_cmp", "v_readlane", "v_readfirstlane")) and not op.startswith("v_cmpx"):
        return set()
    if op.startswith(("v_", "ds_read", "buffer_load", "global_load")):
        return _regs(ops[0])
    return set()


def _touches(op, ops):
    out = set()
    for o in ops:
        out |= _regs(o)
    return out


def _cost(op, ops):
    return int(ops[0], 0) + 1 if op == "s_nop" else 1


def kernels(asm):
    """``{symbol: body}`` of every kernel in a device assembly file."""
    out = {}
    for m in re.finditer(r"^(\w+):[ \t]*(?:;.*)?$", asm, re.M):
        name = m.group(1)
        if not name.startswith("_Z"):
            continue
        end = asm.find("\n.Lfunc_end", m.end())
        if end > 0:
            out[name] = asm[m.end():end]
    return out


def scan(body, window=19):
    """Hazards in one kernel body, as readable strings (empty: none)."""
    ins, labels = _parse(body)

    def succ(i):
        op, ops = ins[i][1], ins[i][2]
        if op == "s_endpgm":
            return []
        if op == "s_branch":
            return [labels[ops[0]]] if ops[0] in labels else []
        nxt = [i + 1] if i + 1 < len(ins) else []
        if op.startswith("s_cbranch") and ops and ops[0] in labels:
            nxt.append(labels[ops[0]])
        return nxt

    pred = {}
    for i in range(len(ins)):
        for j in succ(i):
            pred.setdefault(j, []).append(i)
    found = set()
    for i, (ln, op, ops) in enumerate(ins):
        if not op.startswith("v_mfma"):
            continue
        dst = _regs(ops[0])
        src = set()
        for o in ops[1:]:
            src |= _regs(o)
        # after the product
        stack, seen = [(j, 0) for j in succ(i)], set()
        while stack:
            j, w = stack.pop()
            if w >= window or (j, w) in seen:
                continue
            seen.add((j, w))
            lj, opj, opsj = ins[j]
            if opj.startswith("v_mfma"):
                ab = set()
                for o in opsj[1:3]:
                    ab |= _regs(o)
                c = _regs(opsj[3]) if len(opsj) > 3 else set()
                if ab & dst:
                    found.add(f"line {lj}: {opj} takes the result of line {ln} as A/B after {w} wait states")
                if (c & dst) and c != dst:
                    found.add(f"line {lj}: {opj} overlaps the result of line {ln} partly as C")
            elif opj.startswith(("v_", "ds_", "buffer_", "global_")) and _touches(opj, opsj) & dst:
                found.add(f"line {lj}: {opj} touches the result of line {ln} after {w} wait states")
            stack.extend((k, w + _cost(opj, opsj)) for k in succ(j))
        # before the product
        stack, seen = [(j, 0) for j in pred.get(i, [])], set()
        while stack:
            j, w = stack.pop()
            if w >= 2 or (j, w) in seen:
                continue
            seen.add((j, w))
            lj, opj, opsj = ins[j]
            if opj.startswith("v_") and not opj.startswith("v_mfma") and _writes(opj, opsj) & src:
                found.add(f"line {lj}: {opj} writes an operand of line {ln} {w} wait states before it")
            stack.extend((k, w + _cost(opj, opsj)) for k in pred.get(j, []))
    return sorted(found)
