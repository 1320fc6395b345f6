"""Static check of MFMA data hazards in gfx950 assembly emitted for the library.

The decode kernel issues its MFMAs through inline asm, so the compiler's hazard
recognizer does not see them; the wait states are written into the asm by
hand.  This checker re-derives the two rules that matter from the assembly:

  * an MFMA result must not be read or overwritten by any instruction other
    than an MFMA accumulating into exactly the same registers for RESULT_WAIT
    wait states after the MFMA issues;
  * an MFMA must not read an A/B operand register written by a VALU instruction
    within OPERAND_WAIT wait states before it.

An `s_nop N` counts as N + 1 wait states, every other instruction as one.  The
rules are the ones the compiler itself applies on gfx950: it emits 11-12 wait
states between v_mfma_f32_32x32x16_bf16 and a dependent VALU, 20 after the
16-pass v_mfma_f32_32x32x64_f8f6f4, and 2 between a VALU write and an MFMA
source read.  Windows are carried
across basic blocks along every branch and fall-through edge (a forward
dataflow pass to a fixed point), so loop back-edges are covered.
"""

import re

RESULT_WAIT = 12
OPERAND_WAIT = 2
# result windows of MFMAs with more passes than the bf16 32x32x16 one
RESULT_WAIT_BY_OP = {"v_mfma_f32_32x32x64_f8f6f4": 20}

_REG = re.compile(r"(?<![\w.])([va])(?:\[(\d+):(\d+)\]|(\d+)(?!\w))")
_LABEL = re.compile(r"^(\.LBB\d+_\d+|\.Ltmp\d+):")


def _regs(text):
    out = set()
    for m in _REG.finditer(text):
        cls = m.group(1)
        if m.group(4) is not None:
            out.add((cls, int(m.group(4))))
        else:
            for i in range(int(m.group(2)), int(m.group(3)) + 1):
                out.add((cls, i))
    return out


def _split(line):
    body = line.split(";")[0].strip()
    if not body or body.endswith(":") or body.startswith("."):
        return None, []
    parts = body.split(None, 1)
    op = parts[0]
    ops = [o.strip() for o in parts[1].split(",")] if len(parts) > 1 else []
    return op, ops


def kernel_bodies(asm_text):
    """Yield (name, [lines]) for every function body in the assembly."""
    name, body = None, []
    for line in asm_text.splitlines():
        m = re.match(r"^([A-Za-z_][\w.$]*):\s*(;.*)?$", line)
        if m and not m.group(1).startswith(".L"):
            if name is not None:
                yield name, body
            name, body = m.group(1), []
            continue
        if name is not None:
            body.append(line)
            if line.strip().startswith("s_endpgm"):
                yield name, body
                name, body = None, []


def _blocks(lines):
    """Split a body into basic blocks: list of (label, [(line_no, op, ops, text)], successors)."""
    blocks, cur_label, cur = [], "<entry>", []
    for no, line in enumerate(lines):
        s = line.strip()
        m = _LABEL.match(s)
        if m:
            blocks.append([cur_label, cur])
            cur_label, cur = m.group(1), []
            continue
        op, ops = _split(line)
        if op is None:
            continue
        cur.append((no, op, ops, s))
        if op.startswith("s_cbranch") or op == "s_branch" or op == "s_endpgm" or op.startswith("s_setpc"):
            blocks.append([cur_label, cur])
            cur_label, cur = f"<after {no}>", []
    blocks.append([cur_label, cur])
    blocks = [b for b in blocks if b[1] or b[0] != "<entry>"]
    index = {b[0]: i for i, b in enumerate(blocks)}
    out = []
    for i, (label, insts) in enumerate(blocks):
        succ = []
        last = insts[-1] if insts else None
        falls = True
        if last is not None:
            op, ops = last[1], last[2]
            if op == "s_branch":
                falls = False
                if ops and ops[0] in index:
                    succ.append(index[ops[0]])
            elif op.startswith("s_cbranch"):
                if ops and ops[0] in index:
                    succ.append(index[ops[0]])
            elif op == "s_endpgm" or op.startswith("s_setpc"):
                falls = False
        if falls and i + 1 < len(blocks):
            succ.append(i + 1)
        out.append((label, insts, succ))
    return out


def _run_block(insts, pending, recent, problems):
    """Advance hazard state through one block; pending: {reg: (left, dst, line)},
    recent: {reg: (left, line)}.  Appends findings to problems (a set)."""
    pending = dict(pending)
    recent = dict(recent)
    for no, op, ops, text in insts:
        waits = int(ops[0], 0) + 1 if op == "s_nop" and ops else 1
        if op.startswith("v_mfma"):
            dst, srcc = ops[0], (ops[3] if len(ops) > 3 else "")
            dregs = _regs(dst)
            srcs_ab = _regs(ops[1]) | _regs(ops[2])
            key = dst.replace(" ", "")
            chain = srcc.replace(" ", "") == key
            for r in srcs_ab:
                if r in pending:
                    left, pdst, at = pending[r]
                    problems.add(f"line {no}: MFMA reads {r} as A/B {RESULT_WAIT - left} wait states "
                                 f"after MFMA at line {at}")
                if r in recent:
                    left, at = recent[r]
                    problems.add(f"line {no}: MFMA A/B operand {r} written by VALU at line {at} "
                                 f"{OPERAND_WAIT - left} wait states before")
            for r in _regs(srcc) | dregs:
                if r in pending:
                    left, pdst, at = pending[r]
                    if not (chain and pdst == key):
                        problems.add(f"line {no}: MFMA touches in-flight result {pdst} of line {at} "
                                     f"({RESULT_WAIT - left} wait states)")
            pending = {r: (l - waits, d, a) for r, (l, d, a) in pending.items() if l - waits > 0}
            recent = {r: (l - waits, a) for r, (l, a) in recent.items() if l - waits > 0}
            for r in dregs:
                pending[r] = (RESULT_WAIT_BY_OP.get(op, RESULT_WAIT), key, no)
            continue
        if op != "s_nop":
            touched = set()
            for o in ops:
                touched |= _regs(o)
            for r in touched:
                if r in pending:
                    left, pdst, at = pending[r]
                    problems.add(f"line {no}: '{text}' touches MFMA result {pdst} of line {at} "
                                 f"{RESULT_WAIT - left} wait states after issue")
        pending = {r: (l - waits, d, a) for r, (l, d, a) in pending.items() if l - waits > 0}
        recent = {r: (l - waits, a) for r, (l, a) in recent.items() if l - waits > 0}
        if op.startswith("v_") and ops:
            for r in _regs(ops[0]):
                recent[r] = (OPERAND_WAIT, no)
    return pending, recent


def _merge(a, b):
    out = dict(a)
    for r, v in b.items():
        if r not in out or v[0] > out[r][0]:
            out[r] = v
    return out


def check_body(lines):
    """Return a sorted list of hazard descriptions for one function body."""
    blocks = _blocks(lines)
    n = len(blocks)
    entry_p = [dict() for _ in range(n)]
    entry_r = [dict() for _ in range(n)]
    problems = set()
    work = list(range(n))
    seen = set()
    while work:
        i = work.pop(0)
        label, insts, succ = blocks[i]
        p, r = _run_block(insts, entry_p[i], entry_r[i], problems)
        for j in succ:
            np_, nr = _merge(entry_p[j], p), _merge(entry_r[j], r)
            if (np_ != entry_p[j] or nr != entry_r[j]) or j not in seen:
                entry_p[j], entry_r[j] = np_, nr
                seen.add(j)
                if j not in work:
                    work.append(j)
        seen.add(i)
    return sorted(problems)


def check_asm(asm_text, name_filter=None):
    """Map function name -> hazard list for every function whose name contains name_filter."""
    res = {}
    for name, body in kernel_bodies(asm_text):
        if name_filter and name_filter not in name:
            continue
        res[name] = check_body(body)
    return res
