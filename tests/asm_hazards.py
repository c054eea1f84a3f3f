"""Static check of hand-written LDS reads in gfx950 assembly.

The kernels issue some LDS reads (ds_read_b128, ds_read_b64_tr_b16) as inline
assembly so that the compiler does not wait for the LDS copies in flight
before each of them.  The compiler then treats the destination registers as
written when the instruction issues, although the hardware writes them when
the read returns, after the next s_waitcnt that covers it.  Any other
instruction that reads or writes one of those registers in between sees or
leaves the wrong value: an accumulator copied into such a register before the
wait is overwritten by the late read.

check_function() walks one kernel's assembly (the text between its label and
its .Lfunc_end) as a control-flow graph: a pending-register state flows along
fall-through and branch edges until it is stable.  An inline-assembly LDS read
adds its destination registers to the pending set; an s_waitcnt with
lgkmcnt(0) clears the set (lgkmcnt(n), n > 0, clears the reads older than the
n most recent LGKM operations when the order is known, else nothing); any
other instruction naming a pending VGPR is reported (another such LDS read may
target one, since LDS reads return in issue order, but not read one as its
address).
"""
import re

_LABEL = re.compile(r"^(\.LBB\d+_\d+|[A-Za-z_.$][\w.$]*):")
_VREG = re.compile(r"(?<![\w\[])v(\d+)\b|(?<![\w])v\[(\d+):(\d+)\]")
_LGKM = re.compile(r"lgkmcnt\((\d+)\)")
_ASM_READ = re.compile(r"^(ds_read_b128|ds_read_b64_tr_b16|ds_read_b64|ds_read_b96|ds_read_b32|"
                       r"ds_read_u16|ds_read2_b32|ds_read2_b64|ds_read_tr\w*)\s")
_LGKM_OPS = re.compile(r"^(ds_|s_load|s_buffer_load|s_sendmsg|s_memtime|s_memrealtime|s_dcache)")
_BRANCH = re.compile(r"^s_(c?branch\w*)\s+(\S+)")


def _regs(text):
    out = set()
    for m in _VREG.finditer(text):
        if m.group(1) is not None:
            out.add(int(m.group(1)))
        else:
            out.update(range(int(m.group(2)), int(m.group(3)) + 1))
    return out


def _parse(lines):
    """(instructions, label -> index); an instruction is (text, in_asm)."""
    instrs, labels = [], {}
    in_asm = False
    for raw in lines:
        line = raw.split(";", 1)[0].strip() if not raw.strip().startswith(";;#ASM") else raw.strip()
        if line == ";;#ASMSTART":
            in_asm = True
            continue
        if line == ";;#ASMEND":
            in_asm = False
            continue
        if not line:
            continue
        m = _LABEL.match(line)
        if m:
            labels[m.group(1)] = len(instrs)
            continue
        if line.startswith("."):
            continue
        instrs.append((line, in_asm))
    return instrs, labels


def _successors(i, instrs, labels):
    text = instrs[i][0]
    m = _BRANCH.match(text)
    if m:
        target = labels.get(m.group(2))
        succ = [target] if target is not None else []
        if m.group(1) != "branch":        # conditional: also falls through
            succ.append(i + 1)
        return succ
    if text.startswith("s_endpgm") or text.startswith("s_setpc") or text.startswith("s_trap"):
        return []
    return [i + 1]


def _merge(a, b):
    """States are (ordered tuple of LGKM ops, unordered frozenset); an op is a
    frozenset of pending registers (empty for an LGKM op that writes none we
    track)."""
    if a is None:
        return b
    if a == b:
        return a
    regs = set(a[1]) | set(b[1])
    for st in (a, b):
        for op in st[0]:
            regs |= op
    return ((), frozenset(regs))


def check_function(lines):
    """Hazards in one function: a list of (instruction index, instruction, registers)."""
    instrs, labels = _parse(lines)
    n = len(instrs)
    state_in = [None] * (n + 1)
    state_in[0] = ((), frozenset())
    work = [0]
    hazards = {}
    while work:
        i = work.pop()
        if i >= n:
            continue
        ops, fuzzy = state_in[i]
        text, in_asm = instrs[i]
        pending = set(fuzzy)
        for op in ops:
            pending |= op
        # hazard check: any instruction naming a pending register, except the
        # LGKM instruction that defines it (reported once per instruction)
        is_asm_read = in_asm and _ASM_READ.match(text)
        # LDS reads return in issue order, so a later read may target a
        # pending register; its address operand must not be pending
        named = _regs(text.split(",", 1)[1]) if is_asm_read and "," in text else _regs(text)
        touched = named & pending
        if touched and not text.startswith("s_waitcnt"):
            hazards[i] = (text, sorted(touched))
        # state update
        if text.startswith("s_waitcnt"):
            m = _LGKM.search(text)
            if m:
                keep = int(m.group(1))
                if keep == 0:
                    ops, fuzzy = (), frozenset()
                else:
                    ops = ops[len(ops) - keep:] if len(ops) > keep else ops
        elif is_asm_read:
            dest = text.split(None, 1)[1].split(",")[0]
            ops = ops + (frozenset(_regs(dest)),)
        elif _LGKM_OPS.match(text):
            ops = ops + (frozenset(),)
        new = (ops, fuzzy)
        for s in _successors(i, instrs, labels):
            merged = _merge(state_in[s], new)
            if merged != state_in[s]:
                state_in[s] = merged
                work.append(s)
    return [(i, hazards[i][0], hazards[i][1]) for i in sorted(hazards)]


def functions(asm_text):
    """{kernel symbol: its lines} for every function in an assembly file."""
    out = {}
    cur, buf = None, []
    for line in asm_text.splitlines():
        if cur is None:
            m = re.match(r"^(_Z\w+):", line)
            if m:
                cur, buf = m.group(1), []
            continue
        if line.startswith(".Lfunc_end"):
            out[cur] = buf
            cur = None
            continue
        buf.append(line)
    return out


def check_file(asm_text):
    """{kernel symbol: hazards} for the kernels of one assembly file that have any."""
    res = {}
    for name, lines in functions(asm_text).items():
        h = check_function(lines)
        if h:
            res[name] = h
    return res
