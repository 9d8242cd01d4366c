"""Static check of gfx9 device assembly: no instruction touches a register whose vector
memory load is still in flight.

The kernels issue some global loads from inline assembly and wait for them with explicit
``s_waitcnt vmcnt(N)``.  The compiler does not know such a load writes its destination
later than the instruction issues, so it could move arithmetic on the value above the
wait, copy the register early, or hand the register to another value while the data is
still on its way (the late write then corrupts that value, possibly an address).  This
module replays the vector-memory counter over the control-flow graph of each kernel in
the assembly that hipcc emits and reports every such access.

Model (the one the compiler's own wait insertion uses on gfx9): every vector memory
instruction (load, store, atomic, LDS-DMA load) takes one slot of the counter; they
complete in issue order; ``s_waitcnt vmcnt(N)`` leaves at most the N newest in flight;
at most 63 are in flight (issue stalls beyond that).  A load's destination registers are
pending while its slot is in flight.  At a block with several predecessors the pending
state is the slot-wise union, aligned on the newest slot, so a register pending on any
path counts as pending.

Lanes: the check is per register, not per lane, with one refinement.  The compiler puts
``s_cbranch_execz`` skips after code that leaves the exec mask alone; that edge is taken
only with exec all zero, and a load issued since the last write of exec then had no lane
active and writes nothing, so along an exec-zero edge such loads no longer count.
"""
from __future__ import annotations

import re
from dataclasses import dataclass, field

_VMEM_PREFIX = ("global_", "buffer_", "flat_", "scratch_")
_REG_RANGE = re.compile(r"\b([va])\[(\d+):(\d+)\]")
_REG_ONE = re.compile(r"\b([va])(\d+)\b")
_VMCNT = re.compile(r"vmcnt\((\d+)\)")
_LABEL = re.compile(r"^([.\w$]+):")
_MAX_INFLIGHT = 63


def regs_of(text: str) -> set[tuple[str, int]]:
    """VGPRs and AGPRs named in an operand string, as (file, index) pairs."""
    out: set[tuple[str, int]] = set()
    for f, lo, hi in _REG_RANGE.findall(text):
        out.update((f, i) for i in range(int(lo), int(hi) + 1))
    text = _REG_RANGE.sub(" ", text)
    for f, i in _REG_ONE.findall(text):
        out.add((f, int(i)))
    return out


@dataclass
class Insn:
    line: int
    op: str
    operands: str


@dataclass
class Block:
    label: str | None
    insns: list[Insn] = field(default_factory=list)
    succ: list[tuple[int, bool]] = field(default_factory=list)  # (block, exec all zero on the edge)


def split_functions(asm: str) -> dict[str, list[tuple[int, str]]]:
    """Kernel bodies (symbol -> numbered lines) from the text between a kernel's label
    and its .Lfunc_end label."""
    funcs: dict[str, list[tuple[int, str]]] = {}
    lines = asm.splitlines()
    kernels = set(re.findall(r"^\s*\.type\s+([\w$.]+),@function", asm, re.M))
    cur = None
    for n, raw in enumerate(lines, 1):
        m = _LABEL.match(raw)
        if m and m.group(1) in kernels:
            cur = m.group(1)
            funcs[cur] = []
            continue
        if cur is None:
            continue
        if m and m.group(1).startswith(".Lfunc_end"):
            cur = None
            continue
        funcs[cur].append((n, raw))
    return funcs


def build_cfg(body: list[tuple[int, str]]) -> list[Block]:
    blocks: list[Block] = [Block(None)]
    for n, raw in body:
        text = raw.split(";", 1)[0].rstrip()
        if not text.strip():
            continue
        m = _LABEL.match(text.strip())
        if m:
            if blocks[-1].insns or blocks[-1].label is not None:
                blocks.append(Block(m.group(1)))
            else:
                blocks[-1].label = m.group(1)
            continue
        s = text.strip()
        if s.startswith("."):
            continue  # directive
        op, _, rest = s.partition(" ")
        blocks[-1].insns.append(Insn(n, op, rest.strip()))
        if op.startswith("s_branch") or op.startswith("s_cbranch") or op in ("s_endpgm", "s_setpc_b64"):
            blocks.append(Block(None))
    index = {b.label: i for i, b in enumerate(blocks) if b.label}
    for i, b in enumerate(blocks):
        last = b.insns[-1] if b.insns else None
        nxt = i + 1 if i + 1 < len(blocks) else None
        if last is None or not (last.op.startswith("s_branch") or last.op.startswith("s_cbranch")
                                or last.op in ("s_endpgm", "s_setpc_b64")):
            b.succ = [(nxt, False)] if nxt is not None else []
        elif last.op == "s_branch":
            b.succ = [(index[last.operands.split()[0]], False)]
        elif last.op.startswith("s_cbranch"):
            tgt = index[last.operands.split()[0]]
            b.succ = [(tgt, last.op == "s_cbranch_execz")]
            if nxt is not None:
                b.succ.append((nxt, last.op == "s_cbranch_execnz"))
        else:
            b.succ = []
    return blocks


def _is_vmem(op: str) -> bool:
    return op.startswith(_VMEM_PREFIX)


def _load_dst(insn: Insn) -> set[tuple[str, int]]:
    """Registers a vector memory instruction writes when its data returns."""
    op = insn.op
    mods = set(insn.operands.replace(",", " ").split())
    if "_lds" in op or "store" in op or "lds" in mods:  # LDS-DMA forms write LDS, not VGPRs
        return set()
    first = insn.operands.split(",", 1)[0]
    # an atomic returns the old value only with glc (gfx9) or sc0 (gfx940 and later)
    if "atomic" in op and not ({"glc", "sc0"} & mods):
        return set()
    return regs_of(first)


# A state is a tuple of slots, oldest first; a slot is (registers it will write, whether
# it was issued after the last write of exec on every path reaching here).
State = tuple
_EMPTY = (frozenset(), False)


def _merge(a: State, b: State) -> State:
    if len(a) < len(b):
        a, b = b, a
    pad = (_EMPTY,) * (len(a) - len(b)) + tuple(b)
    return tuple((x[0] | y[0], x[1] and y[1]) for x, y in zip(a, pad))


def _pending(state: State) -> set[tuple[str, int]]:
    out: set[tuple[str, int]] = set()
    for regs, _ in state:
        out |= regs
    return out


def _writes_exec(insn: Insn) -> bool:
    if "saveexec" in insn.op or insn.op.startswith("v_cmpx"):
        return True
    first = insn.operands.split(",", 1)[0].strip()
    return first in ("exec", "exec_lo", "exec_hi")


def _exec_zero(state: State) -> State:
    """The state along an edge taken only when exec is all zero."""
    return tuple((frozenset(), True) if fresh else (regs, fresh) for regs, fresh in state)


def _step(state: State, insn: Insn, report) -> State:
    if insn.op == "s_waitcnt":
        m = _VMCNT.search(insn.operands)
        if m:
            n = int(m.group(1))
            state = state[len(state) - n:] if n < len(state) else state
            if n == 0:
                state = ()
        return state
    used = regs_of(insn.operands)
    dst = _load_dst(insn) if _is_vmem(insn.op) else set()
    if dst:
        # a load may target a register whose earlier load is still in flight: loads
        # complete in order, so the later value lands last (its address and data
        # operands still count)
        used = regs_of(insn.operands.split(",", 1)[1] if "," in insn.operands else "")
    hit = used & _pending(state)
    if hit and report is not None:
        report(insn, hit)
    if _is_vmem(insn.op):
        state = state + ((frozenset(dst), True),)
        if len(state) > _MAX_INFLIGHT:
            state = state[len(state) - _MAX_INFLIGHT:]
    if _writes_exec(insn):
        state = tuple((regs, False) for regs, _ in state)
    return state


def check_function(body: list[tuple[int, str]]) -> list[str]:
    """Accesses to in-flight load destinations in one kernel, as readable strings."""
    blocks = build_cfg(body)
    entry: list[State | None] = [None] * len(blocks)
    entry[0] = ()
    work = [0]
    while work:
        i = work.pop()
        st = entry[i]
        for insn in blocks[i].insns:
            st = _step(st, insn, None)
        for j, zero in blocks[i].succ:
            out = _exec_zero(st) if zero else st
            new = out if entry[j] is None else _merge(entry[j], out)
            if new != entry[j]:
                entry[j] = new
                work.append(j)
    found: list[str] = []

    def report(insn: Insn, hit):
        regs = ", ".join("%s%d" % r for r in sorted(hit))
        found.append("line %d: %s %s  <- in flight: %s" % (insn.line, insn.op, insn.operands, regs))

    for i, b in enumerate(blocks):
        if entry[i] is None:
            continue
        st = entry[i]
        for insn in b.insns:
            st = _step(st, insn, report)
    return found


def check_asm(asm: str) -> dict[str, list[str]]:
    """Kernel symbol -> its accesses to in-flight load destinations (empty if none)."""
    return {name: check_function(body) for name, body in split_functions(asm).items()}
