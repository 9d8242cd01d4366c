"""Static check of gfx9 device assembly: no instruction touches a register whose vector
memory load is still in flight, and no LDS access happens while an earlier group of
LDS-DMA copies may still be landing.

Loads issued from inline assembly and waited for with explicit ``s_waitcnt vmcnt(N)`` are
invisible to the compiler: it could move arithmetic on the value above the wait, copy the
register early, or hand the register to another value while the data is still on its way
(the late write then corrupts that value, possibly an address).  The attention kernel's
direct global-to-LDS copies (``global_load_lds_dwordx4`` from inline assembly) are waited
for by hand the same way; there the hazard is an LDS read of a tile that is still being
copied.  This module replays the vector-memory counter over the control-flow graph of each
kernel in the assembly that hipcc emits and reports every such access.

LDS copies are checked by groups: a run of LDS-DMA instructions with no LDS access and no
``s_waitcnt`` on vmcnt between them is one group (one tile's rows; waits on lgkmcnt alone,
for the scalar loads of row addresses, may sit inside it), and a new group makes the ones
before it "earlier".  A kernel that double-buffers tiles waits, after issuing a group, for
everything before it and then reads the tile that has landed; so after every ``s_waitcnt``
that follows a copy group, each LDS access (``ds_*`` other than the lane permutes) up to the
next copy must find no copy of an earlier group in flight: at most the newest group is
landing, into the other half of the buffer (the half is the kernel's construction; the check
sees counts, not addresses).  This is the wait a miscount would break.

Model (the one the compiler's own wait insertion uses on gfx9): every vector memory
instruction (load, store, atomic, LDS-DMA load) takes one slot of the counter; they
complete in issue order; ``s_waitcnt vmcnt(N)`` leaves at most the N newest in flight;
at most 63 are in flight (issue stalls beyond that).  A load's destination registers are
pending while its slot is in flight.  The replay is path-sensitive: each distinct state
reaching a block is carried on by itself, never joined with another (joining the slot
lists of two paths lines up loads of different tiles and invents hazards), so the check
sees every path through the kernel's branches and loops that the counter model can tell
apart.  Only where a block is reached in more than a few hundred distinct states (long
loops of stores, say) are the rest joined: slot-wise union aligned on the newest slot, so
a register pending on any of those paths counts as pending there (coarser, never blind).

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


# A state is (slots, open, waited): slots oldest first, each (registers it will write,
# whether it was issued after the last write of exec on every path reaching here, copy
# group: 0 not an LDS copy, 1 the newest group, 2 an earlier group); open is whether the
# newest copy group may still grow (no LDS access or wait since its last copy); waited is
# whether an s_waitcnt has come since the last copy (LDS accesses are checked then).
State = tuple
_EMPTY = (frozenset(), False, 0)
_NO_LDS = ("ds_bpermute", "ds_permute", "ds_swizzle")


def _merge(a: State, b: State) -> State:
    """Join of two states (sound, coarser): slots aligned on the newest, registers united."""
    (sa, oa, wa), (sb, ob, wb) = a, b
    if len(sa) < len(sb):
        sa, sb = sb, sa
    pad = (_EMPTY,) * (len(sa) - len(sb)) + tuple(sb)
    return (tuple((x[0] | y[0], x[1] and y[1], max(x[2], y[2])) for x, y in zip(sa, pad)), oa and ob, wa or wb)


def _pending(slots) -> set[tuple[str, int]]:
    out: set[tuple[str, int]] = set()
    for regs, _, _ in slots:
        out |= regs
    return out


def _is_lds_copy(insn: Insn) -> bool:
    return _is_vmem(insn.op) and ("_lds" in insn.op or "lds" in set(insn.operands.replace(",", " ").split()))


def _is_lds_access(insn: Insn) -> bool:
    return insn.op.startswith("ds_") and not insn.op.startswith(_NO_LDS)


def _writes_exec(insn: Insn) -> bool:
    if "saveexec" in insn.op or insn.op.startswith("v_cmpx"):
        return True
    first = insn.operands.split(",", 1)[0].strip()
    return first in ("exec", "exec_lo", "exec_hi")


def _exec_zero(state: State) -> State:
    """The state along an edge taken only when exec is all zero (such instructions had no
    lane active: they write no register and copy nothing)."""
    slots, op, wt = state
    return (tuple((frozenset(), True, 0) if fresh else (regs, fresh, g) for regs, fresh, g in slots), op, wt)


def _step(state: State, insn: Insn, report) -> State:
    slots, open_, waited = state
    if insn.op == "s_waitcnt":
        m = _VMCNT.search(insn.operands)
        if m:
            n = int(m.group(1))
            slots = slots[len(slots) - n:] if n < len(slots) else slots
            if n == 0:
                slots = ()
            return (slots, False, True)
        # a wait on lgkmcnt alone (scalar loads, LDS reads) neither lands a copy nor
        # touches LDS: the copies around it still form one group
        return (slots, open_, waited)
    used = regs_of(insn.operands)
    dst = _load_dst(insn) if _is_vmem(insn.op) else set()
    if dst:
        # a load may target a register whose earlier load is still in flight: loads
        # complete in order, so the later value lands last (its address and data
        # operands still count)
        used = regs_of(insn.operands.split(",", 1)[1] if "," in insn.operands else "")
    hit = used & _pending(slots)
    if hit and report is not None:
        report(insn, hit)
    if _is_lds_access(insn):
        if report is not None and waited and any(g == 2 for _, _, g in slots):
            report(insn, None)
        open_ = False
    if _is_vmem(insn.op):
        group = 0
        if _is_lds_copy(insn):
            if not open_:  # a new group: the ones before it become earlier groups
                slots = tuple((r, f, 2 if g else 0) for r, f, g in slots)
            group, open_, waited = 1, True, False
        slots = slots + ((frozenset(dst), True, group),)
        if len(slots) > _MAX_INFLIGHT:
            slots = slots[len(slots) - _MAX_INFLIGHT:]
    if _writes_exec(insn):
        slots = tuple((regs, False, g) for regs, _, g in slots)
    return (slots, open_, waited)


def check_function(body: list[tuple[int, str]], exact_per_block: int = 256) -> list[str]:
    """Accesses to in-flight load destinations in one kernel, as readable strings.

    Path-sensitive: up to exact_per_block distinct states reaching a block are carried on
    one by one (joining the slot lists of two paths lines up loads that belong to different
    tiles and invents hazards).  Beyond that budget a block's further states are joined into
    one widened state, which covers them all, so the replay ends on any kernel."""
    blocks = build_cfg(body)
    seen: list[set] = [set() for _ in blocks]
    wide: list[State | None] = [None] * len(blocks)
    init: State = ((), False, False)
    seen[0].add(init)
    work = [(0, init)]
    found: dict[int, str] = {}

    def report(insn: Insn, hit):
        if hit is None:
            found.setdefault(insn.line, "line %d: %s %s  <- an earlier LDS copy group may still be landing"
                             % (insn.line, insn.op, insn.operands))
            return
        regs = ", ".join("%s%d" % r for r in sorted(hit))
        found.setdefault(insn.line, "line %d: %s %s  <- in flight: %s" % (insn.line, insn.op, insn.operands, regs))

    while work:
        i, st = work.pop()
        for insn in blocks[i].insns:
            st = _step(st, insn, report)
        for j, zero in blocks[i].succ:
            out = _exec_zero(st) if zero else st
            if out in seen[j] or out == wide[j]:
                continue
            if len(seen[j]) < exact_per_block:
                seen[j].add(out)
                work.append((j, out))
                continue
            joined = out if wide[j] is None else _merge(wide[j], out)
            if joined != wide[j]:
                wide[j] = joined
                work.append((j, joined))
    return [found[k] for k in sorted(found)]


def check_asm(asm: str) -> dict[str, list[str]]:
    """Kernel symbol -> its accesses to in-flight load destinations and LDS accesses under
    an earlier copy group (empty if none)."""
    return {name: check_function(body) for name, body in split_functions(asm).items()}
