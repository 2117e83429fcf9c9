"""Static check of the hand-placed waits after inline-assembly loads.

The decode and dense kernels issue some loads as inline assembly (Q rows with
global_load_dwordx4, V operands with the transposing LDS read
ds_read_b64_tr_b16) so that the compiler does not wait for every buffer load
in flight before using them. The compiler then treats the destination
registers as written at once: nothing stops it from reading, copying or
reusing them before the wait placed by hand. This module checks, on the AMD
GPU assembly of this repository's own build, that on every control-flow path
from such a load to any instruction touching one of its destination registers
there is an s_waitcnt that covers the load.

Model (GFX9 counters, as on gfx950):
  * an LDS read is complete after `s_waitcnt lgkmcnt(M)` when at least M LDS
    operations (ds_*) were issued after it on that path (LDS operations complete
    in order; scalar memory loads share the counter but may complete in any
    order, so they are not counted). The transposing V reads are waited for
    with constant counts, so this is checked exactly;
  * a vector-memory load (the Q rows) is waited for with a count the kernel
    picks at run time (the number of pool fetches it issued after the Q load,
    dispatched to one of several s_waitcnt immediates), which no path-insensitive
    analysis can follow. What is checked is the compiler's part: on every path
    the registers are untouched until an `s_waitcnt` with a vmcnt field has
    executed. That the run-time count covers the Q load is a property of the
    kernel source (the count never exceeds the fetches issued after Q);
  * where paths meet, a load pending on any of them is pending, with the
    smallest count of younger operations;
  * the compiler routes multi-way branches through 64-bit flag registers set to
    -1 or 0 (s_mov_b64) and tested with s_and_b64 / s_andn2_b64 vcc, exec, flag
    followed by s_cbranch_vccz / vccnz. Those flag values are tracked along each
    path (with exec taken as nonzero, as it is in the wave-uniform code where the
    waits are dispatched), so edges that contradict them are not followed;
    anything else that writes a flag register forgets its value.
Violations are any read or write of a destination register while its load may
still be in flight.
"""
from __future__ import annotations

import dataclasses
import re
from typing import Dict, FrozenSet, List, Optional, Tuple

_FUNC = re.compile(r"^([A-Za-z_.$][\w.$]*):\s*(;.*)?$")
_LABEL = re.compile(r"^(\.L\w+):")
_VRANGE = re.compile(r"\bv\[(\d+):(\d+)\]")
_VREG = re.compile(r"\bv(\d+)\b")
_WAIT_FIELD = re.compile(r"(vmcnt|lgkmcnt|expcnt)\((\d+)\)")
_BRANCHES = ("s_branch", "s_cbranch_")
_CAP = 64


@dataclasses.dataclass
class Inst:
    line: int
    op: str
    args: str
    in_asm: bool


@dataclasses.dataclass
class Block:
    label: Optional[str]
    insts: List[Inst]
    succ: List[int] = dataclasses.field(default_factory=list)
    loop_header: bool = False


@dataclasses.dataclass
class Function:
    name: str
    blocks: List[Block]
    scratch: Optional[int] = None


def vregs(text: str) -> FrozenSet[int]:
    """VGPR numbers named in an operand string."""
    regs = set()
    for a, b in _VRANGE.findall(text):
        regs.update(range(int(a), int(b) + 1))
    text = _VRANGE.sub(" ", text)
    regs.update(int(x) for x in _VREG.findall(text))
    return frozenset(regs)


def parse(asm_text: str) -> List[Function]:
    """Functions of an AMDGPU assembly file, split into basic blocks."""
    funcs: List[Function] = []
    cur: Optional[Function] = None
    in_asm = False
    block: Optional[Block] = None
    scratch_re = re.compile(r"^; ScratchSize: (\d+)")
    pending_scratch: Optional[int] = None
    for no, raw in enumerate(asm_text.splitlines(), 1):
        line = raw.rstrip()
        m = scratch_re.match(line)
        if m and funcs:
            funcs[-1].scratch = int(m.group(1))
            continue
        if cur is None:
            m = _FUNC.match(line)
            if m and not line.startswith(".") and not line.startswith("\t"):
                cur = Function(m.group(1), [])
                block = Block(None, [])
                cur.blocks.append(block)
                in_asm = False
            continue
        if line.startswith(".Lfunc_end"):
            funcs.append(cur)
            cur = None
            continue
        s = line.strip()
        if s.startswith(";;#ASMSTART"):
            in_asm = True
            continue
        if s.startswith(";;#ASMEND"):
            in_asm = False
            continue
        m = _LABEL.match(line)
        if m:
            block = Block(m.group(1), [], loop_header="Loop Header" in line)
            cur.blocks.append(block)
            continue
        if not s or s.startswith(";") or s.startswith("."):
            continue
        code = s.split(";", 1)[0].strip()
        if not code:
            continue
        parts = code.split(None, 1)
        inst = Inst(no, parts[0], parts[1] if len(parts) > 1 else "", in_asm)
        block.insts.append(inst)
        if inst.op.startswith(_BRANCHES) or inst.op == "s_endpgm" or inst.op.startswith("s_setpc"):
            block = Block(None, [])
            cur.blocks.append(block)
    # successors
    for f in funcs:
        index = {b.label: i for i, b in enumerate(f.blocks) if b.label}
        for i, b in enumerate(f.blocks):
            last = b.insts[-1] if b.insts else None
            nxt = i + 1 if i + 1 < len(f.blocks) else None
            if last is None:
                b.succ = [nxt] if nxt is not None else []
            elif last.op == "s_endpgm" or last.op.startswith("s_setpc"):
                b.succ = []
            elif last.op == "s_branch":
                b.succ = [index[last.args.split()[0]]]
            elif last.op.startswith("s_cbranch_"):
                b.succ = [index[last.args.split()[0]]] + ([nxt] if nxt is not None else [])
            else:
                b.succ = [nxt] if nxt is not None else []
    return funcs


def _kind(op: str) -> Optional[str]:
    if op.startswith(("buffer_load", "global_load")):
        return "vm"
    if op.startswith("ds_"):
        return "lgkm"
    return None


# pending load: site line -> (counter kind, destination registers, younger ops)
Pending = Dict[int, Tuple[str, FrozenSet[int], int]]
_SPAIR = re.compile(r"^s\[(\d+):(\d+)\]$")
_SREG = re.compile(r"\bs\[(\d+):(\d+)\]|\bs(\d+)\b")


_MAX_FLAGS = 4  # flag assignments tracked at once (the most recent ones)


@dataclasses.dataclass(frozen=True)
class State:
    pending: Tuple[Tuple[int, Tuple[str, FrozenSet[int], int]], ...]
    flags: Tuple[Tuple[int, int], ...]  # first SGPR of a pair -> -1 or 0 (sorted)
    vcc: Optional[int]  # 0: vcc is zero, 1: vcc is nonzero, None: unknown
    order: Tuple[int, ...] = ()  # the flags' registers, oldest assignment first

    @staticmethod
    def make(pending: Pending, flags: Dict[int, int], vcc: Optional[int]) -> "State":
        return State(tuple(sorted(pending.items())), tuple(sorted(flags.items())), vcc,
                     tuple(flags))

    @property
    def flags_in_order(self) -> Dict[int, int]:
        d = dict(self.flags)
        return {k: d[k] for k in self.order}

    def forget_flags(self) -> "State":
        return State(self.pending, (), None, ())


def _merge(a: State, b: State) -> State:
    out = dict(a.pending)
    for k, (kind, regs, n) in b.pending:
        out[k] = (kind, regs, min(out[k][2], n)) if k in out else (kind, regs, n)
    fa, fb = a.flags_in_order, dict(b.flags)
    flags = {k: v for k, v in fa.items() if fb.get(k) == v}
    return State.make(out, flags, a.vcc if a.vcc == b.vcc else None)


def _sgprs(text: str) -> FrozenSet[int]:
    regs = set()
    for a, b, c in _SREG.findall(text):
        regs.update(range(int(a), int(b) + 1) if a else [int(c)])
    return frozenset(regs)


def _step(state: State, inst: Inst, violations: List[str], fname: str) -> State:
    pending: Pending = dict(state.pending)
    flags = dict(state.flags_in_order)
    vcc = state.vcc
    ops = [x.strip() for x in inst.args.split(",")] if inst.args else []
    # flag registers and vcc
    first = ops[0] if ops else ""
    if inst.op.startswith("s_") and first:
        if first == "vcc":
            vcc = None
            if inst.op in ("s_and_b64", "s_andn2_b64") and len(ops) == 3 and ops[1] == "exec":
                m = _SPAIR.match(ops[2])
                if m and int(m.group(1)) in flags:
                    f = flags[int(m.group(1))]
                    bit = (f != 0) if inst.op == "s_and_b64" else (f == 0)
                    vcc = 1 if bit else 0
        else:
            hit = _sgprs(first)
            for k in [k for k in flags if k in hit or k + 1 in hit]:
                del flags[k]
            m = _SPAIR.match(first)
            if inst.op == "s_mov_b64" and m and len(ops) == 2 and ops[1] in ("-1", "0"):
                flags[int(m.group(1))] = int(ops[1])
                while len(flags) > _MAX_FLAGS:  # keep the most recent assignments
                    del flags[next(iter(flags))]
    elif inst.op.startswith("v_cmp") and (inst.op.endswith("_e32") or first == "vcc"):
        vcc = None  # a compare that writes vcc
    if inst.op == "s_waitcnt":
        fields = dict((k, int(v)) for k, v in _WAIT_FIELD.findall(inst.args))
        raw = inst.args.strip()
        if raw and (raw.isdigit() or raw.startswith("0x")):
            fields = {"vmcnt": 0, "lgkmcnt": 0} if int(raw, 0) == 0 else {}
        out = {}
        for k, (kind, regs, n) in pending.items():
            lim = fields.get("vmcnt" if kind == "vm" else "lgkmcnt")
            if lim is not None and (kind == "vm" or n >= lim):
                continue
            out[k] = (kind, regs, n)
        return State.make(out, flags, vcc)
    used = vregs(inst.args)
    if used:
        for k, (kind, regs, n) in pending.items():
            hit = used & regs
            if hit:
                violations.append(f"{fname}: v{min(hit)} of the load at line {k} is touched at "
                                  f"line {inst.line} ({inst.op}) before a covering wait")
    kind = _kind(inst.op)
    out = dict(pending)
    if kind is not None and not inst.op.startswith(("buffer_store", "global_store")):
        for k, (kk, regs, n) in pending.items():
            if kk == kind:
                out[k] = (kk, regs, min(_CAP, n + 1))
    if inst.in_asm and kind is not None and "store" not in inst.op and "write" not in inst.op:
        if "lds" not in inst.args.split():  # a buffer-to-LDS load writes no VGPR
            out[inst.line] = (kind, vregs(ops[0]), 0)
    return State.make(out, flags, vcc)


def _edges(block: Block, st: State) -> List[int]:
    """Successors that the tracked vcc value does not rule out."""
    last = block.insts[-1] if block.insts else None
    if last is None or not last.op.startswith("s_cbranch_vcc") or st.vcc is None:
        return block.succ
    taken = (st.vcc == 0) if last.op == "s_cbranch_vccz" else (st.vcc == 1)
    target, rest = block.succ[0], block.succ[1:]
    return [target] if taken else rest


def check_function(f: Function, max_states: int = 256) -> List[str]:
    """Violations in one function (empty if every inline-asm load is waited for).

    Each block keeps one state per distinct assignment of the tracked flag
    registers and vcc (states that agree on them are merged), so paths that
    set a flag differently are not mixed before it is tested."""
    n = len(f.blocks)
    entry: List[Dict[tuple, State]] = [dict() for _ in range(n)]
    start = State.make({}, {}, None)
    entry[0][(start.flags, start.vcc)] = start
    work = [(0, (start.flags, start.vcc))]
    violations: List[str] = []
    seen_viol = set()
    while work:
        i, key = work.pop()
        st = entry[i][key]
        local: List[str] = []
        for inst in f.blocks[i].insts:
            st = _step(st, inst, local, f.name)
        for v in local:
            if v not in seen_viol:
                seen_viol.add(v)
                violations.append(v)
        for s_ in _edges(f.blocks[i], st):
            nst = st.forget_flags() if f.blocks[s_].loop_header else st
            k = (nst.flags, nst.vcc)
            old = entry[s_].get(k)
            new = nst if old is None else _merge(old, nst)
            if new != old:
                if old is None and len(entry[s_]) >= max_states:
                    raise RuntimeError(f"{f.name}: more than {max_states} flag states at a block")
                entry[s_][k] = new
                work.append((s_, k))
    return violations


def asm_load_functions(funcs: List[Function]) -> List[Function]:
    """Functions that issue loads from inline assembly."""
    out = []
    for f in funcs:
        if any(i.in_asm and _kind(i.op) and "lds" not in i.args.split()
               for b in f.blocks for i in b.insts):
            out.append(f)
    return out
