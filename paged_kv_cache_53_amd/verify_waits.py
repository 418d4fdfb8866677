"""Static check of the decode kernel's explicitly waited loads, run on the compiled device assembly.

The persistent decode kernel issues its tile loads, its early q loads and its work-claim atomic
through inline assembly, outside the compiler's wait tracking, and waits for them with explicit
``s_waitcnt vmcnt(N)`` instructions.  That is only correct if no compiled instruction touches a
destination register of such an operation while it may still be in flight: a copy, spill or
temporary in one of those registers would read data that has not arrived, or be overwritten by it.

This module walks every basic block of each kernel with a per-register distance: the number of
vector-memory instructions issued since the register's pending inline-asm load or atomic.
``s_waitcnt vmcnt(N)`` retires every operation with at least N issued after it (vmcnt counts
loads, stores and atomics, which retire in order).  At a join, each register keeps its smallest
distance, and the walk repeats to a fixed point.  Any non-asm instruction that reads or writes a
register with a pending asm operation is reported, except a readfirstlane: the compiler materialises
undefined scalar values that way on exit paths, so its result is tracked instead (through s_mov
copies) and any other use of it is reported.  Branches on the CFG
structurizer's flag registers are followed only where their constant values allow.  The build
fails on a report.

Usage: python -m paged_kv_cache_53_amd.verify_waits FILE.s [KERNEL_SUBSTRING]
"""
from __future__ import annotations

import re
import sys
from typing import Dict, List, Optional, Set, Tuple

_MAX_CTX = 256   # flag contexts kept apart per block before falling back to one merged state
_CAP = 64  # vmcnt is 6 bits: an operation with 64 issued after it has retired under any wait
_STORE = ("global_store", "buffer_store", "scratch_store", "flat_store")
_VMEM = ("global_", "buffer_", "scratch_", "flat_")
_TO_LDS = ("global_load_lds_", "buffer_load_lds_", "scratch_load_lds_")


_AGPR = 1024   # accumulation registers a0.. are tracked as _AGPR + index


def _regs(tok: str) -> Set[int]:
    """Vector registers named by an operand: v-registers by index, a-registers as _AGPR + index."""
    tok = tok.rstrip(",")
    m = re.match(r"([va])\[(\d+):(\d+)\]$", tok)
    if m:
        base = _AGPR if m.group(1) == "a" else 0
        return set(range(base + int(m.group(2)), base + int(m.group(3)) + 1))
    m = re.match(r"([va])(\d+)$", tok)
    if not m:
        return set()
    return {(_AGPR if m.group(1) == "a" else 0) + int(m.group(2))}


class _Insn:
    __slots__ = ("text", "op", "asm", "reads", "writes", "vmem", "wait", "asm_dst")

    def __init__(self, text: str, asm: bool):
        self.text = text
        parts = text.replace(",", " ").split()
        self.op = parts[0]
        self.asm = asm
        ops = parts[1:]
        self.vmem = self.op.startswith(_VMEM)
        m = re.search(r"vmcnt\((\d+)\)", text) if self.op == "s_waitcnt" else None
        self.wait = int(m.group(1)) if m else None
        if self.op.startswith(_STORE) or self.op.startswith(_TO_LDS) or self.op.endswith("_lds"):
            # stores, and loads that deliver straight into LDS: every register operand is a source
            self.writes, self.reads = set(), set().union(*[_regs(o) for o in ops]) if ops else set()
        elif ops:
            self.writes = _regs(ops[0])
            self.reads = set().union(*[_regs(o) for o in ops[1:]]) if len(ops) > 1 else set()
        else:
            self.writes, self.reads = set(), set()
        # destinations whose arrival the kernel waits for explicitly
        self.asm_dst = self.writes if (asm and self.vmem and self.writes) else set()


def _asm_local_labels(body: List[str]):
    """Numeric local labels ("1:") inside inline-assembly regions, and the resolution of each branch to
    one ("1f": the next such label, "1b": the previous one), as unique block names "asm<line>"."""
    in_asm, defs = False, []
    for i, raw in enumerate(body):
        t = raw.strip()
        if t.startswith(";;#ASMSTART"):
            in_asm = True
        elif t.startswith(";;#ASMEND"):
            in_asm = False
        elif in_asm and re.match(r"^\d+:$", t.split(";")[0].strip()):
            defs.append((i, t.split(";")[0].strip()[:-1]))

    def resolve(i: int, ref: str) -> Optional[str]:
        m = re.match(r"^(\d+)([fb])$", ref)
        if not m:
            return None
        num, d = m.group(1), m.group(2)
        cands = [j for j, n in defs if n == num and (j > i if d == "f" else j < i)]
        if not cands:
            return None
        return f"asm{min(cands) if d == 'f' else max(cands)}"
    return {i for i, _ in defs}, resolve


def _kernel_blocks(body: List[str]):
    """Basic blocks: (label, [insn], successors by label, falls_through)."""
    blocks: List[Tuple[str, List[_Insn], List[str], bool]] = []
    label, insns, in_asm, n = "entry", [], False, 0
    asm_labels, resolve = _asm_local_labels(body)

    def close(next_label: Optional[str]):
        nonlocal label, insns, n
        blocks.append((label, insns, [], True))
        label = next_label or f"anon{n}"
        n += 1
        insns = []

    for li, raw in enumerate(body):
        t = raw.split(";")[0].strip() if not raw.strip().startswith(";;#ASM") else raw.strip()
        if li in asm_labels:
            close(f"asm{li}")
            continue
        if raw.strip().startswith(";;#ASMSTART"):
            in_asm = True
            continue
        if raw.strip().startswith(";;#ASMEND"):
            in_asm = False
            continue
        if raw.strip().startswith("; %bb."):
            if insns:
                close(None)
            continue
        m = re.match(r"^(\.LBB\d+_\d+):", raw.strip())
        if m:
            close(m.group(1))
            continue
        if not t or t.startswith("."):
            continue
        ins = _Insn(t, in_asm)
        if in_asm and (ins.op == "s_branch" or ins.op.startswith("s_cbranch")):
            target = resolve(li, ins.text.split()[1])
            if target is None:
                raise RuntimeError(f"inline-assembly branch with no local label: {ins.text}")
            ins.text = f"{ins.op} {target}"
        insns.append(ins)
        if ins.op in ("s_branch", "s_endpgm", "s_setpc_b64") or ins.op.startswith("s_cbranch"):
            close(None)
    close(None)
    # successors
    out = []
    for i, (lab, ins, _, _) in enumerate(blocks):
        succ: List[str] = []
        last = ins[-1] if ins else None
        fall = True
        if last is not None:
            if last.op == "s_branch":
                succ.append(last.text.split()[1])
                fall = False
            elif last.op.startswith("s_cbranch"):
                succ.append(last.text.split()[1])
            elif last.op in ("s_endpgm", "s_setpc_b64"):
                fall = False
        if fall and i + 1 < len(blocks):
            succ.append(blocks[i + 1][0])
        out.append((lab, ins, succ))
    return out


def _sregs(tok: str) -> List[int]:
    tok = tok.rstrip(",")
    m = re.match(r"s\[(\d+):(\d+)\]$", tok)
    if m:
        return list(range(int(m.group(1)), int(m.group(2)) + 1))
    m = re.match(r"s(\d+)$", tok)
    return [int(m.group(1))] if m else []


def _flag_regs(blocks) -> Set[int]:
    """SGPRs that decide a branch through vcc (the structurizer's flow flags)."""
    out: Set[int] = set()
    for _, insns, _ in blocks:
        for ins in insns:
            parts = ins.text.replace(",", " ").split()
            if ins.op in ("s_and_b64", "s_andn2_b64") and len(parts) >= 4 and parts[1] == "vcc":
                for t in parts[2:4]:
                    out.update(_sregs(t))
    return out


def _step_consts(ins: "_Insn", consts: Dict[int, int], flags: Set[int]) -> None:
    """Updates the known values of flag SGPRs (and vcc, key -1) after one scalar instruction."""
    parts = ins.text.replace(",", " ").split()
    op = ins.op
    if not op.startswith("s_") or len(parts) < 2:
        return
    dst = -1 if parts[1] == "vcc" else None
    dregs = _sregs(parts[1]) if dst is None else []

    def val(tok):
        r = _sregs(tok)
        if r:
            vs = [consts.get(x) for x in r]
            return None if any(v is None for v in vs) else tuple(vs)
        if tok == "exec":
            return "exec"
        try:
            iv = int(tok, 0)
        except ValueError:
            return None
        return ("imm", iv)

    if op in ("s_and_b64", "s_andn2_b64") and dst == -1 and len(parts) >= 4 and parts[2] == "exec":
        v = val(parts[3])
        if isinstance(v, tuple) and v and v[0] != "imm":
            nz = any(x != 0 for x in v)
            consts[-1] = int(nz) if op == "s_and_b64" else int(not all(x == 0xFFFFFFFF for x in v))
        elif isinstance(v, tuple) and v[0] == "imm":
            consts[-1] = int(v[1] != 0) if op == "s_and_b64" else int(v[1] != -1)
        else:
            consts.pop(-1, None)
        return
    if dst == -1:
        consts.pop(-1, None)
        return
    if op in ("s_mov_b64", "s_mov_b32") and dregs:
        v = val(parts[2]) if len(parts) > 2 else None
        if isinstance(v, tuple) and v and v[0] == "imm":
            iv = v[1] & 0xFFFFFFFFFFFFFFFF
            words = [iv & 0xFFFFFFFF, (iv >> 32) & 0xFFFFFFFF] if op == "s_mov_b64" else [iv & 0xFFFFFFFF]
            if op == "s_mov_b64" and v[1] in (-1, 0):
                words = [0xFFFFFFFF if v[1] == -1 else 0] * 2
            for r, w in zip(dregs, words):
                if r in flags:
                    consts[r] = w
            return
        if isinstance(v, tuple) and v and v[0] != "imm" and len(v) == len(dregs):
            for r, w in zip(dregs, v):
                if r in flags:
                    consts[r] = w
            return
    for r in dregs:
        consts.pop(r, None)


_NO_DEF = ("s_cmp", "s_bitcmp", "s_cbranch", "s_branch", "s_waitcnt", "s_nop", "s_barrier", "s_endpgm",
           "s_setprio", "s_sleep", "s_sendmsg", "s_setpc", "s_trap", "s_dcache")


# VOP3b instructions: vector destination first, then a scalar carry-out (or a scale flag) that the
# instruction writes
_VOP3B = ("v_mad_u64_u32", "v_mad_i64_i32", "v_add_co_u32", "v_sub_co_u32", "v_subrev_co_u32",
          "v_addc_co_u32", "v_subb_co_u32", "v_subbrev_co_u32", "v_div_scale_f32", "v_div_scale_f64")


def _sgpr_use_def(ins: "_Insn") -> Tuple[Set[int], Set[int]]:
    """Conservative SGPR reads (over-approximated) and definitions (under-approximated)."""
    toks = ins.text.replace(",", " ").split()[1:]
    regs = [_sregs(t) for t in toks]
    op = ins.op
    defines_first = (not ins.asm) and (
        (op.startswith("s_") and not op.startswith(_NO_DEF) and not op.startswith(("s_store", "s_buffer_store")))
        or op in ("v_readfirstlane_b32", "v_readlane_b32")
        or (op.startswith("v_cmp_") and op.endswith("_e64")))
    defined = {0} if defines_first else set()
    if not ins.asm and op.startswith(_VOP3B):
        defined = {1}
    d: Set[int] = set()
    u: Set[int] = set()
    for i, r in enumerate(regs):
        (d if i in defined else u).update(r)
    return u, d


def check_kernel(body: List[str]) -> List[str]:
    blocks = _kernel_blocks(body)
    index = {lab: i for i, (lab, _, _) in enumerate(blocks)}
    flags = _flag_regs(blocks)
    # per block: flag-constant context -> reg -> (distance, pending from asm)
    states: Dict[int, Dict[tuple, Dict[int, Tuple[int, bool]]]] = {0: {(): {}}}
    work = [(0, ())]
    reports: Set[str] = set()
    visits = 0
    while work:
        bi, ctx = work.pop()
        visits += 1
        if visits > 500000:
            raise RuntimeError("wait check did not converge")
        lab, insns, succ = blocks[bi]
        st = dict(states[bi][ctx])
        consts = dict(ctx)   # flag SGPR -> value; -1: vcc; -2: scalars read from in-flight registers
        taken = None
        for k, ins in enumerate(insns):
            if ins.wait is not None:
                st = {r: v for r, v in st.items() if v[0] < ins.wait}
                continue
            if not ins.asm:
                touched = ins.reads | ins.writes
                bad = [r for r in touched if r in st and st[r][1]]
                u, d = _sgpr_use_def(ins)
                pois = consts.get(-2, frozenset())
                if u & pois:
                    if ins.op in ("s_mov_b32", "s_mov_b64"):
                        pois = pois | d
                    else:
                        reports.add(f"{lab}: '{ins.text}' uses a scalar read from an in-flight register")
                        pois = pois - d
                else:
                    pois = pois - d
                if bad and ins.op in ("v_readfirstlane_b32", "v_readlane_b32"):
                    # an undefined-value materialisation: harmless unless the scalar it produces is used
                    pois = pois | d
                    bad = []
                if pois:
                    consts[-2] = frozenset(pois)
                else:
                    consts.pop(-2, None)
                if bad:
                    r = min(bad)
                    name = f"a{r - _AGPR}" if r >= _AGPR else f"v{r}"
                    reports.add(f"{lab}: '{ins.text}' touches {name} while its explicitly waited load may be in flight")
                _step_consts(ins, consts, flags)
            else:
                # asm may write any sgpr it names: forget flag values it touches
                for t in ins.text.replace(",", " ").split()[1:]:
                    for r in _sregs(t):
                        consts.pop(r, None)
            if ins.vmem:
                st = {r: (min(v[0] + 1, _CAP), v[1]) for r, v in st.items() if v[0] + 1 < _CAP}
                for r in ins.writes if not ins.op.startswith(_STORE) else ():
                    st[r] = (0, bool(ins.asm_dst))
            elif ins.writes and not ins.asm:
                for r in ins.writes:
                    st.pop(r, None)
            if ins.op in ("s_cbranch_vccnz", "s_cbranch_vccz") and -1 in consts:
                taken = (consts[-1] == 1) == (ins.op == "s_cbranch_vccnz")
        succs = list(succ)
        if taken is not None and insns and insns[-1].op in ("s_cbranch_vccnz", "s_cbranch_vccz") and len(succs) == 2:
            succs = [succs[0]] if taken else [succs[1]]
        nctx = tuple(sorted(((r, v) for r, v in consts.items() if r in flags), key=lambda x: x[0]))
        if -2 in consts:
            nctx = nctx + ((-2, consts[-2]),)
        for sname in succs:
            j = index.get(sname)
            if j is None:
                continue
            bucket = states.setdefault(j, {})
            if len(bucket) >= _MAX_CTX and nctx not in bucket:
                key = ()   # too many contexts: fall back to the unconstrained one
            else:
                key = nctx
            old = bucket.get(key)
            if old is None:
                bucket[key] = dict(st)
                work.append((j, key))
                continue
            merged = dict(old)
            changed = False
            for r, v in st.items():
                o = merged.get(r)
                nv = v if o is None else (min(o[0], v[0]), o[1] or v[1])
                if o != nv:
                    merged[r] = nv
                    changed = True
            if changed:
                bucket[key] = merged
                work.append((j, key))
    return sorted(reports)


def _check_body(body: List[str]) -> List[str]:
    return check_kernel(body)


def check_file(path: str, substring: str = "decode_kernel", workers: Optional[int] = None) -> Dict[str, List[str]]:
    """Checks every kernel whose name contains `substring`, the kernels spread over worker processes."""
    import os
    from concurrent.futures import ProcessPoolExecutor
    s = open(path).read()
    names = sorted(set(re.findall(r"^(\S*" + re.escape(substring) + r"\S*):\s*(?:;.*)?$", s, re.M)))
    bodies = []
    for name in names:
        a = s.index(name + ":")
        b = s.index(".Lfunc_end", a)
        bodies.append(s[a:b].splitlines()[1:])
    n = workers or min(16, len(os.sched_getaffinity(0)))
    if n <= 1 or len(bodies) <= 1:
        return {name: check_kernel(body) for name, body in zip(names, bodies)}
    # largest bodies first, so that the long checks start early
    order = sorted(range(len(bodies)), key=lambda i: -len(bodies[i]))
    with ProcessPoolExecutor(n) as ex:
        results = dict(zip(order, ex.map(_check_body, [bodies[i] for i in order])))
    return {names[i]: results[i] for i in range(len(names))}


def main(argv: List[str]) -> int:
    res = check_file(argv[1], argv[2] if len(argv) > 2 else "decode_kernel")
    bad = {k: v for k, v in res.items() if v}
    for k, v in bad.items():
        print(k)
        for line in v[:20]:
            print("   ", line)
    print(f"{len(res)} kernels checked, {len(bad)} with reports")
    return 1 if bad else 0


if __name__ == "__main__":
    sys.exit(main(sys.argv))
