"""Build-time check of the GEMMs' untracked loads.

The expert GEMM and gate GEMM kernels load their weights with inline-assembly vector loads,
and read their LDS fragments with inline-assembly ``ds_read_b128``; the
compiler tracks neither (its wait-count pass cannot follow a register ring
across the loop edge, and would order a tracked LDS read after every DMA in
flight).  They are correct only if the generated code never touches a load's
destination registers before the data has landed: a weight load lands at an
``s_waitcnt vmcnt(N)`` issued after at least N later vector-memory instructions
(vector memory operations complete in issue order), an LDS read at an
``s_waitcnt`` with ``lgkmcnt(0)``.  This module compiles the kernels to assembly
and runs a dataflow analysis over each kernel's control-flow graph, with the
pending registers (loading, not yet landed) as the state -- for a weight load,
with the number of vector-memory instructions issued after it:

  * an inline-assembly ``global_load_dwordx4`` or ``ds_read_b128`` adds its
    destination registers (they must not be pending already, nor its address
    registers);
  * every vector-memory instruction (``global_``, ``buffer_``, ``flat_``,
    ``scratch_``: loads, stores, the DMA into LDS) counts one more for each
    pending weight load;
  * ``s_waitcnt vmcnt(N)`` lands the weight loads with at least N instructions
    after them, an ``s_waitcnt`` with ``lgkmcnt(0)`` the LDS reads;
  * any instruction that reads or writes a pending register -- the MFMA that
    consumes it included -- is a violation (a copy, a spill or an MFMA would
    take the value before it lands), and so is a pending register at
    ``s_endpgm``; so the check also proves the kernels' wait counts;
  * at control-flow joins a register pending on either path is pending, with
    the smaller count, iterated to a fixed point.

``check()`` raises on any violation; the library's build calls it, so a build
whose register allocation or wait counts break the invariant leaves no library.
Not covered: the A operand's DMA into LDS (a compiler builtin) must also have
landed before the barrier after which other wavefronts read that stage; the
check does not follow LDS addresses, so that rests on the same wait counts and
on the GPU parity tests.
"""
from __future__ import annotations

import os
import re
import subprocess
import tempfile

_VREG = re.compile(r"v\[(\d+):(\d+)\]|(?<![\w\[])v(\d+)\b")


def _regs(text: str) -> set:
    out = set()
    for m in _VREG.finditer(text):
        if m.group(1) is not None:
            out |= set(range(int(m.group(1)), int(m.group(2)) + 1))
        else:
            out.add(int(m.group(3)))
    return out


def _instructions(lines):
    """(text, is_inline_asm) for every instruction and label; comments stripped."""
    out, in_asm = [], False
    for raw in lines:
        t = raw.strip()
        if t == ";;#ASMSTART":
            in_asm = True
            continue
        if t == ";;#ASMEND":
            in_asm = False
            continue
        t = t.split(";")[0].strip()
        if not t or (t.startswith(".") and not t.startswith(".LBB")):
            continue
        out.append((t, in_asm))
    return out


def _operands(t: str):
    op, _, rest = t.partition(" ")
    return op, [a.strip() for a in rest.split(",")] if rest else []


def _blocks(ins):
    """Basic blocks: (first, last) instruction indices, and successor lists."""
    starts = {0}
    for k, (t, _) in enumerate(ins):
        if t.endswith(":"):
            starts.add(k)
        elif t.startswith(("s_branch", "s_cbranch", "s_endpgm")):
            starts.add(k + 1)
    starts = sorted(x for x in starts if x < len(ins))
    blocks = [(b, (starts[i + 1] if i + 1 < len(starts) else len(ins)) - 1)
              for i, b in enumerate(starts)]
    labels = {ins[b][0][:-1]: i for i, (b, _) in enumerate(blocks) if ins[b][0].endswith(":")}
    succ = []
    for i, (b, e) in enumerate(blocks):
        t = ins[e][0]
        nxt = [i + 1] if i + 1 < len(blocks) else []
        m = re.match(r"(s_branch|s_cbranch\w*) (\.LBB\w+)$", t)
        if t.startswith("s_endpgm"):
            succ.append([])
        elif m and m.group(1) == "s_branch":
            succ.append([labels[m.group(2)]])
        elif m:
            succ.append(nxt + [labels[m.group(2)]])
        else:
            succ.append(nxt)
    return blocks, succ


_VMEM = ("global_", "buffer_", "flat_", "scratch_")
_VMCNT_MAX = 63


def _vmcnt(t: str):
    m = re.search(r"vmcnt\((\d+)\)", t)
    return int(m.group(1)) if m else None


def _step(t: str, is_asm: bool, pending: dict, bad: list, name: str) -> dict:
    """One instruction's effect on the pending map.  Keys: ("vm", r) for a register an
    untracked global load is filling, ("lds", r) for one an untracked LDS read is
    filling; the value of a "vm" key counts the vector-memory instructions issued
    after that load (they complete in issue order, so s_waitcnt vmcnt(N) has landed
    every load with at least N issued after it)."""
    if t.endswith(":"):
        return pending
    op, args = _operands(t)
    if op == "s_waitcnt":
        n = _vmcnt(t)
        if n is not None:
            pending = {k: c for k, c in pending.items() if k[0] != "vm" or c < n}
        if "lgkmcnt(0)" in t:
            pending = {k: c for k, c in pending.items() if k[0] != "lds"}
        return pending
    if op == "s_endpgm":
        if pending:
            bad.append(f"{name}: registers {_names(pending)} still loading at s_endpgm")
        return pending
    regs = {r for _, r in pending}
    if op.startswith(_VMEM):
        pending = {k: (min(c + 1, _VMCNT_MAX + 1) if k[0] == "vm" else c)
                   for k, c in pending.items()}
    if is_asm and op in ("global_load_dwordx4", "ds_read_b128"):
        dst, addr = _regs(args[0]), _regs(args[1])
        if (dst | addr) & regs:
            bad.append(f"{name}: '{t}' while {sorted((dst | addr) & regs)[:8]} are still loading")
        kind = "vm" if op.startswith("global") else "lds"
        pending = {k: c for k, c in pending.items() if k[1] not in dst}
        pending.update({(kind, r): 0 for r in dst})
        return pending
    touched = _regs(t) & regs
    if not touched:
        return pending
    hit = {k for k in pending if k[1] in touched}
    bad.append(f"{name}: '{t}' touches {_names(hit)} before the load into them "
               + ("is waited for (lgkmcnt(0))" if any(k == "lds" for k, _ in hit)
                  else "has landed (no s_waitcnt vmcnt(N) with N loads issued after it)"))
    return {k: c for k, c in pending.items() if k not in hit}


def _names(pending) -> str:
    return str(sorted(f"{k}:v{r}" for k, r in pending)[:8])


def _join(a: dict, b: dict) -> dict:
    """Control-flow join: a register pending on either path, with the fewer loads
    issued after it (the later possible landing)."""
    out = dict(a)
    for k, c in b.items():
        out[k] = min(c, out[k]) if k in out else c
    return out


def check_kernel(name: str, lines) -> list:
    """Violations (strings) in one kernel's assembly."""
    ins = _instructions(lines)
    if not any(a and t.startswith(("global_load_dwordx4", "ds_read_b128")) for t, a in ins):
        return []
    # the control-flow graph below knows direct branches only
    for t, _ in ins:
        if t.startswith(("s_setpc", "s_swappc", "s_getpc", "s_cbranch_join", "s_call")):
            return [f"{name}: '{t}': indirect control flow, not analysed"]
    blocks, succ = _blocks(ins)
    state_in = [None] * len(blocks)
    state_in[0] = {}
    work = [0]
    bad_all = []
    while work:
        i = work.pop()
        pending = dict(state_in[i])
        bad = []
        b, e = blocks[i]
        for k in range(b, e + 1):
            pending = _step(ins[k][0], ins[k][1], pending, bad, name)
        for j in succ[i]:
            new = pending if state_in[j] is None else _join(state_in[j], pending)
            if state_in[j] is None or new != state_in[j]:
                state_in[j] = new
                work.append(j)
    # report from the fixed point
    for i, (b, e) in enumerate(blocks):
        if state_in[i] is None:
            continue
        pending = dict(state_in[i])
        for k in range(b, e + 1):
            pending = _step(ins[k][0], ins[k][1], pending, bad_all, name)
    return sorted(set(bad_all))


KERNELS = r"(ffn_gemm_kernel|router_gemm_kernel)"


def inline_loads(lines) -> int:
    """Instructions of the kinds the check tracks that sit between the
    compiler's inline-assembly markers."""
    return sum(1 for t, a in _instructions(lines)
               if a and t.startswith(("global_load_dwordx4", "ds_read_b128")))


def check_asm(path: str, kernel_regex: str = KERNELS) -> list:
    lines = open(path).read().splitlines()
    starts = [i for i, l in enumerate(lines)
              if re.match(r"^_Z\S*" + kernel_regex + r"\S*:", l)]
    bad, checked = [], 0
    for i in starts:
        end = next((j for j in range(i, len(lines)) if lines[j].startswith(".Lfunc_end")),
                   len(lines))
        body = lines[i:end + 1]
        name = lines[i].split(":")[0]
        if any("global_load_dwordx4" in l or "ds_read_b128" in l for l in body):
            checked += 1
            # the kernels issue these loads only from inline assembly: if none is
            # recognised as such (the compiler's markers changed, say), the
            # analysis below would pass without having tracked anything
            if inline_loads(body) == 0:
                bad.append(f"{name}: no inline-assembly load recognised; the listing's "
                           "format is not the one this check reads")
        bad += check_kernel(name, body)
    if checked == 0:
        bad.append(f"{path}: no kernel with inline-assembly loads was found")
    return bad


def check(hipcc: str, flags: list, src: str, include_dirs: list) -> None:
    """Compile src to gfx950 assembly with the build's flags and check it (the
    source must hold at least one kernel with such loads)."""
    with tempfile.TemporaryDirectory() as d:
        asm = os.path.join(d, "k.s")
        cmd = [hipcc, *flags, "--cuda-device-only", "-S", "-o", asm, src]
        for inc in include_dirs:
            cmd += ["-I", inc]
        subprocess.run(cmd, check=True, capture_output=True)
        bad = check_asm(asm)
    if bad:
        raise RuntimeError("GEMM untracked-load check failed:\n  " + "\n  ".join(bad[:20]))
