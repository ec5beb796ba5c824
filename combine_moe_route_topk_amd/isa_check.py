"""Build-time check of the expert GEMMs' untracked weight loads.

The expert GEMM kernels load their weights with inline-assembly vector loads
that the compiler does not track (its wait-count pass cannot follow a register
ring across the loop edge).  They are correct only if the generated code never
touches a load's destination registers before the data has landed; the
kernel's own waits guarantee landing at the MFMA that consumes a buffer.  This
module compiles the kernels to assembly and runs a dataflow analysis over each
kernel's control-flow graph, with the set of pending registers (loaded, not
yet consumed) as the state:

  * an inline-assembly ``global_load_dwordx4`` adds its destination registers
    (they must not be pending already, nor its address registers);
  * a ``v_mfma`` reading pending registers as sources consumes them (its
    destination must not be pending);
  * ``s_waitcnt vmcnt(0)`` clears the set (everything has landed);
  * any other instruction that reads or writes a pending register is a
    violation, and so is a pending register at ``s_endpgm``;
  * at control-flow joins the sets are united, iterated to a fixed point.

``check()`` raises on any violation; the library's build calls it, so a build
whose register allocation breaks the invariant leaves no library.
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


def _step(t: str, is_asm: bool, pending: set, bad: list, name: str) -> set:
    if t.endswith(":"):
        return pending
    op, args = _operands(t)
    if op == "s_waitcnt" and "vmcnt(0)" in t:
        return set()
    if op == "s_endpgm":
        if pending:
            bad.append(f"{name}: registers {sorted(pending)[:8]}... still loading at s_endpgm")
        return pending
    if is_asm and op == "global_load_dwordx4":
        dst, addr = _regs(args[0]), _regs(args[1])
        if (dst | addr) & pending:
            bad.append(f"{name}: '{t}' while {sorted((dst | addr) & pending)[:8]} are still loading")
        return pending | dst
    touched = _regs(t) & pending
    if not touched:
        return pending
    if op.startswith("v_mfma") and not (_regs(args[0]) & pending):
        return pending - touched  # consumed: the kernel's waits make the data land here
    bad.append(f"{name}: '{t}' touches {sorted(touched)[:8]} before the load into them is consumed")
    return pending - touched


def check_kernel(name: str, lines) -> list:
    """Violations (strings) in one kernel's assembly."""
    ins = _instructions(lines)
    if not any(a and t.startswith("global_load_dwordx4") for t, a in ins):
        return []
    # the control-flow graph below knows direct branches only
    for t, _ in ins:
        if t.startswith(("s_setpc", "s_swappc", "s_getpc", "s_cbranch_join", "s_call")):
            return [f"{name}: '{t}': indirect control flow, not analysed"]
    blocks, succ = _blocks(ins)
    state_in = [None] * len(blocks)
    state_in[0] = frozenset()
    work = [0]
    bad_all = []
    while work:
        i = work.pop()
        pending = set(state_in[i])
        bad = []
        b, e = blocks[i]
        for k in range(b, e + 1):
            pending = _step(ins[k][0], ins[k][1], pending, bad, name)
        for j in succ[i]:
            new = frozenset(pending) | (state_in[j] or frozenset())
            if state_in[j] is None or new != state_in[j]:
                state_in[j] = new
                work.append(j)
    # report from the fixed point
    for i, (b, e) in enumerate(blocks):
        if state_in[i] is None:
            continue
        pending = set(state_in[i])
        for k in range(b, e + 1):
            pending = _step(ins[k][0], ins[k][1], pending, bad_all, name)
    return sorted(set(bad_all))


def check_asm(path: str, kernel_regex: str = r"ffn_gemm_kernel") -> list:
    lines = open(path).read().splitlines()
    starts = [i for i, l in enumerate(lines)
              if re.match(r"^_Z\S*" + kernel_regex + r"\S*:", l)]
    bad, checked = [], 0
    for i in starts:
        end = next((j for j in range(i, len(lines)) if lines[j].startswith(".Lfunc_end")),
                   len(lines))
        body = lines[i:end + 1]
        if any("global_load_dwordx4" in l for l in body):
            checked += 1
        bad += check_kernel(lines[i].split(":")[0], body)
    if checked == 0:
        bad.append("no kernel with inline-assembly weight loads was found")
    return bad


def check(hipcc: str, flags: list, src: str, include_dirs: list) -> None:
    """Compile src to gfx950 assembly with the build's flags and check it."""
    with tempfile.TemporaryDirectory() as d:
        asm = os.path.join(d, "k.s")
        cmd = [hipcc, *flags, "--cuda-device-only", "-S", "-o", asm, src]
        for inc in include_dirs:
            cmd += ["-I", inc]
        subprocess.run(cmd, check=True, capture_output=True)
        bad = check_asm(asm)
    if bad:
        raise RuntimeError("expert GEMM weight-load check failed:\n  " + "\n  ".join(bad[:20]))
