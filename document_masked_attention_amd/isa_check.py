"""Wait-state check of the dK/dV kernel's inline-assembly MFMAs on the ISA
the compiler generates for it (gfx950 assembly of this library's own build).

The dK/dV kernel issues its S and dP tiles as inline-assembly
v_mfma_f32_32x32x16_bf16 with VGPR accumulators (so the softmax reads them
without AGPR copies).  The compiler does not see those MFMAs and therefore
inserts no wait states for them; the hardware does not interlock either: a
vector instruction that reads or writes such a tile less than 12 wait states
after the MFMA that writes it sees stale data.  This module walks every
control-flow path after every MFMA with a VGPR destination and reports any
other instruction that touches the destination registers before 12 wait states
have passed (each issued instruction counts one, `s_nop n` counts n + 1).  A
later MFMA that accumulates into exactly the same registers continues the
chain (it is checked itself); one that reads them as a multiplicand, or
overlaps them only partly, is reported too.

`build()` runs it on every build and fails on any report, so a toolchain that
schedules a read of those tiles into the window cannot produce a library.

    python -m document_masked_attention_amd.isa_check <file.s> [symbol ...]
"""
from __future__ import annotations

import re
import sys

WAIT_STATES = 12          # gfx950, 8-pass XDL write of a VGPR -> any other access
_LABEL = re.compile(r"^(\.LBB\d+_\d+):")
_VRANGE = re.compile(r"^v\[(\d+):(\d+)\]$")
_VONE = re.compile(r"^v(\d+)$")


def _function_body(asm: str, symbol: str):
    start = asm.index("\n" + symbol + ":") + 1
    end = asm.index(".Lfunc_end", start)
    instrs, labels = [], {}
    for line in asm[start:end].splitlines()[1:]:
        t = line.split(";")[0].strip()
        if not t:
            continue
        m = _LABEL.match(t)
        if m:
            labels[m.group(1)] = len(instrs)
            continue
        if t.startswith("."):
            continue
        instrs.append(t)
    return instrs, labels


def _operands(instr: str):
    parts = instr.split(None, 1)
    if len(parts) < 2:
        return []
    return [o.strip().split()[0] for o in parts[1].split(",") if o.strip()]


def _vregs(op: str) -> set[int]:
    m = _VRANGE.match(op)
    if m:
        return set(range(int(m.group(1)), int(m.group(2)) + 1))
    m = _VONE.match(op)
    return {int(m.group(1))} if m else set()


def _successors(instrs, labels, i):
    t = instrs[i]
    op = t.split()[0]
    if op in ("s_endpgm", "s_setpc_b64"):
        return []
    if op == "s_branch":
        return [labels[t.split()[1]]]
    out = [i + 1] if i + 1 < len(instrs) else []
    if op.startswith("s_cbranch"):
        out.append(labels[t.split()[1]])
    return out


def _wait_states(instr: str) -> int:
    parts = instr.split()
    if parts[0] == "s_nop":
        return int(parts[1], 0) + 1
    return 1


def check(asm: str, symbol: str, need: int = WAIT_STATES):
    """(number of VGPR-destination MFMAs checked, list of violation strings)."""
    instrs, labels = _function_body(asm, symbol)
    violations, checked = [], 0
    for i, t in enumerate(instrs):
        if not t.startswith("v_mfma"):
            continue
        dst = _vregs(_operands(t)[0])
        if not dst:
            continue                      # AGPR destination: the compiler's own
        checked += 1
        stack = [(j, 0) for j in _successors(instrs, labels, i)]
        seen = set()
        while stack:
            j, w = stack.pop()
            if w >= need or (j, w) in seen:
                continue
            seen.add((j, w))
            u = instrs[j]
            ops = _operands(u)
            if u.startswith("v_mfma"):
                d2 = _vregs(ops[0])
                c2 = _vregs(ops[3]) if len(ops) > 3 else set()
                if (_vregs(ops[1]) | _vregs(ops[2])) & dst or (d2 & dst and d2 != dst) or (c2 & dst and c2 != dst):
                    violations.append(f"{symbol}: `{t}` -> `{u}` after {w} wait states")
                    continue
                if d2 == dst:
                    continue              # the chain goes on in that MFMA
            else:
                touched = set()
                for o in ops:
                    touched |= _vregs(o)
                if touched & dst:
                    violations.append(f"{symbol}: `{t}` -> `{u}` after {w} wait states")
                    continue
            for k in _successors(instrs, labels, j):
                stack.append((k, w + _wait_states(u)))
    return checked, violations


def kernel_symbols(asm: str, prefix: str = "_ZN7docmask11dkdv_kernel"):
    return sorted(set(re.findall(r"^(" + re.escape(prefix) + r"\w*):", asm, flags=re.M)))


def main(argv):
    asm = open(argv[0]).read()
    syms = argv[1:] or kernel_symbols(asm)
    bad = 0
    for sym in syms:
        n, v = check(asm, sym)
        print(f"{sym}: {n} VGPR-destination MFMAs, {len(v)} violations")
        for x in v:
            print("  " + x)
        bad += len(v)
    return 1 if bad or not syms else 0


if __name__ == "__main__":
    sys.exit(main(sys.argv[1:]))
