"""Check of the built device code for one gfx950 hazard that the compiler
cannot see through inline assembly: a DPP instruction reading, as its DPP
source, a VGPR that a VALU instruction wrote fewer than two wait states
before (an `s_nop N` gives N + 1 wait states, any other instruction one).
The kernels put their own `s_nop 1` in front of hand-written DPP
instructions whose source may have just been computed; this walks the
disassembly of every kernel in the library and reports any DPP read that
lacks them, on the fall-through path and on every branch into it.

    python -m dense_linear_solvers_amd.dpp_check [LIBRARY]

Uses llvm-objdump of the ROCm install on the library this package built.
"""
from __future__ import annotations

import os
import re
import shutil
import subprocess
import sys
import tempfile

OBJDUMP = "/opt/rocm/llvm/bin/llvm-objdump"

_INSN = re.compile(r"^\s+([a-z_0-9]+)\s*(.*?)\s*//\s*([0-9A-Fa-f]+):")
_LABEL = re.compile(r"^([0-9a-f]+) <(.+)>:$")
_TARGET = re.compile(r"<(.+)\+0x([0-9a-f]+)>")
_VREG = re.compile(r"v\[(\d+):(\d+)\]|\bv(\d+)\b")


def _vregs(op: str) -> set:
    out = set()
    for m in _VREG.finditer(op):
        if m.group(3) is not None:
            out.add(int(m.group(3)))
        else:
            out.update(range(int(m.group(1)), int(m.group(2)) + 1))
    return out


def _operands(rest: str) -> list:
    rest = rest.split(" row_")[0].split(" quad_perm")[0].split(" wave_")[0]
    return [o.strip() for o in re.split(r",(?![^\[]*\])", rest) if o.strip()]


def _valu_dst(mn: str, ops: list) -> set:
    """VGPRs a VALU instruction writes (none for those writing SGPRs only)."""
    if not mn.startswith("v_") or not ops:
        return set()
    if mn.startswith(("v_cmp", "v_readlane", "v_readfirstlane")):
        return set()
    return _vregs(ops[0])


def _is_dpp(mn: str, rest: str) -> bool:
    return mn.startswith("v_") and ("_dpp" in mn or "row_" in rest or "quad_perm" in rest)


def scan_disassembly(text: str) -> list:
    """Hazards in llvm-objdump -d output: (kernel, address, instruction,
    register, writer address)."""
    kernels = []
    cur = None
    for line in text.splitlines():
        m = _LABEL.match(line.strip())
        if m:
            cur = (m.group(2), [])
            kernels.append(cur)
            continue
        m = _INSN.match(line)
        if m and cur is not None:
            mn, rest, addr = m.group(1), m.group(2), int(m.group(3), 16)
            t = _TARGET.search(line) if mn.startswith(("s_branch", "s_cbranch")) else None
            cur[1].append((addr, mn, rest, t))
    found = []
    for name, insns in kernels:
        index = {ins[0]: i for i, ins in enumerate(insns)}
        base = insns[0][0] if insns else 0
        into = {}   # instruction index -> indices of branches that jump to it
        for i, (a, mn, rest, t) in enumerate(insns):
            if t is not None:
                j = index.get(base + int(t.group(2), 16))
                if j is not None:
                    into.setdefault(j, []).append(i)
        for i, (a, mn, rest, _) in enumerate(insns):
            if not _is_dpp(mn, rest):
                continue
            ops = _operands(rest)
            if len(ops) < 2:
                continue
            src = _vregs(ops[1].lstrip("-|"))
            # walk back along the fall-through path and along each branch in
            starts = []
            if i > 0 and insns[i - 1][1] not in ("s_branch", "s_endpgm"):
                starts.append(i - 1)
            starts += [b for b in into.get(i, [])]
            for j0 in starts:
                ws = 0
                j = j0
                while j >= 0 and ws < 2:
                    ja, jmn, jrest, _ = insns[j]
                    if _valu_dst(jmn, _operands(jrest)) & src:
                        found.append((name, hex(a), f"{mn} {rest}", sorted(src), hex(ja)))
                        break
                    if jmn == "s_nop":
                        ws += int(jrest.split()[0], 0) + 1
                    else:
                        ws += 1
                    j -= 1
    return found


def device_images(library: str, workdir: str) -> list:
    """The gfx950 code objects of a HIP shared library, extracted into workdir."""
    lib = os.path.join(workdir, os.path.basename(library))
    shutil.copyfile(library, lib)
    subprocess.run([OBJDUMP, "--offloading", lib], check=True, capture_output=True)
    return sorted(os.path.join(workdir, f) for f in os.listdir(workdir) if "amdgcn" in f)


def check_library(library: str) -> tuple:
    """(number of DPP instructions seen, hazards) over every kernel."""
    with tempfile.TemporaryDirectory() as wd:
        n_dpp, found = 0, []
        for img in device_images(library, wd):
            out = subprocess.run([OBJDUMP, "-d", "--mcpu=gfx950", img], check=True,
                                 capture_output=True, text=True).stdout
            n_dpp += sum(1 for ln in out.splitlines()
                         if (m := _INSN.match(ln)) and _is_dpp(m.group(1), m.group(2)))
            found += scan_disassembly(out)
    return n_dpp, found


if __name__ == "__main__":
    from dense_linear_solvers_amd.build import library_path
    lib = sys.argv[1] if len(sys.argv) > 1 else library_path()
    n, bad = check_library(lib)
    for b in bad:
        print("hazard:", *b)
    print(f"{n} DPP instructions checked, {len(bad)} hazards")
    sys.exit(1 if bad else 0)
