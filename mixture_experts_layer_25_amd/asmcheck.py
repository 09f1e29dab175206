"""Check of the grouped-GEMM assembly for MFMA result hazards.

The GEMM inner loops are inline-asm blocks that end with MFMAs. The compiler
does not look inside inline asm, so if it places an instruction that reads
or overwrites an MFMA destination register right after such a block (a
register move, a spill), nothing guarantees the wait states the hardware
needs, and the value read can be stale. This module compiles a HIP source
to gfx950 assembly and reports every compiler instruction, within the first
few executed after an asm block that issues MFMAs (following branches), that
touches a register one of the block's last MFMAs writes.

    python -m mixture_experts_layer_25_amd.asmcheck [source.hip]
"""
from __future__ import annotations

import os
import re
import subprocess
import sys
import tempfile

HERE = os.path.dirname(os.path.abspath(__file__))
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
WINDOW = 6  # instructions checked after each block
PAD = 19    # wait states after which a 16-pass MFMA result is readable


def _regs(op: str) -> set:
    m = re.match(r"([av])\[(\d+):(\d+)\]$", op)
    if m:
        return {(m.group(1), r) for r in range(int(m.group(2)), int(m.group(3)) + 1)}
    m = re.match(r"([av])(\d+)$", op)
    if m:
        return {(m.group(1), int(m.group(2)))}
    return set()


def find_hazards(asm: str) -> list[str]:
    lines = asm.split("\n")
    labels = {l.split(":")[0]: n for n, l in enumerate(lines) if re.match(r"^\.LBB\w+:", l)}
    found = []
    func = "?"
    i = 0
    while i < len(lines):
        line = lines[i]
        if re.match(r"^_Z\S+:", line):
            func = line.split(":")[0]
        if ";;#ASMSTART" in line:
            j = i + 1
            body = []
            while j < len(lines) and ";;#ASMEND" not in lines[j]:
                t = lines[j].strip()
                if t and not t.startswith(";"):
                    body.append(t)
                j += 1
            # destinations of the block's last MFMAs (up to 8, the most a
            # block issues back to back), unless the block itself waits
            # PAD wait states after its last MFMA (s_nop N counts N + 1,
            # another instruction 1, s_waitcnt nothing)
            mf = [n for n, t in enumerate(body) if t.startswith("v_mfma")]
            dst = set()
            if mf:
                pad = 0
                for t in body[mf[-1] + 1:]:
                    if t.startswith("s_nop"):
                        pad += int(t.split()[1], 0) + 1
                    elif not t.startswith("s_waitcnt"):
                        pad += 1
                if pad < PAD:
                    for n in mf[-8:]:
                        dst |= _regs(body[n].split()[1].rstrip(","))
            if dst:
                found.extend(f"{func}: {t}" for t in _touches(lines, labels, j + 1, dst))
            i = j
        i += 1
    return found


def _touches(lines, labels, start, dst):
    """Instructions among the first WINDOW executed after line `start` (on
    every path: an unconditional branch continues at its target, a
    conditional one on both sides) that touch a register in dst; a path
    ends at the next asm block or at s_endpgm."""
    out, todo, seen = [], [(start, 0)], set()
    while todo:
        k, n = todo.pop()
        while n < WINDOW and k < len(lines) and ";;#ASMSTART" not in lines[k]:
            if (k, n) in seen:
                break
            seen.add((k, n))
            t = lines[k].strip()
            k += 1
            if not t or t.startswith((";", ".")):
                continue
            touched = set()
            for op in re.findall(r"[av]\[\d+:\d+\]|\b[av]\d+\b", t):
                touched |= _regs(op)
            if touched & dst:
                out.append(t)
            n += 1
            op = t.split()[0]
            if op == "s_endpgm":
                break
            if op.startswith("s_cbranch") and t.split()[-1] in labels:
                todo.append((labels[t.split()[-1]], n))
            elif op == "s_branch" and t.split()[-1] in labels:
                k = labels[t.split()[-1]]
    return out


def compile_to_asm(src: str) -> str:
    with tempfile.TemporaryDirectory() as d:
        out = os.path.join(d, "k.s")
        subprocess.run([HIPCC, "--offload-arch=gfx950", "-O3", "-std=c++17", "-Xclang",
                        "-target-feature", "-Xclang", "-packed-fp32-ops", "--cuda-device-only",
                        "-S", src, "-o", out], check=True, capture_output=True,
                       cwd=os.path.dirname(src))
        return open(out).read()


SOURCES = ("gemm16.hip", "gemm_a8.hip")


def main(argv=None) -> int:
    argv = sys.argv[1:] if argv is None else argv
    srcs = argv or [os.path.join(HERE, "csrc", f) for f in SOURCES]
    total = 0
    for src in srcs:
        hazards = find_hazards(compile_to_asm(src))
        for h in hazards:
            print(h)
        print(f"{len(hazards)} MFMA result hazards after asm blocks in {os.path.basename(src)}")
        total += len(hazards)
    return 1 if total else 0


if __name__ == "__main__":
    sys.exit(main())
