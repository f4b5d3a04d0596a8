"""Where the compiled attention kernels keep their register spills.

Compiles a kernel source to gfx950 assembly and, for every kernel in it, counts the
scratch (spill) loads and stores inside the per-block steps and elsewhere (code that runs
once per tile or work item).  A step is the matrix phase, from its s_setprio 1 to the barrier
that ends it, and the softmax phase, from the s_setprio 0 after that barrier to the next one
(the compiler may fuse the block and tile loops, so loop depth does not separate them).
Usage:

    python -m bf16_causal_flashattention_amd.spill_report [source.hip ...]
"""
from __future__ import annotations

import os
import re
import subprocess
import sys

from .build import CSRC, FLAGS, HIPCC

def assembly(src: str) -> str:
    flags = [f for f in FLAGS if f not in ("-fPIC", "-shared")]
    cmd = [HIPCC, *flags, "--cuda-device-only", "-S", "-o", "-", src]
    return subprocess.run(cmd, capture_output=True, text=True, check=True).stdout


def report(asm: str):
    """[(kernel, scratch ops inside the per-block steps, scratch ops elsewhere, steps found)]"""
    out = []
    for m in re.finditer(r"^(_Z\w+):.*?^\s*s_endpgm", asm, re.M | re.S):
        lines = m.group(0).splitlines()
        in_step = [False] * len(lines)
        starts = [i for i, x in enumerate(lines) if x.strip().startswith("s_setprio 1")]
        for i0 in starts:
            # the matrix phase up to its barrier, then the softmax phase from s_setprio 0 to its barrier
            phase, i = 0, i0
            while i < len(lines) and phase < 2:
                t = lines[i].strip()
                if phase == 0 or in_soft:
                    in_step[i] = True
                if t.startswith("s_barrier"):
                    phase += 1
                    in_soft = False
                elif phase == 1 and t.startswith("s_setprio 0"):
                    in_soft = True
                    in_step[i] = True
                i += 1
                if phase == 0:
                    in_soft = False
        spill = ["scratch_load" in x or "scratch_store" in x for x in lines]
        inside = sum(1 for i, f in enumerate(spill) if f and in_step[i])
        out.append((m.group(1), inside, sum(spill) - inside, len(starts)))
    return out


def spill_counts(asm: str):
    """{kernel: (vgpr spills, sgpr spills, scratch bytes per lane)} from the code-object metadata."""
    res = {}
    for m in re.finditer(r"\.name:\s+(\S+).*?\.private_segment_fixed_size:\s+(\d+).*?\.sgpr_spill_count:\s+(\d+)"
                         r".*?\.vgpr_spill_count:\s+(\d+)", asm, re.S):
        res[m.group(1)] = (int(m.group(4)), int(m.group(3)), int(m.group(2)))
    return res


def main(argv):
    srcs = argv or [os.path.join(CSRC, "attn_fp8.hip"), os.path.join(CSRC, "attn_bf16.hip")]
    for src in srcs:
        asm = assembly(src)
        counts = spill_counts(asm)
        for name, inside, outside, steps in report(asm):
            v, sg, sc = counts.get(name, (-1, -1, -1))
            print(f"{os.path.basename(src)} {name}: {v} VGPR / {sg} SGPR spills, {sc} B scratch per lane; "
                  f"scratch loads/stores inside the per-block phases {inside}, elsewhere {outside}")


if __name__ == "__main__":
    main(sys.argv[1:])
