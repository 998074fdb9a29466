"""Static check of the library's gfx950 device code for one store-data hazard.

A buffer store of more than 8 bytes (buffer_store_dwordx3 / dwordx4) reads its
data VGPRs after it issues; a VALU instruction that writes one of those VGPRs
within the next two wait states can reach the store first, and the store then
writes the new value for some lanes. The compiler inserts the wait states
(s_nop) only when the store's soffset is not a register. This module compiles
each csrc/*.hip file to gfx950 assembly with the library's own flags and lists
every such store, with an SGPR soffset, that a VALU write of its data
registers follows without two wait states in between (instructions in
program order; s_nop n counts n + 1).

Run as ``python -m gpt_pretraining_step_bf16_amd.isa_check``.
"""
from __future__ import annotations

import concurrent.futures as cf
import glob
import os
import re
import subprocess
import sys
import tempfile

from . import build as _build

_STORE = re.compile(r"buffer_store_dwordx([34])\s+(v\[\d+:\d+\]),\s*(\S+),\s*(s\[\d+:\d+\]),\s*(\S+)")
_LABEL = re.compile(r"^[A-Za-z_][\w.$]*:$")


def _vgprs(operand: str) -> set:
    m = re.match(r"v\[(\d+):(\d+)\]$", operand)
    if m:
        return set(range(int(m.group(1)), int(m.group(2)) + 1))
    m = re.match(r"v(\d+)$", operand)
    return {int(m.group(1))} if m else set()


def scan_asm(text: str) -> list:
    """(function, line number, store, offending instruction) for each hazard."""
    lines = [ln.strip() for ln in text.splitlines()]
    found = []
    func = "?"
    for i, ln in enumerate(lines):
        if _LABEL.match(ln) and not ln.startswith(".L"):
            func = ln[:-1]
        m = _STORE.match(ln)
        if not m or not m.group(5).startswith("s"):
            continue
        data = _vgprs(m.group(2))
        waits = 0
        for nxt in lines[i + 1:i + 16]:
            if not nxt or nxt.startswith((";", ".")) or _LABEL.match(nxt):
                continue
            nop = re.match(r"s_nop\s+(\d+)", nxt)
            if nop:
                waits += int(nop.group(1)) + 1
                if waits >= 2:
                    break
                continue
            op = nxt.split()[0]
            if op.startswith("v_") and not op.startswith(("v_readlane", "v_readfirstlane", "v_cmp")):
                dst = nxt.split()[1].rstrip(",") if len(nxt.split()) > 1 else ""
                if _vgprs(dst) & data:
                    found.append((func, i + 1, ln, nxt))
                    break
            waits += 1
            if waits >= 2:
                break
    return found


def device_asm(src: str, out: str) -> str:
    cmd = [_build.HIPCC, *_build.CFLAGS, "--cuda-device-only", "-S", src, "-o", out]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc -S failed for {src}:\n{res.stdout}\n{res.stderr}")
    with open(out) as f:
        return f.read()


def check_sources(srcs=None, jobs: int = 8) -> dict:
    """{source file name: hazards} over csrc/*.hip (or the given files)."""
    srcs = srcs or sorted(glob.glob(os.path.join(_build.CSRC, "*.hip")))
    with tempfile.TemporaryDirectory() as tmp:
        def one(src):
            out = os.path.join(tmp, os.path.basename(src) + ".s")
            return os.path.basename(src), scan_asm(device_asm(src, out))
        with cf.ThreadPoolExecutor(max_workers=max(1, min(jobs, len(srcs)))) as ex:
            return dict(ex.map(one, srcs))


if __name__ == "__main__":
    res = check_sources()
    bad = 0
    for name, hits in res.items():
        print(f"{name}: {len(hits)} unguarded wide buffer stores")
        for func, line, store, nxt in hits[:10]:
            print(f"  {func} line {line}: {store}  ->  {nxt}")
        bad += len(hits)
    sys.exit(1 if bad else 0)
