"""Summarise rocprofv3 CSV output of bench.py into per-kernel figures.

    python -m gpt_pretraining_step_bf16_amd.profile_summary trace  KERNEL_TRACE.csv --steps S
    python -m gpt_pretraining_step_bf16_amd.profile_summary traffic FETCH.csv WRITE.csv --copy-bytes N
    python -m gpt_pretraining_step_bf16_amd.profile_summary roofline TRACE.csv FETCH.csv WRITE.csv UTIL.csv \
        --steps S --copy-bytes N

`trace` groups the dispatches of a `--kernel-trace` run by kernel (the two GEMM
templates, gemm_pp_kernel and gemm_bf16_kernel, are split into a fwd/bwd family
and a Newton-Schulz family by their last template argument, the epilogue) and prints launches, average duration and time
per step, where S is the number of steps in the traced run (warm-up
included; every step launches the same kernels).

`traffic` reads two `--pmc` runs (FETCH_SIZE, then WRITE_SIZE; KiB per
dispatch), calibrates each counter against the plain copy kernel of N bytes
that `bench.py --copy-probe-mib` launches (it reads N and writes N bytes),
and prints the calibrated HBM bytes per launch of the fwd/bwd GEMM family.

`roofline` joins the kernel trace (durations) with the two traffic runs and a
`--pmc MfmaUtil LdsUtil` run and prints, per kernel family, the calibrated HBM
bytes per launch, the achieved GB/s against the 8 TB/s HBM peak, and the MFMA
and LDS utilisation the counters report.
"""
from __future__ import annotations

import argparse
import collections
import csv
import hashlib
import os
import re
import sys

# Epilogue ids (GemmEpilogue in csrc/gemm.h) that only Newton-Schulz uses.
NS_EPILOGUES = {7, 8, 9, 11, 12, 13, 14}
GEMM_SOURCES = ("common.h", "lds_dma.h", "gemm.h", "gemm_kernel.h", "gemm.hip",
                "gemm_kk_fwd.hip", "gemm_kk_aux.hip", "gemm_kt.hip", "gemm_tt.hip")


def gemm_source_hash() -> str:
    """sha256 over the GEMM kernel sources, to tie counter data to a kernel version."""
    h = hashlib.sha256()
    root = os.path.join(os.path.dirname(os.path.abspath(__file__)), "csrc")
    for name in GEMM_SOURCES:
        with open(os.path.join(root, name), "rb") as f:
            h.update(name.encode() + b"\0" + f.read())
    return h.hexdigest()


def kernel_family(name: str) -> str:
    m = re.search(r"gemm_(?:bf16|pp)_kernel<([^>]*)>", name)
    if m:
        args = [a.strip() for a in m.group(1).split(",")]
        epi = int(args[-1]) if args and args[-1].lstrip("-").isdigit() else -1
        return "gemm_ns" if epi in NS_EPILOGUES else "gemm_fwd_bwd"
    short = name.replace("(anonymous namespace)::", "")
    short = re.sub(r"^void ", "", short.split("(")[0])
    return short[:80]


def _col(row, *names):
    for n in names:
        if n in row:
            return row[n]
    raise KeyError(f"none of {names} in {sorted(row)}")


def summarise_trace(path: str, steps: int) -> None:
    fam = collections.defaultdict(lambda: [0, 0.0])
    inst = collections.defaultdict(lambda: [0, 0.0])
    with open(path, newline="") as f:
        for row in csv.DictReader(f):
            name = _col(row, "Kernel_Name", "Name")
            dur = float(_col(row, "End_Timestamp")) - float(_col(row, "Start_Timestamp"))
            k = kernel_family(name)
            fam[k][0] += 1
            fam[k][1] += dur
            if k.startswith("gemm"):
                m = re.search(r"gemm_(?:bf16|pp)_kernel<[^>]*>", name)
                inst[(k, m.group(0) if m else name[:60])][0] += 1
                inst[(k, m.group(0) if m else name[:60])][1] += dur
    total = sum(v[1] for v in fam.values())
    print(f"# {path}: {sum(v[0] for v in fam.values())} dispatches, {total / 1e6:.2f} ms kernel time "
          f"over {steps} steps ({total / 1e6 / steps:.2f} ms/step)")
    print(f"{'ms/step':>10} {'launch/step':>11} {'avg us':>10} {'share':>6}  kernel")
    for k, (n, d) in sorted(fam.items(), key=lambda kv: -kv[1][1]):
        print(f"{d / 1e6 / steps:10.3f} {n / steps:11.1f} {d / n / 1e3:10.2f} {100 * d / total:5.1f}%  {k}")
    print("# GEMM instantiations (template args: A k-major, B k-major, [0,] epilogue id)")
    for (k, i), (n, d) in sorted(inst.items(), key=lambda kv: -kv[1][1]):
        print(f"{d / 1e6 / steps:10.3f} {n / steps:11.1f} {d / n / 1e3:10.2f}         {k}: {i}")


def _per_dispatch(path: str, counter: str):
    """{dispatch id: (kernel name, value)} for one counter of a --pmc run."""
    out = {}
    with open(path, newline="") as f:
        for row in csv.DictReader(f):
            if _col(row, "Counter_Name") != counter:
                continue
            did = _col(row, "Dispatch_Id", "Correlation_Id")
            name = _col(row, "Kernel_Name")
            val = float(_col(row, "Counter_Value"))
            prev = out.get(did)
            out[did] = (name, val + (prev[1] if prev else 0.0))
    return out


def summarise_traffic(fetch_csv: str, write_csv: str, copy_bytes: int) -> None:
    res = {}
    for label, path, counter in (("fetch", fetch_csv, "FETCH_SIZE"), ("write", write_csv, "WRITE_SIZE")):
        d = _per_dispatch(path, counter)
        copies = [v for n, v in d.values() if "copy" in n.lower()]
        if not copies:
            sys.exit(f"no copy kernel dispatch in {path}: run bench.py with --copy-probe-mib")
        # The calibration copy is the largest copy dispatch of the run.
        kib = max(copies)
        scale = (copy_bytes / 1024.0) / kib
        g = [v for n, v in d.values() if kernel_family(n) == "gemm_fwd_bwd"]
        res[label] = (scale, sum(g) / len(g) * 1024.0 * scale, len(g))
        print(f"{counter}: copy kernel reads {kib:.0f} KiB for {copy_bytes / 1024:.0f} KiB moved -> "
              f"scale {scale:.4f}; gemm_fwd_bwd: {len(g)} dispatches, "
              f"{res[label][1] / 1e6:.2f} MB per dispatch after scaling")
    per_launch = res["fetch"][1] + res["write"][1]
    print(f"traffic_bytes_per_launch: {per_launch:.6e}")
    print(f"source_sha256: {gemm_source_hash()}")


HBM_PEAK_GBS = 8000.0


def _per_dispatch_all(path):
    """{counter: {dispatch id: (kernel name, value)}} of a --pmc run."""
    out = collections.defaultdict(dict)
    with open(path, newline="") as f:
        for row in csv.DictReader(f):
            c = _col(row, "Counter_Name")
            did = _col(row, "Dispatch_Id", "Correlation_Id")
            name = _col(row, "Kernel_Name")
            val = float(_col(row, "Counter_Value"))
            prev = out[c].get(did)
            out[c][did] = (name, val + (prev[1] if prev else 0.0))
    return out


def summarise_roofline(trace_csv, fetch_csv, write_csv, util_csv, steps, copy_bytes) -> None:
    dur = collections.defaultdict(lambda: [0, 0.0])
    with open(trace_csv, newline="") as f:
        for row in csv.DictReader(f):
            k = kernel_family(_col(row, "Kernel_Name", "Name"))
            dur[k][0] += 1
            dur[k][1] += float(_col(row, "End_Timestamp")) - float(_col(row, "Start_Timestamp"))
    scale = {}
    traffic = collections.defaultdict(lambda: [0, 0.0, 0.0])  # dispatches, fetch B, write B
    for label, path, counter in (("fetch", fetch_csv, "FETCH_SIZE"), ("write", write_csv, "WRITE_SIZE")):
        d = _per_dispatch(path, counter)
        copies = [v for n, v in d.values() if "copy" in n.lower()]
        if not copies:
            sys.exit(f"no copy kernel dispatch in {path}: run bench.py with --copy-probe-mib")
        scale[label] = (copy_bytes / 1024.0) / max(copies)
        for n, v in d.values():
            if "copy" in n.lower():
                continue
            k = kernel_family(n)
            if label == "fetch":
                traffic[k][0] += 1
                traffic[k][1] += v * 1024.0 * scale[label]
            else:
                traffic[k][2] += v * 1024.0 * scale[label]
    util = collections.defaultdict(lambda: collections.defaultdict(list))
    for c, d in _per_dispatch_all(util_csv).items():
        for n, v in d.values():
            util[kernel_family(n)][c].append(v)
    print(f"# counter scales: FETCH_SIZE x{scale['fetch']:.4f}, WRITE_SIZE x{scale['write']:.4f} "
          f"(plain copy of {copy_bytes} bytes); HBM peak {HBM_PEAK_GBS:.0f} GB/s")
    print(f"{'ms/step':>9} {'launch':>6} {'avg us':>9} {'HBM MB/launch':>13} {'GB/s':>7} {'%HBM':>5} "
          f"{'MFMA%':>6} {'LDS%':>5}  kernel")
    for k, (n, t) in sorted(dur.items(), key=lambda kv: -kv[1][1]):
        avg_us = t / n / 1e3
        tr = traffic.get(k)
        if tr and tr[0]:
            mb = (tr[1] + tr[2]) / tr[0] / 1e6
            gbs = mb / 1e3 / (avg_us / 1e6)
            mb_s, gbs_s, pct_s = f"{mb:13.1f}", f"{gbs:7.0f}", f"{100 * gbs / HBM_PEAK_GBS:5.1f}"
        else:
            mb_s, gbs_s, pct_s = f"{'-':>13}", f"{'-':>7}", f"{'-':>5}"
        u = util.get(k, {})
        mf = f"{sum(u['MfmaUtil']) / len(u['MfmaUtil']):6.1f}" if u.get("MfmaUtil") else f"{'-':>6}"
        ls = f"{sum(u['LdsUtil']) / len(u['LdsUtil']):5.1f}" if u.get("LdsUtil") else f"{'-':>5}"
        print(f"{t / 1e6 / steps:9.3f} {n / steps:6.1f} {avg_us:9.1f} {mb_s} {gbs_s} {pct_s} {mf} {ls}  {k}")


def main(argv=None) -> None:
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    sub = ap.add_subparsers(dest="cmd", required=True)
    t = sub.add_parser("trace")
    t.add_argument("csv")
    t.add_argument("--steps", type=int, required=True)
    p = sub.add_parser("traffic")
    p.add_argument("fetch_csv")
    p.add_argument("write_csv")
    p.add_argument("--copy-bytes", type=int, required=True)
    r = sub.add_parser("roofline")
    r.add_argument("trace_csv")
    r.add_argument("fetch_csv")
    r.add_argument("write_csv")
    r.add_argument("util_csv")
    r.add_argument("--steps", type=int, required=True)
    r.add_argument("--copy-bytes", type=int, required=True)
    a = ap.parse_args(argv)
    if a.cmd == "trace":
        summarise_trace(a.csv, a.steps)
    elif a.cmd == "traffic":
        summarise_traffic(a.fetch_csv, a.write_csv, a.copy_bytes)
    else:
        summarise_roofline(a.trace_csv, a.fetch_csv, a.write_csv, a.util_csv, a.steps, a.copy_bytes)


if __name__ == "__main__":
    main()
