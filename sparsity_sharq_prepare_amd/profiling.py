"""HBM traffic of a kernel from rocprofv3 counter passes, and kernel-trace
summaries.

Two `rocprofv3 --pmc` passes of the same command, one collecting FETCH_SIZE
and one WRITE_SIZE (KiB per dispatch), give the bytes a kernel moved between
L2 and HBM.  The counters are scaled by what they read for a reference
dispatch of known size: a plain device-to-device copy of C bytes reads C and
writes C, so the factor is C / counter for each pass.  `bench.py
--copy-calibration MIB` runs such a copy (the runtime's copyBuffer blit) first;
it is the largest copyBuffer dispatch of the run.

    python -m sparsity_sharq_prepare_amd.profiling \\
        --fetch <fetch pass counter_collection.csv> \\
        --write <write pass counter_collection.csv> \\
        --kernel linear_mx_decode --copy-mib 256 --workload decode \\
        --out profiles/linear_mx_decode_decode_traffic.txt --command "..."

The summary records traffic_bytes_per_launch (the kernel's average over its
dispatches) and source_sha256, a hash of the kernel sources, so that bench.py
ignores it once the kernel has changed.

    python -m sparsity_sharq_prepare_amd.profiling trace \
        --stats <rocprofv3 --kernel-trace --stats run_kernel_stats.csv> \
        --title "..." --out profiles/<kernel>_<workload>_kernel_trace.txt --command "..."

writes the per-kernel call count and average / min / max duration table.

    python -m sparsity_sharq_prepare_amd.profiling counters \
        --csv <rocprofv3 --pmc counter_collection.csv> --kernel linear_mx_tile \
        --workload prefill --out profiles/linear_mx_tile_prefill_counters.txt --command "..."

averages SQ / GRBM counters over the kernel's dispatches and derives the
MFMA busy fraction and VALU instructions per unit of work.
"""
from __future__ import annotations

import argparse
import csv
import hashlib
import os
import re
import sys
from collections import defaultdict

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SOURCES = {
    "linear_mx_decode": ["gemm_mx.hip", "common.h", "prep_device.h"],
    "linear_mx_tile": ["gemm_mx.hip", "common.h", "prep_device.h"],   # linear_mx_tile8 instances
    "linear_nv_tile": ["gemm_nv.hip", "common.h"],
    "prepare_mx_kernel": ["prepare.hip", "common.h", "prep_device.h"],
}
# dispatch names a kernel's counters are averaged over (the pattern must
# match the name as the profiler prints it): the decode step's GEMM is the
# two-launch form on the 4:8 backbone with one MFMA tile (up to 8 rows:
# linear_mx_decode<NK, CG, J, FUSED = false, M24 = false, MT = 1>); the tile
# GEMM counts its dual-GEMM instances, not the plain baseline's dense tile
# (linear_mx_tile8<BM, BNE, DENSE = true, ...>)
MATCH = {
    "linear_mx_decode": r"linear_mx_decode<\d+, \d+, \d+, false, false, 1>",
    "linear_mx_tile": r"linear_mx_tile8<\d+, \d+, false,",
    "linear_nv_tile": r"linear_nv_tile",
    "prepare_mx_kernel": r"prepare_mx_kernel<",
}


_COMMENT = re.compile(r"//[^\n]*|/\*.*?\*/", re.S)


def code_text(src: str) -> str:
    """A source file's code without comments and whitespace: what the
    compiler sees, so an edit to comments alone leaves it unchanged."""
    return re.sub(r"\s+", "", _COMMENT.sub(" ", src))


def source_hash(files) -> str:
    """Hash of the code (comments and whitespace dropped) of a kernel's
    source files; a summary whose hash differs was taken on other code."""
    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(ROOT, "sparsity_sharq_prepare_amd", "csrc", f), encoding="utf-8") as fh:
            h.update(code_text(fh.read()).encode())
    return h.hexdigest()[:16]


def per_dispatch(path: str, counter: str) -> dict:
    """{dispatch id: (kernel name, counter value summed over its rows)}."""
    vals = defaultdict(float)
    names = {}
    with open(path, newline="") as fh:
        for r in csv.DictReader(fh):
            if r["Counter_Name"] != counter:
                continue
            d = r["Dispatch_Id"]
            vals[d] += float(r["Counter_Value"])
            names[d] = r["Kernel_Name"]
    return {d: (names[d], v) for d, v in vals.items()}


def selects(kernel: str, name: str) -> bool:
    """Whether dispatch `name` (as the profiler prints it) counts for `kernel`."""
    return re.search(MATCH[kernel], name) is not None


def kernel_bytes(path: str, counter: str, kernel: str, copy_bytes: int):
    disp = per_dispatch(path, counter)
    copies = [v for n, v in disp.values() if "copyBuffer" in n]
    if not copies:
        raise SystemExit(f"{path}: no copyBuffer dispatch for the calibration")
    factor = copy_bytes / (max(copies) * 1024.0)
    ks = [v for n, v in disp.values() if selects(kernel, n)]
    if not ks:
        raise SystemExit(f"{path}: no dispatch of {kernel}")
    return sum(ks) / len(ks) * 1024.0 * factor, factor, len(ks)


def trace_main(argv):
    ap = argparse.ArgumentParser(description="kernel-trace summary from rocprofv3 --stats")
    ap.add_argument("--stats", required=True)
    ap.add_argument("--title", required=True)
    ap.add_argument("--out", required=True)
    ap.add_argument("--command", default="")
    ap.add_argument("--note", default="")
    a = ap.parse_args(argv)
    rows = list(csv.DictReader(open(a.stats, newline="")))
    rows.sort(key=lambda r: -float(r["TotalDurationNs"]))
    with open(a.out, "w") as fh:
        fh.write(f"# rocprofv3 kernel trace summary: {a.title}\n")
        if a.command:
            fh.write(f"# command: {a.command}\n")
        if a.note:
            fh.write(f"# {a.note}\n")
        fh.write(f"{'kernel':<72s} {'calls':>6s} {'avg_us':>9s} {'min_us':>9s} {'max_us':>9s} {'pct':>6s}\n")
        for r in rows:
            name = r["Name"].split("(")[0][:72]
            fh.write(f"{name:<72s} {int(r['Calls']):>6d} {float(r['AverageNs']) / 1e3:>9.2f} "
                     f"{float(r['MinNs']) / 1e3:>9.2f} {float(r['MaxNs']) / 1e3:>9.2f} {float(r['Percentage']):>6.2f}\n")
    print(open(a.out).read())


def counters_main(argv):
    """Per-dispatch averages of SQ / GRBM counters for one kernel selection,
    with the derived figures: MFMA busy cycles per MFMA instruction, the
    MFMA busy fraction of the GPU-active cycles per SIMD (SQ_VALU_MFMA_BUSY_
    CYCLES is summed over the SIMDs and GRBM_GUI_ACTIVE over the XCDs), and
    VALU wave-instructions per unit of work (--units: e.g. groups of 8
    K-values a dispatch prepares; a wave covers 64 of them per instruction)."""
    ap = argparse.ArgumentParser(description="counter summary from a rocprofv3 --pmc run")
    ap.add_argument("--csv", required=True, help="counter_collection.csv")
    ap.add_argument("--kernel", required=True, choices=sorted(SOURCES))
    ap.add_argument("--workload", required=True)
    ap.add_argument("--out", required=True)
    ap.add_argument("--command", default="")
    ap.add_argument("--simds", type=int, default=1024)
    ap.add_argument("--xcds", type=int, default=8)
    ap.add_argument("--units", type=float, default=0.0, help="work units per dispatch (lane-level), for VALU per unit")
    ap.add_argument("--unit-name", default="unit")
    a = ap.parse_args(argv)
    vals = defaultdict(lambda: defaultdict(float))
    names = {}
    with open(a.csv, newline="") as fh:
        for r in csv.DictReader(fh):
            vals[r["Dispatch_Id"]][r["Counter_Name"]] += float(r["Counter_Value"])
            names[r["Dispatch_Id"]] = r["Kernel_Name"]
    sel = [d for d in vals if selects(a.kernel, names[d])]
    if not sel:
        raise SystemExit(f"{a.csv}: no dispatch of {a.kernel}")
    counters = sorted({c for d in sel for c in vals[d]})
    avg = {c: sum(vals[d][c] for d in sel) / len(sel) for c in counters}
    with open(a.out, "w") as fh:
        fh.write(f"# counters of {a.kernel} ({a.workload} workload), rocprofv3 --pmc, averaged over {len(sel)} dispatches\n")
        if a.command:
            fh.write(f"# command: {a.command}\n")
        for c in counters:
            fh.write(f"{c} = {avg[c]:.0f}\n")
        if "SQ_VALU_MFMA_BUSY_CYCLES" in avg and "SQ_INSTS_MFMA" in avg and avg["SQ_INSTS_MFMA"] > 0:
            fh.write(f"mfma_busy_cycles_per_instruction = {avg['SQ_VALU_MFMA_BUSY_CYCLES'] / avg['SQ_INSTS_MFMA']:.2f}\n")
        if "SQ_VALU_MFMA_BUSY_CYCLES" in avg and "GRBM_GUI_ACTIVE" in avg and avg["GRBM_GUI_ACTIVE"] > 0:
            per_simd = avg["SQ_VALU_MFMA_BUSY_CYCLES"] / a.simds
            active = avg["GRBM_GUI_ACTIVE"] / a.xcds
            fh.write(f"gpu_active_cycles = {active:.0f}\n")
            fh.write(f"mfma_busy_fraction = {per_simd / active:.4f}\n")
        if a.units > 0 and "SQ_INSTS_VALU" in avg:
            fh.write(f"valu_wave_instructions_per_64_{a.unit_name}s = {avg['SQ_INSTS_VALU'] * 64.0 / a.units:.1f}\n")
        fh.write(f"source_sha256 = {source_hash(SOURCES[a.kernel])}\n")
    print(open(a.out).read())


def main():
    if len(sys.argv) > 1 and sys.argv[1] == "trace":
        return trace_main(sys.argv[2:])
    if len(sys.argv) > 1 and sys.argv[1] == "counters":
        return counters_main(sys.argv[2:])
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--fetch", required=True)
    ap.add_argument("--write", required=True)
    ap.add_argument("--kernel", required=True, choices=sorted(SOURCES))
    ap.add_argument("--copy-mib", type=int, required=True)
    ap.add_argument("--workload", required=True)
    ap.add_argument("--out", required=True)
    ap.add_argument("--command", default="")
    a = ap.parse_args()
    cb = a.copy_mib << 20
    fb, ff, nf = kernel_bytes(a.fetch, "FETCH_SIZE", a.kernel, cb)
    wb, fw, nw = kernel_bytes(a.write, "WRITE_SIZE", a.kernel, cb)
    with open(a.out, "w") as fh:
        fh.write(f"# HBM traffic of {a.kernel} ({a.workload} workload), rocprofv3 FETCH_SIZE / WRITE_SIZE passes\n")
        if a.command:
            fh.write(f"# command: {a.command}\n")
        fh.write(f"# calibration: copy of {cb} bytes; fetch factor {ff:.4f}, write factor {fw:.4f}\n")
        fh.write(f"# dispatches: fetch pass {nf}, write pass {nw}\n")
        fh.write(f"fetch_bytes_per_launch = {fb:.0f}\n")
        fh.write(f"write_bytes_per_launch = {wb:.0f}\n")
        fh.write(f"traffic_bytes_per_launch = {fb + wb:.0f}\n")
        fh.write(f"source_sha256 = {source_hash(SOURCES[a.kernel])}\n")
    print(open(a.out).read())


if __name__ == "__main__":
    main()
