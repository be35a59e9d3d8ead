"""Per-tile timeline of the tile GEMM (tracing).

``python -m sparsity_sharq_prepare_amd.build --timeline`` builds
``libsharq_timeline.so``, the library with SHARQ_TIMELINE defined: wave 0 of
every tile of the tile GEMM records s_memrealtime stamps (a 100 MHz clock) at
the tile's start, after its first step's wait and barrier, after its last
step and after its epilogue stores are issued (``sharq_timeline_*`` in
include/sharq.h).  This module runs one workload's dual GEMM on that build
and summarizes the records of one launch:

    python -m sparsity_sharq_prepare_amd.timeline --workload moe --out FILE

``moe``: the Qwen3-30B-A3B expert linears (persistent 128-row tile, record
t = tile t); ``prefill``: the 4096 x 4096 x 14336 linear (256-row tile, record
b = workgroup b).  Phases per tile: ``first-step wait`` (the wait for the
first operand stage; on a workgroup's later tiles it also covers the previous
tile's stores, which share the in-order memory counter), ``steps`` (the
K-steps after the first wait), ``epilogue issue`` (issuing the fp32 stores),
and per workgroup the ``gap`` between one tile's epilogue and its next tile.
"""
from __future__ import annotations

import argparse
import ctypes
import os
import sys

import numpy as np

PKG = os.path.dirname(os.path.abspath(__file__))
TIMELINE_LIB = os.path.join(PKG, "libsharq_timeline.so")
CLOCK_HZ = 100e6            # s_memrealtime


def summarize(rec: np.ndarray) -> dict:
    """Phase statistics of the records of one launch (rows of 8 words; unused
    rows are zero).  Times in microseconds."""
    rec = rec[rec[:, 0] > 0].astype(np.int64)
    if len(rec) == 0:
        raise ValueError("no records")
    us = 1e6 / CLOCK_HZ
    t0 = rec[:, 0].min()
    out = {"records": int(len(rec)), "workgroups": int(len(np.unique(rec[:, 5]))),
           "span_us": float((rec[:, 3].max() - t0) * us)}
    phases = {"first-step wait": rec[:, 1] - rec[:, 0], "steps": rec[:, 2] - rec[:, 1],
              "epilogue issue": rec[:, 3] - rec[:, 2]}
    gaps, tiles, ends, first_wait = [], [], [], []
    for wg in np.unique(rec[:, 5]):
        m = rec[rec[:, 5] == wg]
        m = m[np.argsort(m[:, 0])]
        tiles.append(len(m))
        ends.append((m[-1, 3] - t0) * us)
        first_wait.append(m[0, 1] - m[0, 0])
        gaps.extend(m[1:, 0] - m[:-1, 3])
    phases["first tile's first-step wait"] = np.array(first_wait)
    if gaps:
        phases["gap to the next tile"] = np.array(gaps)
    out["phases_us"] = {k: {"mean": float(v.mean() * us), "p10": float(np.percentile(v, 10) * us),
                            "p50": float(np.median(v) * us), "p90": float(np.percentile(v, 90) * us)}
                        for k, v in phases.items()}
    out["tiles_per_workgroup"] = {int(k): int(c) for k, c in enumerate(np.bincount(tiles)) if c}
    ends = np.array(ends)
    out["workgroup_end_us"] = {"p10": float(np.percentile(ends, 10)), "p50": float(np.median(ends)),
                               "max": float(ends.max())}
    return out


def summarize_batch(rec: np.ndarray) -> dict:
    """Events of the batch kernel (17-64 rows), one record per workgroup,
    each as time after the workgroup's start (word 0): staging waves' words
    1 (first chunk staged) and 7 (second chunk staged), compute waves'
    words 6 (first chunk multiplied) and 2 (last chunk multiplied), and word
    3 (results stored).  The two kinds of wave run concurrently, so events
    are reported from the start rather than as consecutive phases."""
    rec = rec[rec[:, 0] > 0].astype(np.int64)
    if len(rec) == 0:
        raise ValueError("no records: the launch did not run the batch kernel")
    us = 1e6 / CLOCK_HZ
    ev = {"first chunk staged": 1, "second chunk staged": 7, "first chunk multiplied": 6,
          "last chunk multiplied": 2, "stored": 3}
    ph = {k: rec[:, i] - rec[:, 0] for k, i in ev.items()}
    t0 = rec[:, 0].min()
    return {"records": int(len(rec)), "workgroups": int(len(rec)), "span_us": float((rec[:, 3].max() - t0) * us),
            "phases_us": {k: {"mean": float(v.mean() * us), "p10": float(np.percentile(v, 10) * us),
                              "p50": float(np.median(v) * us), "p90": float(np.percentile(v, 90) * us)}
                          for k, v in ph.items()},
            "tiles_per_workgroup": {1: int(len(rec))},
            "workgroup_end_us": {"p10": float(np.percentile((rec[:, 3] - t0) * us, 10)),
                                 "p50": float(np.median((rec[:, 3] - t0) * us)),
                                 "max": float((rec[:, 3].max() - t0) * us)}}


def format_summary(name: str, s: dict, event_us: float) -> list:
    lines = [f"{name}: launch {event_us:.1f} us (HIP events); {s['records']} tile records, "
             f"{s['workgroups']} workgroups; first start to last epilogue {s['span_us']:.1f} us"]
    for k, v in s["phases_us"].items():
        lines.append(f"  {k:30s} mean {v['mean']:7.2f}  p10 {v['p10']:7.2f}  p50 {v['p50']:7.2f}  "
                     f"p90 {v['p90']:7.2f} us")
    lines.append("  tiles per workgroup: " + ", ".join(f"{c} with {k}" for k, c in s["tiles_per_workgroup"].items()))
    e = s["workgroup_end_us"]
    lines.append(f"  workgroup end (after start): p10 {e['p10']:.1f}  p50 {e['p50']:.1f}  max {e['max']:.1f} us")
    return lines


def _jobs(workload: str):
    """(name, run) pairs: run() enqueues the dual GEMM once."""
    import torch
    from . import ops, synth

    def bf16(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).cuda()

    jobs = []
    if workload == "moe":
        for proj in ("up", "down"):
            mc = synth.moe_case(proj)
            w = ops.pack_weight(bf16(mc.w))
            act = ops.prepare(bf16(mc.x), torch.from_numpy(mc.gamma).cuda(), 1e-6)
            go = torch.from_numpy(mc.group_offsets).cuda()
            ri = None if mc.row_index is None else torch.from_numpy(mc.row_index).cuda()
            Y = ops.linear(act, w, group_offsets=go, row_index=ri, total_rows=mc.total_rows)
            jobs.append((mc.name, lambda act=act, w=w, go=go, ri=ri, Y=Y, n=mc.total_rows:
                         ops.linear(act, w, group_offsets=go, row_index=ri, total_rows=n, out=Y)))
    elif workload == "batch":
        for i, T in ((1, 40), (2, 64)):               # 4096 x 14336 at 40 rows, 14336 x 4096 at 64
            c = synth.decode_case(i, T=T)
            w = ops.pack_weight(bf16(c.w))
            act = ops.prepare(bf16(c.x), torch.from_numpy(c.gamma).cuda(), 1e-6)
            Y = ops.linear(act, w)
            jobs.append((f"{c.name}_T{T}", lambda act=act, w=w, Y=Y: ops.linear(act, w, out=Y)))
    elif workload == "prefill":
        c = synth.prefill_case()
        w = ops.pack_weight(bf16(c.w))
        act = ops.prepare(bf16(c.x), torch.from_numpy(c.gamma).cuda(), 1e-6)
        Y = ops.linear(act, w)
        jobs.append((c.name, lambda act=act, w=w, Y=Y: ops.linear(act, w, out=Y)))
    else:
        raise ValueError(workload)
    return jobs


def main(argv=None) -> int:
    p = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    p.add_argument("--workload", default="moe", choices=["moe", "prefill", "batch"])
    p.add_argument("--warmup", type=int, default=3)
    p.add_argument("--out", default=None, help="write the summary here as well")
    a = p.parse_args(argv)
    import torch                                   # first: the library shares torch's HIP runtime
    from . import _lib as L
    if os.path.abspath(L.LIB_PATH) != TIMELINE_LIB and not os.environ.get("SHARQ_LIBRARY"):
        L.LIB_PATH = TIMELINE_LIB            # before the first lib() call
    lib = L.lib()
    n = ctypes.c_size_t(0)
    L.check(lib.sharq_timeline_records(ctypes.byref(n)))
    if n.value == 0:
        raise SystemExit(f"{L.LIB_PATH} is not the tile-timeline build: "
                         "run `python -m sparsity_sharq_prepare_amd.build --timeline`")
    buf = np.zeros(n.value * 8, dtype=np.uint64)
    kernel = "linear_mx_batch" if a.workload == "batch" else "linear_mx_tile8"
    lines = [f"# timeline of {kernel} ({a.workload} workload), s_memrealtime stamps of the "
             f"SHARQ_TIMELINE build",
             f"# command: python -m sparsity_sharq_prepare_amd.build --timeline && "
             f"python -m sparsity_sharq_prepare_amd.timeline --workload {a.workload}"
             + (f" --out {a.out}" if a.out else "")]
    for name, run in _jobs(a.workload):
        for _ in range(a.warmup):
            run()
        torch.cuda.synchronize()
        L.check(lib.sharq_timeline_clear())
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        run()
        e1.record()
        torch.cuda.synchronize()
        L.check(lib.sharq_timeline_read(buf.ctypes.data_as(ctypes.c_void_p), ctypes.c_size_t(buf.size)))
        summ = summarize_batch if a.workload == "batch" else summarize
        lines += format_summary(name, summ(buf.reshape(-1, 8)), e0.elapsed_time(e1) * 1e3)
    text = "\n".join(lines) + "\n"
    sys.stdout.write(text)
    if a.out:
        with open(a.out, "w") as fh:
            fh.write(text)
    return 0


if __name__ == "__main__":
    sys.exit(main())
