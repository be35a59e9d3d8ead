"""Benchmark of the SharQ linear-layer hot path on one MI355X.

Default workload (one JSON line on stdout): the Llama-3.1-8B decode linears,
MXFP4, T = 8 tokens, shapes (K, D) = (4096, 4096), (4096, 14336),
(14336, 4096).  One step = the whole per-forward hot path over one batch:
for each of the three linears, the fused prepare (RMSNorm, 4:8 in-pairs mask,
FP4 backbone + residual) and the dual-path FP4 GEMM.  Weight packing is the
offline step and is timed separately (``pack_us``).

Inputs are resident in HBM before timing starts; the packed weights rotate
through ``--copies`` distinct buffers (default 8, about 570 MB) so the 256 MB
Infinity Cache cannot serve them between steps.

The default line also carries a ``prefill`` sub-record: the 4096 x 4096 x
14336 prefill linear's prepare and dual GEMM launch durations, their HBM and
MFMA roofline fractions and the plain unfused breakdown (``--no-prefill``
skips it).

``--workload prefill|nvfp4|moe`` measures the other shapes (4096 x 4096 x
14336 prefill; emulated NVFP4 at T = 2048; grouped MoE up+down) for the
profiles; they are not the headline line.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload decode]
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
FP4_PEAK_TFLOPS = 10100.0      # MI355X dense MXFP4 MFMA
BF16_PEAK_TFLOPS = 2500.0      # MI355X dense 16-bit MFMA (bf16 and fp16 alike)
METRIC = "SharQ linear TFLOPS-eff + tokens/s at Llama-3.1-8B shapes; % HBM/MFMA peak"


def parse():
    p = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=200)
    p.add_argument("--warmup", type=int, default=20)
    p.add_argument("--workload", default="decode", choices=["decode", "prefill", "nvfp4", "moe"])
    p.add_argument("--mask", default="4:8", choices=["4:8", "2:4"],
                   help="backbone mask of the MXFP4 workloads: 4:8 in pairs, or 2:4 element-wise")
    p.add_argument("--copies", type=int, default=0, help="weight copies to rotate (0 = enough for > 512 MB)")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--tokens", type=int, default=8,
                   help="decode workload: tokens per step (8: the headline; up to 16 runs the two-tile decode "
                        "kernel and single-launch form)")
    p.add_argument("--no-prefill", action="store_true",
                   help="decode workload: skip the prefill (4096 x 4096 x 14336) sub-record")
    p.add_argument("--cpu-seconds", type=float, default=12.0, help="target CPU time of the oracle sample")
    p.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                   help="first run one plain device-to-device copy of MIB MiB (a reference dispatch of known "
                        "size for HBM byte counters)")
    return p.parse_args()


# ----------------------------------------------------------------------------
# workloads
# ----------------------------------------------------------------------------
class Job:
    """One SharQ linear of the step: inputs, preallocated outputs, weight copies."""

    def __init__(self, name, fmt, X, gamma, weights, T, K, D, rows=None, group_offsets=None, row_index=None):
        from sparsity_sharq_prepare_amd import ops
        import torch
        # activation copies rotate with the weight copies (same data, distinct buffers)
        self.Xs = [X] + [X.clone() for _ in range(len(weights) - 1)]
        self.X = X
        self.name, self.fmt, self.gamma, self.weights = name, fmt, gamma, weights
        self.T, self.K, self.D = T, K, D
        self.rows = rows if rows is not None else T
        self.group_offsets, self.row_index = group_offsets, row_index
        self.act = ops.empty_act(fmt, X.shape[0], K, X.device)
        self.Y = torch.empty((self.rows, D), dtype=torch.float32, device=X.device)
        self.groups = weights[0].n_groups
        # decode linears: also timed as one launch (sharq_prepare_linear)
        self.fused = fmt == "mxfp4" and self.groups == 1 and rows is None and T <= 16
        self.step_fused = False          # the step uses it when it is the faster form

    # algorithmic work of one launch
    def gemm_flops_nominal(self):
        return 2.0 * self.rows * self.K * self.D

    def gemm_flops_alg(self):            # backbone counted at its nonzeros: 3 T K D
        return 3.0 * self.rows * self.K * self.D

    def gemm_flops_issued(self):         # zero-filled backbone on dense MFMA: 4 T K D
        return 4.0 * self.rows * self.K * self.D

    def act_bytes_per_elem(self):        # prepared activation bytes per input element
        return {"mxfp4": 0.875, "mxfp4_24": 0.9375, "nvfp4": 0.90625}[self.fmt]

    def gemm_bytes(self):
        w = self.groups * self.D * self.K * (0.5 + 1.0 / 32)
        a = self.X.shape[0] * self.K * self.act_bytes_per_elem()
        return w + a + 4.0 * self.rows * self.D

    def prep_bytes(self):
        xb = self.X.element_size()
        return self.X.shape[0] * self.K * (xb + self.act_bytes_per_elem()) + 4.0 * self.K

    def fused_bytes(self):               # X, gamma and weights in; prepared activations and Y out
        w = self.D * self.K * (0.5 + 1.0 / 32)
        return w + self.prep_bytes() + 4.0 * self.rows * self.D


def _dev(a, bf16=True):
    import numpy as np
    import torch
    if bf16:
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).cuda()
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def build_jobs(workload: str, copies: int, mask: str = "4:8", tokens: int = 8):
    import numpy as np
    import torch
    from sparsity_sharq_prepare_amd import ops, synth

    jobs, cases, pack_times = [], [], []
    afmt = "mxfp4_24" if mask == "2:4" else "mxfp4"      # activation format of the MXFP4 workloads

    def pack_copies(W, fmt, n):
        out = []
        for i in range(n):
            ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            ev0.record()
            out.append(ops.pack_weight(W, fmt))
            ev1.record()
            torch.cuda.synchronize()
            pack_times.append((ev0.elapsed_time(ev1) * 1e3, W.numel()))
        return out

    def n_copies(bytes_one):
        return copies or max(2, min(64, int(np.ceil(600e6 / bytes_one))))

    if workload == "decode":
        trio_bytes = sum(K * D * 0.53125 for K, D in synth.DECODE_SHAPES)
        n = n_copies(trio_bytes)
        for i in range(3):
            c = synth.decode_case(i, T=tokens)
            W = _dev(c.w)
            jobs.append(Job(c.name, afmt, _dev(c.x), _dev(c.gamma, False), pack_copies(W, "mxfp4", n),
                            c.T, c.K, c.D))
            del W
            cases.append(c)
    elif workload == "prefill":
        c = synth.prefill_case()
        W = _dev(c.w)
        jobs.append(Job(c.name, afmt, _dev(c.x), _dev(c.gamma, False),
                        pack_copies(W, "mxfp4", n_copies(c.K * c.D * 0.53125)), c.T, c.K, c.D))
        cases.append(c)
    elif workload == "nvfp4":
        for c in synth.nvfp4_cases():
            W = _dev(c.w)
            jobs.append(Job(c.name, "nvfp4", _dev(c.x), _dev(c.gamma, False),
                            pack_copies(W, "nvfp4", n_copies(c.K * c.D * 0.53125)), c.T, c.K, c.D))
            cases.append(c)
    elif workload == "moe":
        for proj in ("up", "down"):
            mc = synth.moe_case(proj)
            W = _dev(mc.w)
            go = torch.from_numpy(mc.group_offsets).cuda()
            ri = None if mc.row_index is None else torch.from_numpy(mc.row_index).cuda()
            jobs.append(Job(mc.name, afmt, _dev(mc.x), _dev(mc.gamma, False),
                            pack_copies(W, "mxfp4", n_copies(W.numel() * 0.53125)), mc.x.shape[0], mc.K, mc.D,
                            rows=mc.total_rows, group_offsets=go, row_index=ri))
            cases.append(mc)
    torch.cuda.synchronize()
    return jobs, cases, pack_times


# ----------------------------------------------------------------------------
# timing
# ----------------------------------------------------------------------------
def run_step(jobs, it):
    from sparsity_sharq_prepare_amd import ops
    for job in jobs:
        w = job.weights[it % len(job.weights)]
        if job.step_fused:
            ops.prepare_linear(job.Xs[it % len(job.Xs)], job.gamma, w, 1e-6, act=job.act, out=job.Y)
            continue
        ops.prepare(job.Xs[it % len(job.Xs)], job.gamma, 1e-6, job.fmt, out=job.act)
        ops.linear(job.act, w, group_offsets=job.group_offsets, row_index=job.row_index, total_rows=job.rows,
                   out=job.Y)


def capture(jobs, first, count):
    """One HIP graph holding `count` consecutive steps starting at step
    `first` (step i uses weight copy i mod copies), so the timed loop is not
    bound by host-side launch overhead."""
    import torch
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for i in range(first, first + count):
            run_step(jobs, i)
    return g


def timed(jobs, steps, warmup):
    """Wall time of exactly `steps` steps (graph replays after `warmup`
    steps), plus each kernel's average launch duration (kernel_times)."""
    import torch
    R = len(jobs[0].weights)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):           # eager warm-up before capture
        for i in range(R):
            run_step(jobs, i)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    full = capture(jobs, 0, R)              # R steps: one per weight copy
    singles = [capture(jobs, i, 1) for i in range(R)]
    torch.cuda.synchronize()

    def run(n):
        for _ in range(n // R):
            full.replay()
        for i in range(n % R):
            singles[i].replay()

    run(warmup)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    run(steps)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    n_steps = steps
    prep_ms, gemm_ms, fused_ms = kernel_times(jobs, R)
    return wall, n_steps, prep_ms, gemm_ms, fused_ms


def kernel_times(jobs, R, reps=3):
    """Average launch duration of each job's prepare, GEMM and (decode) single-
    launch prepare + GEMM: a HIP graph of
    R back-to-back launches of that kernel alone (the GEMM rotating over the R
    weight copies, the prepare over the input copies), replayed `reps` times
    between two HIP events on the stream it runs on, divided by the launch
    count.  Back-to-back launches inside a graph are how the kernels run in
    the timed steps, so this agrees with a kernel trace of the same run."""
    import torch
    from sparsity_sharq_prepare_amd import ops
    prep_ms, gemm_ms, fused_ms = [], [], []
    for job in jobs:
        gp, gg = torch.cuda.CUDAGraph(), torch.cuda.CUDAGraph()
        with torch.cuda.graph(gp):
            for i in range(R):
                ops.prepare(job.Xs[i % len(job.Xs)], job.gamma, 1e-6, job.fmt, out=job.act)
        with torch.cuda.graph(gg):
            for i in range(R):
                ops.linear(job.act, job.weights[i % len(job.weights)], group_offsets=job.group_offsets,
                           row_index=job.row_index, total_rows=job.rows, out=job.Y)
        graphs = [gp, gg]
        if job.fused:
            gf = torch.cuda.CUDAGraph()
            with torch.cuda.graph(gf):
                for i in range(R):
                    ops.prepare_linear(job.Xs[i % len(job.Xs)], job.gamma, job.weights[i % len(job.weights)],
                                       1e-6, act=job.act, out=job.Y)
            graphs.append(gf)
        res = []
        for g in graphs:
            g.replay()                                  # warm
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            for _ in range(reps):
                g.replay()
            e1.record()
            torch.cuda.synchronize()
            res.append(e0.elapsed_time(e1) / (reps * R))
        prep_ms.append(res[0])
        gemm_ms.append(res[1])
        fused_ms.append(res[2] if job.fused else None)
    return prep_ms, gemm_ms, fused_ms


def plain_breakdown(jobs, prep_ms, gemm_ms, R, reps=3):
    """MI355X analogue of the pages' prefill kernel-latency breakdown (xllm-io
    paper review §5): the unfused plain MXFP4 pipeline (RMSNorm kernel,
    quantize kernel, dense one-operand MXFP4 GEMM) against SharQ's fused
    prepare and dual-path GEMM on the same inputs and weights.  Each kernel is
    timed like kernel_times: R back-to-back launches in a HIP graph."""
    import torch
    from sparsity_sharq_prepare_amd import ops
    out = {}
    for job, pm, gm in zip(jobs, prep_ms, gemm_ms):
        T, K = job.X.shape
        y = torch.empty((T, K), dtype=torch.float32, device="cuda")
        codes = torch.empty((T, K // 2), dtype=torch.uint8, device="cuda")
        scales = torch.empty((T, K // 32), dtype=torch.uint8, device="cuda")
        Yd = torch.empty((T, job.D), dtype=torch.float32, device="cuda")
        ops.rmsnorm(job.Xs[0], job.gamma, 1e-6, out=y)
        ops.quantize_mx(y, codes, scales)
        torch.cuda.synchronize()
        graphs = []
        for kind in ("rmsnorm", "quantize", "dense"):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                for i in range(R):
                    if kind == "rmsnorm":
                        ops.rmsnorm(job.Xs[i % len(job.Xs)], job.gamma, 1e-6, out=y)
                    elif kind == "quantize":
                        ops.quantize_mx(y, codes, scales)
                    else:
                        ops.linear_dense(codes, scales, job.weights[i % len(job.weights)], out=Yd)
            graphs.append(g)
        res = []
        for g in graphs:
            g.replay()
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            for _ in range(reps):
                g.replay()
            e1.record()
            torch.cuda.synchronize()
            res.append(e0.elapsed_time(e1) / (reps * R) * 1e3)
        rms, qnt, dense = res
        sp, sg = pm * 1e3, gm * 1e3
        out[job.name] = {
            "plain": {"rmsnorm_us": round(rms, 2), "quantize_us": round(qnt, 2), "dense_gemm_us": round(dense, 2),
                      "total_us": round(rms + qnt + dense, 2)},
            "sharq": {"prepare_us": round(sp, 2), "dual_gemm_us": round(sg, 2), "total_us": round(sp + sg, 2)},
            "prepare_over_rmsnorm_plus_quantize": round(sp / (rms + qnt), 3),
            "dual_over_dense_gemm": round(sg / dense, 3),
            "sharq_over_plain_total": round((sp + sg) / (rms + qnt + dense), 3),
        }
    return out


# ----------------------------------------------------------------------------
# CPU oracle baseline
# ----------------------------------------------------------------------------
def cpu_baseline(cases, workload, target_s):
    """Time the CPU oracle (as it stands) on a bounded sample of the workload."""
    import numpy as np
    from oracle import sharq as O
    from sparsity_sharq_prepare_amd import synth
    def blas_threads():
        # threads of the BLAS the oracle's GEMMs run on (the prepare itself is
        # single-threaded numpy); queried after a matmul has loaded the BLAS
        try:
            from threadpoolctl import threadpool_info
            np.ones((2, 2)) @ np.ones((2, 2))
            return max([p.get("num_threads", 1) for p in threadpool_info()] + [1])
        except Exception:
            return 1
    cores = blas_threads()
    host_cpus = len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else os.cpu_count()
    if workload in ("decode", "prefill", "nvfp4"):
        items = []
        for c in cases:
            rows = c.T if workload == "decode" else min(c.T, 64)
            wp = O.pack_weight(c.w_f32(), c.fmt)          # offline step, not timed
            items.append((c.x_f32()[:rows], c.gamma, wp, c.fmt, rows * c.K * c.D * 2.0))
        flops, n, t = 0.0, 0, 0.0
        while t < target_s and n < 50:
            for x, g, wp, fmt, fl in items:
                t0 = time.perf_counter()
                act = O.prepare(x, g, 1e-6, fmt)
                O.sharq_linear(act, wp)
                t += time.perf_counter() - t0
                flops += fl
            n += 1
        rows_desc = f"all {items[0][0].shape[0]} rows" if workload == "decode" else "the first 64 rows"
        sample = f"{n} pass(es) of the workload's {len(items)} linear(s) on {rows_desc} (prepare + dual GEMM, weights pre-packed)"
        # the prepare alone on one thread (it is elementwise numpy: no BLAS)
        tp, n_el = 0.0, 0
        while tp < min(3.0, target_s / 4):
            for x, g, _, fmt, _ in items:
                t0 = time.perf_counter()
                O.prepare(x, g, 1e-6, fmt)
                tp += time.perf_counter() - t0
                n_el += x.size
        return {"value": flops / t / 1e12, "unit": "TFLOPS-eff", "cores": cores, "kind": "oracle", "sample": sample,
                "seconds": round(t, 2), "host_cpus": host_cpus,
                "prepare_single_thread": {"elements_per_s": round(n_el / tp, 1), "seconds": round(tp, 2),
                                          "threads": 1}}
    # moe: a few experts of each projection
    flops, t = 0.0, 0.0
    n_exp = 0
    for mc in cases:
        x = mc.x_f32()
        for e in range(mc.n_experts):
            a, b = int(mc.group_offsets[e]), int(mc.group_offsets[e + 1])
            rows = np.arange(a, b) if mc.row_index is None else mc.row_index[a:b]
            wp = O.pack_weight(synth.bf16_bits_to_f32(mc.w[e]), "mxfp4")     # offline step, not timed
            t0 = time.perf_counter()
            act = O.prepare(x[rows], mc.gamma, 1e-6)
            O.sharq_linear(act, wp)
            t += time.perf_counter() - t0
            flops += 2.0 * (b - a) * mc.K * mc.D
            n_exp += 1
            if t > target_s / 2 * (1 + (mc is cases[-1])):
                break
    return {"value": flops / t / 1e12, "unit": "TFLOPS-eff", "cores": cores, "kind": "oracle",
            "sample": f"{n_exp} experts' rows (prepare + dual GEMM, weights pre-packed)", "seconds": round(t, 2),
            "host_cpus": host_cpus}


# ----------------------------------------------------------------------------
# traffic counters recorded by rocprofv3 (profiles/<kernel>_<workload>_traffic.txt)
# ----------------------------------------------------------------------------
def read_traffic(name, sources):
    path = os.path.join(ROOT, "profiles", f"{name}_traffic.txt")
    if not os.path.exists(path):
        return None
    vals = {}
    for line in open(path):
        if "=" in line and not line.startswith("#"):
            k, v = line.split("=", 1)
            vals[k.strip()] = v.strip()
    from sparsity_sharq_prepare_amd.profiling import source_hash
    if vals.get("source_sha256") != source_hash(sources):
        return None                          # the kernel changed since the counters were taken
    try:
        return float(vals["traffic_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def gpu_error_outputs(jobs, rows):
    """GPU outputs on the first ``rows`` rows of each linear for the error
    report: the plain MXFP4 pipeline (RMSNorm, quantize, dense GEMM; K % 512
    == 0) and the sparse backbone alone (the dual GEMM with the residual codes
    zeroed).  MXFP4 linears only."""
    from sparsity_sharq_prepare_amd import ops
    out = []
    for j, r in zip(jobs, rows):
        e = {}
        if j.fmt in ("mxfp4", "mxfp4_24") and j.groups == 1:
            X = j.X[:r]
            if j.K % 512 == 0:
                y = ops.rmsnorm(X, j.gamma, 1e-6)
                codes, scales = ops.quantize_mx(y)
                e["plain"] = ops.linear_dense(codes, scales, j.weights[0])
            act = ops.prepare(X, j.gamma, 1e-6, j.fmt)
            act.res_codes.zero_()
            e["sparse_only"] = ops.linear(act, j.weights[0])
        out.append({k: v.float().cpu().numpy() for k, v in e.items()})
    return out


def oracle_errors(cases, y_gpu, extra_gpu, workload):
    """Relative Frobenius error against the unquantized product y W (fp64),
    y = RMSNorm(x), on the rows the CPU baseline samples (all rows at decode,
    the first 64 otherwise; MoE: not reported):
    - the GPU's SharQ output, and GPU plain MXFP4 / sparse-only outputs;
    - the oracle's operator-level analogue of the review's Table 5
      (sparse only, sparse + sparse, dense + dense, SharQ, plain FP4) with
      the packed FP4 weights, and with unquantized weights
      (activation error alone)."""
    import numpy as np
    from oracle import sharq as O
    if workload == "moe":
        return None
    out = {}
    for c, Yg, ex in zip(cases, y_gpu, extra_gpu):
        rows = Yg.shape[0]
        x = c.x_f32()[:rows]
        prep = O.prepare(x, c.gamma, 1e-6, c.fmt)
        ref = prep["y"].astype(np.float64) @ c.w_f32().astype(np.float64)
        wp = O.pack_weight(c.w_f32(), c.fmt)
        st = O.decomposition_study(x, c.gamma, c.w_f32(), c.fmt, wp=wp)
        e = {"rows": rows, "sharq": round(O.rel_frobenius(Yg.astype(np.float64), ref), 6),
             f"plain_{c.fmt}": round(st["weights_fp4"]["plain"], 6)}
        for k, v in ex.items():
            e[f"{k}_gpu"] = round(O.rel_frobenius(v.astype(np.float64), ref), 6)
        e["table5"] = {k: round(v, 6) for k, v in st["weights_fp4"].items()}
        e["table5_activation_only"] = {k: round(v, 6) for k, v in st["activation_only"].items()}
        out[c.name] = e
    return out


# ----------------------------------------------------------------------------
def prefill_subrecord(mask: str = "4:8"):
    """The 4096 x 4096 x 14336 prefill linear (MXFP4), measured beside the
    decode headline: each kernel's average launch duration (as kernel_times),
    its roofline fraction (prepare: HBM; dual GEMM: MXFP4 MFMA on the
    algorithmic 3 T K D and on the issued 4 T K D) and the plain unfused
    breakdown (review §5 kernel latency breakdown)."""
    import torch
    from sparsity_sharq_prepare_amd.profiling import SOURCES
    jobs, _, _ = build_jobs("prefill", 0, mask)
    R = len(jobs[0].weights)
    prep_ms, gemm_ms, _ = kernel_times(jobs, R)
    j, pm, gm = jobs[0], prep_ms[0], gemm_ms[0]
    prep_gbs = j.prep_bytes() / (pm * 1e-3) / 1e9
    alg = j.gemm_flops_alg() / (gm * 1e-3) / 1e12
    issued = j.gemm_flops_issued() / (gm * 1e-3) / 1e12
    out = {
        "workload": "llama3.1-8b prefill linear 4096x4096x14336, MXFP4",
        "prepare_us": round(pm * 1e3, 2), "prepare_GBs": round(prep_gbs, 1),
        "prepare_frac_hbm": round(prep_gbs / HBM_PEAK_GBS, 4),
        "dual_gemm_us": round(gm * 1e3, 2), "dual_gemm_TFLOPS_alg": round(alg, 1),
        "dual_gemm_TFLOPS_issued": round(issued, 1),
        "dual_gemm_frac_mfma_alg": round(alg / FP4_PEAK_TFLOPS, 4),
        "dual_gemm_frac_mfma_issued": round(issued / FP4_PEAK_TFLOPS, 4),
        "dual_gemm_traffic": read_traffic("linear_mx_tile_prefill", SOURCES["linear_mx_tile"]),
        "step_us": round((pm + gm) * 1e3, 2),
        "TFLOPS_eff": round(j.gemm_flops_nominal() / ((pm + gm) * 1e-3) / 1e12, 1),
        "tokens_per_s": round(j.T / ((pm + gm) * 1e-3), 1),
        "breakdown": plain_breakdown(jobs, prep_ms, gemm_ms, R)[j.name],
    }
    del jobs
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    return out


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (got --gpus {args.gpus}); the SharQ hot path here runs on a "
              "single MI355X and has no multi-GPU mode.", file=sys.stderr)
        sys.exit(2)
    import torch
    from sparsity_sharq_prepare_amd import _lib

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    _lib.lib()                                # fail loudly if libsharq.so is missing
    if args.copy_calibration:
        n = args.copy_calibration << 20
        src = torch.full((n,), 7, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    if args.mask == "2:4" and args.workload == "nvfp4":
        print("the 2:4 backbone is an MXFP4 option", file=sys.stderr)
        sys.exit(2)
    if args.tokens != 8 and args.workload != "decode":
        print("--tokens applies to the decode workload", file=sys.stderr)
        sys.exit(2)
    jobs, cases, pack_times = build_jobs(args.workload, args.copies, args.mask, args.tokens)
    wall, n_steps, prep_ms, gemm_ms, fused_ms = timed(jobs, args.steps, args.warmup)
    ms_step = wall * 1e3 / n_steps

    nominal = sum(j.gemm_flops_nominal() for j in jobs)
    tflops = nominal / (ms_step * 1e-3) / 1e12
    tokens = jobs[0].X.shape[0]                      # tokens of the step (MoE: before routing)
    tok_s = tokens / (ms_step * 1e-3)

    gemm_total_ms = sum(gemm_ms)
    prep_total_ms = sum(prep_ms)
    kernels = {}
    for j, p, g, f in zip(jobs, prep_ms, gemm_ms, fused_ms):
        kernels[j.name] = {
            "prepare_us": round(p * 1e3, 2), "prepare_GBs": round(j.prep_bytes() / (p * 1e-3) / 1e9, 1),
            "gemm_us": round(g * 1e3, 2), "gemm_GBs": round(j.gemm_bytes() / (g * 1e-3) / 1e9, 1),
            "gemm_TFLOPS_alg": round(j.gemm_flops_alg() / (g * 1e-3) / 1e12, 1),
            "gemm_TFLOPS_issued": round(j.gemm_flops_issued() / (g * 1e-3) / 1e12, 1),
        }
        if f is not None:
            kernels[j.name]["prepare_linear_us"] = round(f * 1e3, 2)
            kernels[j.name]["prepare_linear_GBs"] = round(j.fused_bytes() / (f * 1e-3) / 1e9, 1)
    n = len(jobs)
    if args.workload == "decode" and any(j.step_fused for j in jobs):
        # the step runs one single-launch prepare + GEMM kernel per linear
        dom, bound, unit, peak = "linear_mx_decode", "hbm", "GB/s", HBM_PEAK_GBS
        fused_total_ms = sum(fused_ms)
        ach = sum(j.fused_bytes() for j in jobs) / n / (fused_total_ms / n * 1e-3) / 1e9
        gemm_total_ms = fused_total_ms
    elif args.workload == "decode":
        dom, bound, unit, peak = "linear_mx_decode", "hbm", "GB/s", HBM_PEAK_GBS
        ach = sum(j.gemm_bytes() for j in jobs) / n / (gemm_total_ms / n * 1e-3) / 1e9
    elif args.workload == "nvfp4":
        dom, bound, unit, peak = "linear_nv_tile", "mfma", "TFLOP/s", BF16_PEAK_TFLOPS
        ach = sum(j.gemm_flops_alg() for j in jobs) / n / (gemm_total_ms / n * 1e-3) / 1e12
    else:
        dom = "linear_mx_tile"
        bound, unit, peak = "mfma", "TFLOP/s", FP4_PEAK_TFLOPS
        ach = sum(j.gemm_flops_alg() for j in jobs) / n / (gemm_total_ms / n * 1e-3) / 1e12

    from sparsity_sharq_prepare_amd.profiling import SOURCES
    roofline = {"bound": bound, "achieved": round(ach, 2), "peak": peak, "unit": unit,
                "frac": round(ach / peak, 4), "traffic": read_traffic(f"{dom}_{args.workload}", SOURCES[dom]),
                "kernel": dom, "launch_us": round(gemm_total_ms / n * 1e3, 2)}
    prep_ach = sum(j.prep_bytes() for j in jobs) / (prep_total_ms * 1e-3) / 1e9
    pack_us = sum(t for t, _ in pack_times) / len(pack_times)

    out = {
        "metric": METRIC, "value": round(tflops, 3), "unit": "TFLOPS-eff", "n_gpus": 1, "steps": n_steps,
        "warmup": args.warmup, "ms_per_step": round(ms_step, 5), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "mxfp4" if args.workload != "nvfp4" else "nvfp4-emu(fp16 mfma)",
        "data": "synthetic",
        "config": {"workload": {"decode": f"llama3.1-8b decode linears, T={args.tokens}, (4096x4096, 4096x14336, 14336x4096), MXFP4",
                                "prefill": "llama3.1-8b prefill linear 4096x4096x14336, MXFP4",
                                "nvfp4": "qwen2.5-7b linears T=2048 (3584x18944, 18944x3584), NVFP4 emulated",
                                "moe": "qwen3-30b-a3b moe linears, 128 experts top-8, 4096 tokens, up 2048x768 + down 768x2048, MXFP4"}[args.workload],
                   "backbone_mask": "4:8 in pairs" if args.mask == "4:8" else "2:4 element-wise",
                   "tokens_per_step": tokens, "weight_copies_rotated": len(jobs[0].weights)},
        "tokens_per_s": round(tok_s, 1),
        "roofline": roofline,
        "prepare": {"achieved_GBs": round(prep_ach, 1), "frac_hbm": round(prep_ach / HBM_PEAK_GBS, 4),
                    "launch_us": round(prep_total_ms / n * 1e3, 2)},
        "kernels": kernels,
        "pack_us": round(pack_us, 1),
    }
    if args.workload == "prefill":
        out["breakdown"] = plain_breakdown(jobs, prep_ms, gemm_ms, len(jobs[0].weights))
    if args.workload == "moe":
        # the grouped GEMMs sit near the ridge: both fractions, per launch
        for j, g in zip(jobs, gemm_ms):
            k = kernels[j.name]
            k["gemm_frac_hbm"] = round(k["gemm_GBs"] / HBM_PEAK_GBS, 4)
            k["gemm_frac_mfma_alg"] = round(k["gemm_TFLOPS_alg"] / FP4_PEAK_TFLOPS, 4)
            k["gemm_frac_mfma_issued"] = round(k["gemm_TFLOPS_issued"] / FP4_PEAK_TFLOPS, 4)
        roofline["frac_hbm"] = round(sum(j.gemm_bytes() for j in jobs) / n / (gemm_total_ms / n * 1e-3) / 1e9
                                     / HBM_PEAK_GBS, 4)
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(cases, args.workload, args.cpu_seconds)
        if args.workload != "moe":
            rows = [j.rows if args.workload == "decode" else 64 for j in jobs]
            y_gpu = [j.Y[:r].float().cpu().numpy() for j, r in zip(jobs, rows)]
            out["errors"] = oracle_errors(cases, y_gpu, gpu_error_outputs(jobs, rows), args.workload)
    if args.workload == "decode" and not args.no_prefill:
        out["prefill"] = prefill_subrecord(args.mask)
    print(json.dumps(out))


if __name__ == "__main__":
    main()
