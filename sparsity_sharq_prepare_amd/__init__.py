"""SharQ linear-layer hot path for AMD Instinct MI355X (gfx950).

The work runs in libsharq.so (hand-written HIP kernels behind the C ABI in
include/sharq.h): ``ops.pack_weight`` (shared FP4 payload + two scale views),
``ops.prepare`` (fused RMSNorm, 4:8 in-pairs mask, FP4 backbone and dense FP4
residual) and ``ops.linear`` (dual-path FP4 GEMM into one accumulator).
``synth`` draws the seeded synthetic inputs.
"""
__all__ = ["ops", "synth", "build"]
