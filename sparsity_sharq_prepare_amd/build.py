"""Build libsharq.so (the HIP kernels + C ABI) in-tree for gfx950.

``python -m sparsity_sharq_prepare_amd.build`` compiles every source under
``csrc/`` with hipcc and links ``sparsity_sharq_prepare_amd/libsharq.so``;
with ``--timeline`` it links the tile-timeline (tracing) build
``libsharq_timeline.so`` instead.  Objects go to ``_build/`` at the
repository root (not committed).
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
OUT = os.path.join(PKG, "libsharq.so")
BUILD = os.path.join(ROOT, "_build")

ARCH = "gfx950"
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

# -ffp-contract=off: the pinned fp32 RMSNorm order must not be fused into FMAs.
# -fno-gpu-flush-denormals-to-zero: the residual R = y - X~_sp is exact only
#   with gradual underflow.
# packed-fp32-ops disabled: hipcc must not emit v_pk_{add,mul,fma}_f32.
HIP_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    "-ffp-contract=off", "-fno-gpu-flush-denormals-to-zero",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument",
]

SOURCES = ["prepare.hip", "pack.hip", "gemm_mx.hip", "gemm_nv.hip", "api.cpp"]

# Per-file additions.  prepare.hip: IEEE mode off, so fmax/fmin take |x|
# operands directly instead of first quieting signalling NaNs (inputs are
# finite; a NaN input gives unspecified codes, never a fault).
EXTRA_FLAGS = {"prepare.hip": ["-mno-amdgpu-ieee", "-fno-honor-nans"]}


# the tile-timeline build (tracing): the tile GEMM records per-tile stamps
TIMELINE_OUT = os.path.join(PKG, "libsharq_timeline.so")
TIMELINE_BUILD = os.path.join(ROOT, "_build", "timeline")
TIMELINE_FLAGS = {"gemm_mx.hip": ["-DSHARQ_TIMELINE"]}


def _compile(src: str, build_dir: str = BUILD, extra: dict = None) -> str:
    obj = os.path.join(build_dir, os.path.basename(src) + ".o")
    lang = ["-x", "hip"] if src.endswith(".hip") else []
    cmd = [HIPCC, *HIP_FLAGS, *EXTRA_FLAGS.get(src, []), *(extra or {}).get(src, []), *lang, "-I",
           os.path.join(ROOT, "include"), "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    return obj


def build(verbose: bool = False, timeline: bool = False) -> str:
    """Compile all sources and link libsharq.so (with ``timeline``: the
    tile-timeline build, libsharq_timeline.so); returns its path."""
    if shutil.which(HIPCC) is None and not os.path.exists(HIPCC):
        raise RuntimeError(f"hipcc not found at {HIPCC}")
    build_dir, out, extra = (TIMELINE_BUILD, TIMELINE_OUT, TIMELINE_FLAGS) if timeline else (BUILD, OUT, None)
    os.makedirs(build_dir, exist_ok=True)
    with ThreadPoolExecutor(max_workers=min(len(SOURCES), os.cpu_count() or 4)) as ex:
        objs = list(ex.map(lambda src: _compile(src, build_dir, extra), SOURCES))
    tmp = out + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, out)
    if verbose:
        print(f"built {out}")
    return out


if __name__ == "__main__":
    try:
        build(verbose=True, timeline="--timeline" in sys.argv[1:])
    except RuntimeError as e:
        print(e, file=sys.stderr)
        sys.exit(1)
