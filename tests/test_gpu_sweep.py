"""Seeded parity sweep over the routing space of sharq_linear (GPU).

The fixed-shape tests elsewhere pin each kernel at chosen shapes; this sweep
draws (T, K, D) from value lists that straddle every routing boundary of the
dual GEMM -- 8 / 9, 16 / 17 and 64 / 65 rows, K around 7168 (two-tile decode
limit) and 16384 (decode limit), K % 512 != 0 (partial side group of the
tile), D not a multiple of 16 or of the tile width -- for the three
activation formats (MXFP4 with the 4:8-in-pairs backbone, MXFP4 with the 2:4
backbone, emulated NVFP4), bf16 or fp32 inputs, with or without the RMSNorm
weight, plus random grouped (MoE) layouts.  Each case checks the prepared
bytes bit for bit and every output element against the fp64 oracle within
1e-5 * sum_k |x~_k w~_k|.  The case list is a fixed
function of its seed, so test ids are stable.
"""
import numpy as np
import pytest
import torch

from oracle import sharq as O
from sparsity_sharq_prepare_amd import ops, synth
from gpu_util import assert_gemm_close, compare_act, dev_gamma, dev_w, dev_x

pytestmark = pytest.mark.gpu

T_VALUES = [1, 2, 7, 8, 9, 12, 16, 17, 24, 33, 48, 64, 65, 100, 256, 257, 300]
K_VALUES = [128, 256, 384, 640, 1024, 1536, 3584, 4096, 7168, 7296, 8192, 16384, 16512]
D_VALUES = [16, 40, 100, 224, 257, 300, 520]
FORMATS = ["mxfp4", "mxfp4", "mxfp4_24", "nvfp4"]
MAX_WORK = 3e8          # T * K * D of a case (the fp64 oracle's matmul)


def _dense_cases(seed: int = 2024, n: int = 72):
    rng = np.random.default_rng(seed)
    cases = [
        # routes named explicitly: two-tile batch kernel (9-16 rows, K > 7168),
        # batch kernel beyond the decode limit, skinny kernel (2:4 and 4:8 at
        # K > 16384), tile with a partial side group and ragged rows/columns
        ("mxfp4", 12, 8192, 100, "bf16", True), ("mxfp4", 40, 16512, 64, "bf16", True),
        ("mxfp4", 5, 16512, 48, "bf16", True), ("mxfp4_24", 20, 16512, 48, "bf16", True),
        ("mxfp4", 257, 640, 257, "bf16", True), ("mxfp4_24", 65, 1536, 300, "bf16", True),
    ]
    while len(cases) < n:
        fmt = FORMATS[rng.integers(len(FORMATS))]
        T = int(rng.choice(T_VALUES))
        K = int(rng.choice(K_VALUES))
        D = int(rng.choice(D_VALUES))
        dtype = "f32" if rng.random() < 0.25 else "bf16"
        gamma = bool(rng.random() < 0.85)
        if T * K * D > MAX_WORK:
            continue
        cases.append((fmt, T, K, D, dtype, gamma))
    return cases


DENSE = _dense_cases()


@pytest.mark.parametrize("fmt,T,K,D,dtype,gamma", DENSE,
                         ids=[f"{c[0]}-{c[1]}x{c[2]}x{c[3]}-{c[4]}{'' if c[5] else '-nogamma'}" for c in DENSE])
def test_sweep_linear(fmt, T, K, D, dtype, gamma):
    base = "nvfp4" if fmt == "nvfp4" else "mxfp4"
    spec = synth.QWEN_OUTLIERS if fmt == "nvfp4" else synth.LLAMA_OUTLIERS
    case = synth.random_case(1000 + T * 7 + K * 3 + D, T, K, D, fmt=base, dtype=dtype, spec=spec, gamma=gamma)
    act = ops.prepare(dev_x(case), dev_gamma(case.gamma), 1e-6, fmt)
    w = ops.pack_weight(dev_w(case.w, case.dtype), base)
    Y = ops.linear(act, w)
    torch.cuda.synchronize()
    mask = "2:4" if fmt == "mxfp4_24" else "4:8"
    ref = O.prepare(case.x_f32(), case.gamma, 1e-6, base, mask=mask)
    compare_act(act, ref)
    Yr, S = O.sharq_linear(ref, O.pack_weight(case.w_f32(), base))
    assert_gemm_close(Y.cpu().numpy(), Yr, S)


def _grouped_cases(seed: int = 77, n: int = 16):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        fmt = "mxfp4_24" if i % 4 == 3 else "mxfp4"
        E = int(rng.choice([3, 8, 40]))
        tokens = int(rng.choice([5, 64, 200]))
        top_k = int(rng.choice([1, 2, 4]))
        top_k = min(top_k, E)
        K = int(rng.choice([256, 640, 1024]))
        D = int(rng.choice([48, 160, 300]))
        gather = bool(i % 2)
        out.append((fmt, E, tokens, top_k, K, D, gather, 500 + i))
    return out


GROUPED = _grouped_cases()


@pytest.mark.parametrize("fmt,E,tokens,top_k,K,D,gather,seed", GROUPED,
                         ids=[f"{c[0]}-E{c[1]}-t{c[2]}-k{c[3]}-{c[4]}x{c[5]}-{'g' if c[6] else 's'}" for c in GROUPED])
def test_sweep_grouped(fmt, E, tokens, top_k, K, D, gather, seed):
    rng = np.random.default_rng(seed)
    go, ri = synth.draw_routing(rng, tokens, E, top_k)
    R = int(go[-1])
    if not gather:
        ri = None                                      # rows expert-sorted: row r reads activation r
    T = tokens if gather else R
    case = synth.random_case(seed, T, K, 1)
    W = synth.f32_to_bf16_bits(rng.standard_normal((E, K, D)).astype(np.float32) * 0.02)
    act = ops.prepare(dev_x(case), dev_gamma(case.gamma), 1e-6, fmt)
    w = ops.pack_weight(dev_w(W, "bf16"))
    Y = ops.linear(act, w, group_offsets=torch.from_numpy(go).cuda(),
                   row_index=None if ri is None else torch.from_numpy(ri).cuda(), total_rows=R)
    torch.cuda.synchronize()
    mask = "2:4" if fmt == "mxfp4_24" else "4:8"
    ref = O.prepare(case.x_f32(), case.gamma, 1e-6, "mxfp4", mask=mask)
    compare_act(act, ref)
    wps = [O.pack_weight(synth.bf16_bits_to_f32(W[e])) for e in range(E)]
    Yr, S = O.grouped_linear(ref, wps, go, ri)
    assert_gemm_close(Y.cpu().numpy(), Yr, S)
