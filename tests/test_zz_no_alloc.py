"""The allocation-free prepare (sharq_prepare_no_alloc, for callers that
cannot allocate device memory) gives exactly sharq_prepare's outputs: two
calls in a row on the library's static scratch, the second with a smaller
input, each against sharq_prepare with its own workspace (bit for bit), and
the NVFP4 outputs against the oracle."""
import ctypes

import numpy as np
import pytest
import torch

from oracle import sharq as O
from sparsity_sharq_prepare_amd import _lib as L
from sparsity_sharq_prepare_amd import ops, synth

from gpu_util import compare_act, dev_gamma, dev_x

pytestmark = pytest.mark.gpu

KEYS = ("bb_codes", "bb_meta", "bb_scale", "res_codes", "res_scale")


@pytest.fixture(autouse=True, scope="module")
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    yield


@pytest.mark.parametrize("fmt", ["nvfp4", "mxfp4"])
def test_no_alloc_matches_workspace_prepare(fmt):
    spec = synth.QWEN_OUTLIERS if fmt == "nvfp4" else synth.LLAMA_OUTLIERS
    for seed, (T, K) in enumerate([(3000, 3584), (37, 768)]):      # second call smaller
        case = synth.random_case(900 + seed, T, K, 8, fmt=fmt, spec=spec)
        X, g = dev_x(case), dev_gamma(case.gamma)
        ref = ops.prepare(X, g, 1e-6, fmt)                         # caller workspace
        out = ops.empty_act(fmt, T, K)
        for k in KEYS:
            getattr(out, k).fill_(0xA5)                              # stale bytes must all be overwritten
        if out.tensor_scales is not None:
            out.tensor_scales.fill_(-1.0)
        ops.prepare_no_alloc(X, g, 1e-6, out)
        torch.cuda.synchronize()
        for k in KEYS:
            assert torch.equal(getattr(out, k), getattr(ref, k)), (T, K, k)
        if fmt == "nvfp4":
            assert torch.equal(out.tensor_scales, ref.tensor_scales)
            compare_act(out, O.prepare(case.x_f32(), case.gamma, 1e-6, fmt))


def test_no_alloc_rejects_over_maximum_before_any_work():
    # 100000 rows of K = 2048 need 12 bytes per row of NVFP4 scratch, more
    # than the static 1 MiB: rejected on the host, nothing enqueued
    T, K = 100000, 2048
    act = L.SharqAct(L.SHARQ_NVFP4_EMU, T, K, 0x10000, 0x20000, 0x30000, 0x40000, 0x50000, 0x60000)
    st = L.lib().sharq_prepare_no_alloc(0x70000, L.SHARQ_BF16, T, K, K, None, ctypes.c_float(1e-6),
                                        ctypes.byref(act), None)
    assert st == L.SHARQ_ERR_UNSUPPORTED_SHAPE
    assert "scratch" in L.lib().sharq_last_error().decode()
