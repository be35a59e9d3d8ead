"""Helpers for the GPU parity tests: move seeded synthetic inputs to the GPU and
compare the GPU library's outputs with the CPU oracle's."""
import numpy as np
import torch

from oracle import sharq as O
from sparsity_sharq_prepare_amd import ops, synth

ACT_KEYS = ("bb_codes", "bb_meta", "bb_scale", "res_codes", "res_scale")


def dev_x(case) -> torch.Tensor:
    if case.dtype == "f32":
        return torch.from_numpy(np.ascontiguousarray(case.x)).cuda()
    return torch.from_numpy(np.ascontiguousarray(case.x).view(np.int16)).view(torch.bfloat16).cuda()


def dev_w(w: np.ndarray, dtype: str) -> torch.Tensor:
    if dtype == "f32":
        return torch.from_numpy(np.ascontiguousarray(w)).cuda()
    return torch.from_numpy(np.ascontiguousarray(w).view(np.int16)).view(torch.bfloat16).cuda()


def dev_gamma(g):
    return None if g is None else torch.from_numpy(np.ascontiguousarray(g, dtype=np.float32)).cuda()


def assert_bytes_equal(name, got: np.ndarray, exp: np.ndarray):
    got = np.asarray(got).reshape(exp.shape)
    if np.array_equal(got, exp):
        return
    bad = np.argwhere(got != exp)
    idx = tuple(bad[0])
    raise AssertionError(f"{name}: {len(bad)} mismatching bytes; first at {idx}: gpu={got[idx]:#04x} "
                         f"oracle={exp[idx]:#04x}")


def compare_act(gpu_act: ops.PreparedAct, ref: dict):
    torch.cuda.synchronize()
    g = gpu_act.as_numpy()
    for k in ACT_KEYS:
        assert_bytes_equal(k, g[k], ref[k])
    if ref["tensor_scales"] is not None:
        assert np.array_equal(g["tensor_scales"].view(np.uint32), ref["tensor_scales"].view(np.uint32)), \
            (g["tensor_scales"], ref["tensor_scales"])


def compare_weight(gpu_w: ops.PackedWeight, ref: dict, group: int = 0):
    torch.cuda.synchronize()
    assert_bytes_equal("payload", gpu_w.payload[group].cpu().numpy(), ref["payload"])
    assert_bytes_equal("scale_sp", gpu_w.scale_sp[group].cpu().numpy(), ref["scale_sp"])
    assert_bytes_equal("scale_dn", gpu_w.scale_dn[group].cpu().numpy(), ref["scale_dn"])
    if ref["tensor_scale"] is not None:
        got = gpu_w.tensor_scale[group:group + 1].cpu().numpy()
        assert np.array_equal(got.view(np.uint32), ref["tensor_scale"].view(np.uint32)), (got, ref["tensor_scale"])


def assert_gemm_close(Y_gpu: np.ndarray, Y_ref: np.ndarray, S: np.ndarray, rel: float = 1e-5):
    """|Y_gpu - Y| <= rel * sum_k |x~_k w~_k| per element (fp64 oracle)."""
    err = np.abs(Y_gpu.astype(np.float64) - Y_ref)
    tol = rel * S
    bad = err > tol
    if bad.any():
        i = np.argwhere(bad)[0]
        raise AssertionError(f"{bad.sum()} of {bad.size} outputs out of tolerance; first {tuple(i)}: "
                             f"gpu={Y_gpu[tuple(i)]} oracle={Y_ref[tuple(i)]} tol={tol[tuple(i)]}")
    return float((err / np.maximum(S, 1e-300)).max())


def sample_pairs(rows: int, cols: int, n: int, seed: int = 0):
    rng = np.random.default_rng(seed)
    r = rng.integers(0, rows, n)
    c = rng.integers(0, cols, n)
    r = np.concatenate([r, [0, rows - 1, 0, rows - 1]])
    c = np.concatenate([c, [0, cols - 1, cols - 1, 0]])
    return r, c


def run_case(case, fmt=None, eps=1e-6):
    """GPU prepare + pack + linear of a LinearCase; returns (act, weight, Y)."""
    fmt = fmt or case.fmt
    act = ops.prepare(dev_x(case), dev_gamma(case.gamma), eps, fmt)
    w = ops.pack_weight(dev_w(case.w, case.dtype), fmt)
    Y = ops.linear(act, w)
    torch.cuda.synchronize()
    return act, w, Y
