"""The review's Table 5 path combinations (§5.3: sparse only, sparse +
sparse, dense + dense, SharQ, plain FP4; and the 2:4 backbone) computed with
the library's kernels and compared piece by piece with the oracle's
``decomposition_pieces``: every quantized piece's bytes bit for bit, every
piece's GEMM output within 1e-5 * sum_k |x~_k w~_k| of the fp64 product, and
the relative Frobenius errors of the combinations against the oracle study's.

The second paths take their fp32 inputs (R = y - X~_sp, and y - Q(y)) from the
oracle: both are exact fp32 differences, and the GPU's quantization of them is
what is under test."""
import numpy as np
import pytest
import torch

from oracle import sharq as O
from sparsity_sharq_prepare_amd import ops, synth

from gpu_util import assert_bytes_equal, assert_gemm_close, compare_act, dev_gamma, dev_w, dev_x

pytestmark = pytest.mark.gpu

BB_KEYS = ("bb_codes", "bb_meta", "bb_scale")


@pytest.fixture(autouse=True, scope="module")
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    yield


def backbone_only(act):
    """The prepared activations with the residual codes zeroed: the sparse
    path alone through the dual GEMM."""
    a = ops.empty_act(act.fmt, act.T, act.K)
    for k in BB_KEYS + ("res_scale",):
        getattr(a, k).copy_(getattr(act, k))
    if act.tensor_scales is not None:
        a.tensor_scales.copy_(act.tensor_scales)
    a.res_codes.zero_()
    return a


def gemm_check(Y_gpu, V, W):
    """Y_gpu against V @ W (fp64) within 1e-5 * |V| @ |W|."""
    return assert_gemm_close(Y_gpu.astype(np.float64), V @ W, np.abs(V) @ np.abs(W))


CASES = [("decode_4096x4096", None), ("random_64x1024x300", (64, 1024, 300))]


@pytest.mark.parametrize("name,shape", CASES, ids=[c[0] for c in CASES])
def test_table5_mxfp4_pieces(name, shape):
    case = synth.decode_case(0) if shape is None else synth.random_case(55, *shape)
    x, g = case.x_f32(), case.gamma
    pc = O.decomposition_pieces(x, g, "mxfp4")
    wp = O.pack_weight(case.w_f32(), "mxfp4")
    W = O.weight_dequant(wp, "dn")
    X, G = dev_x(case), dev_gamma(g)
    w = ops.pack_weight(dev_w(case.w, case.dtype), "mxfp4")
    # SharQ: the fused preparation and the dual GEMM
    act = ops.prepare(X, G, 1e-6, "mxfp4")
    compare_act(act, pc["prep"])
    Y_sharq = ops.linear(act, w)
    # sparse only: the backbone alone
    Y_sp1 = ops.linear(backbone_only(act), w)
    # sparse + sparse: the pair-top-2 rule and backbone quantization applied to R
    R = torch.from_numpy(np.ascontiguousarray(pc["R"])).cuda()
    act_r = ops.prepare(R, None, 1e-6, "mxfp4")
    ref_r = O.prepare(pc["R"], None, 1e-6, "mxfp4")
    torch.cuda.synchronize()
    got_r = act_r.as_numpy()
    for k in BB_KEYS:
        assert_bytes_equal("sparse_second " + k, got_r[k], ref_r[k])
    Y_sp2 = ops.linear(backbone_only(act_r), w)
    # dense + dense: y quantized densely, then its residual densely
    y = ops.rmsnorm(X, G, 1e-6)
    c1, s1 = ops.quantize_mx(y)
    ymq = torch.from_numpy(np.ascontiguousarray(pc["y_minus_q"])).cuda()
    c2, s2 = ops.quantize_mx(ymq)
    ref1, ref2 = O.plain_prepare_mx(x, g), O.plain_prepare_mx(pc["y_minus_q"], None)
    torch.cuda.synchronize()
    assert_bytes_equal("y bits", y.cpu().numpy().view(np.uint32), pc["y"].view(np.uint32))
    assert_bytes_equal("dense_first codes", c1.cpu().numpy(), ref1["codes"])
    assert_bytes_equal("dense_first scales", s1.cpu().numpy(), ref1["scales"])
    assert_bytes_equal("dense_second codes", c2.cpu().numpy(), ref2["codes"])
    assert_bytes_equal("dense_second scales", s2.cpu().numpy(), ref2["scales"])
    Y_d1, Y_d2 = ops.linear_dense(c1, s1, w), ops.linear_dense(c2, s2, w)
    # 2:4 backbone and its dense residual
    act24 = ops.prepare(X, G, 1e-6, "mxfp4_24")
    compare_act(act24, O.prepare(x, g, 1e-6, "mxfp4", mask="2:4"))
    Y_24 = ops.linear(act24, w)
    Y_24sp = ops.linear(backbone_only(act24), w)
    torch.cuda.synchronize()
    Yg = {k: v.cpu().numpy() for k, v in dict(sharq=Y_sharq, sp1=Y_sp1, sp2=Y_sp2, d1=Y_d1, d2=Y_d2, s24=Y_24,
                                                s24sp=Y_24sp).items()}
    # every piece's GEMM against the exact product of the oracle's piece
    gemm_check(Yg["sp1"], pc["sparse_first"], W)
    gemm_check(Yg["sp2"], pc["sparse_second"], W)
    gemm_check(Yg["d1"], pc["dense_first"], W)
    gemm_check(Yg["d2"], pc["dense_second"], W)
    gemm_check(Yg["sharq"], pc["sparse_first"] + pc["dense_residual"], W)
    gemm_check(Yg["s24sp"], pc["sparse_first_24"], W)
    gemm_check(Yg["s24"], pc["sparse_first_24"] + pc["dense_residual_24"], W)
    # the combinations' errors agree with the oracle study's
    st = O.decomposition_study(x, g, case.w_f32(), "mxfp4", wp=wp)["weights_fp4"]
    ref = pc["y"].astype(np.float64) @ case.w_f32().astype(np.float64)
    gpu = {"sparse_only": Yg["sp1"], "sparse_sparse": Yg["sp1"].astype(np.float64) + Yg["sp2"],
           "dense_dense": Yg["d1"].astype(np.float64) + Yg["d2"], "sharq": Yg["sharq"], "plain": Yg["d1"],
           "sparse_only_2:4": Yg["s24sp"], "sharq_2:4": Yg["s24"]}
    for k, v in gpu.items():
        e = O.rel_frobenius(np.asarray(v, np.float64), ref)
        assert abs(e - st[k]) <= 1e-4 * st[k], (k, e, st[k])
    # the pages' ordering: sparse only worst, SharQ below sparse + sparse and plain
    assert st["sparse_only"] > st["sparse_sparse"] > st["sharq"] and st["plain"] > st["sharq"]


def test_table5_nvfp4_pieces():
    case = synth.random_case(66, 64, 3584, 200, fmt="nvfp4", spec=synth.QWEN_OUTLIERS)
    x, g = case.x_f32(), case.gamma
    pc = O.decomposition_pieces(x, g, "nvfp4")
    wp = O.pack_weight(case.w_f32(), "nvfp4")
    W_sp, W_dn = O.weight_dequant(wp, "sp"), O.weight_dequant(wp, "dn")
    X, G = dev_x(case), dev_gamma(g)
    w = ops.pack_weight(dev_w(case.w, case.dtype), "nvfp4")
    act = ops.prepare(X, G, 1e-6, "nvfp4")
    compare_act(act, pc["prep"])
    Y_sharq = ops.linear(act, w)
    Y_sp1 = ops.linear(backbone_only(act), w)
    R = torch.from_numpy(np.ascontiguousarray(pc["R"])).cuda()
    act_r = ops.prepare(R, None, 1e-6, "nvfp4")
    ref_r = O.prepare(pc["R"], None, 1e-6, "nvfp4")
    torch.cuda.synchronize()
    got_r = act_r.as_numpy()
    for k in BB_KEYS:
        assert_bytes_equal("sparse_second " + k, got_r[k], ref_r[k])
    assert got_r["tensor_scales"][:1].view(np.uint32)[0] == ref_r["tensor_scales"][:1].view(np.uint32)[0]
    Y_sp2 = ops.linear(backbone_only(act_r), w)
    torch.cuda.synchronize()
    # both paths read the sparse (per 32) weight view; the dense view holds
    # the same scales twice, so the two products agree
    assert np.array_equal(W_sp, W_dn)
    gemm_check(Y_sp1.cpu().numpy(), pc["sparse_first"], W_sp)
    gemm_check(Y_sp2.cpu().numpy(), pc["sparse_second"], W_sp)
    gemm_check(Y_sharq.cpu().numpy(), pc["sparse_first"] + pc["dense_residual"], W_sp)
