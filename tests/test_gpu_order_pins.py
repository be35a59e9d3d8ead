"""The hand-derived order fixtures (RMSNorm chain and operation order,
two-level NVFP4 scaling at a tensor scale other than 1) run through the HIP
library: the GPU must give the fixtures' bits directly, and every other byte
must equal the oracle's."""
import numpy as np
import pytest
import torch

from oracle import sharq as O
from sparsity_sharq_prepare_amd import ops

from gpu_util import compare_act, compare_weight
from test_oracle_order_pins import chain_row, golden_map, nvfp4_row, rmsnorm_row

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True, scope="module")
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    yield


def _rows():
    g1 = golden_map("rmsnorm_order_row.txt")
    x1, gamma1 = rmsnorm_row(g1)
    g2 = golden_map("rmsnorm_chain_row.txt")
    x2, gamma2, eps2 = chain_row(g2)
    return [(g1, x1, gamma1, float(g1["eps"][0])), (g2, x2, gamma2, eps2)]


@pytest.mark.parametrize("which", [0, 1], ids=["order_k32", "chain_k96"])
def test_rmsnorm_fixture_rows(which):
    g, x, gamma, eps = _rows()[which]
    X = torch.from_numpy(x).cuda()
    G = torch.from_numpy(gamma).cuda()
    y = ops.rmsnorm(X, G, eps)
    torch.cuda.synchronize()
    yb = y.cpu().numpy().view(np.uint32)[0]
    assert yb[5] == int(g["y5"][0], 16)
    if "y18" in g:
        assert yb[18] == int(g["y18"][0], 16)
    assert np.array_equal(yb, O.rmsnorm(x, gamma, eps).view(np.uint32)[0])
    for fmt in ("mxfp4", "nvfp4", "mxfp4_24"):
        act = ops.prepare(X, G, eps, fmt)
        base = "nvfp4" if fmt == "nvfp4" else "mxfp4"
        compare_act(act, O.prepare(x, gamma, eps, base, mask="2:4" if fmt == "mxfp4_24" else "4:8"))


def test_nvfp4_fixture_row_prepare_and_pack():
    g = golden_map("nvfp4_scale_order_row.txt")
    x = nvfp4_row(g)
    X = torch.from_numpy(x).cuda()
    act = ops.prepare(X, None, 1e-6, "nvfp4")
    torch.cuda.synchronize()
    got = act.as_numpy()
    assert got["tensor_scales"][:1].view(np.uint32)[0] == int(g["s_T"][0], 16)
    assert got["bb_scale"][0].tolist() == [int(h, 16) for h in g["scales"]]
    assert got["bb_meta"][0].tolist() == [int(h, 16) for h in g["bb_meta"]]
    bb = got["bb_codes"][0].reshape(-1, 2)
    for grp in (0, 4, 8):
        assert bb[grp].tolist() == [int(h, 16) for h in g["bb_group%d" % grp]], grp
    compare_act(act, O.prepare(x, None, 1e-6, "nvfp4"))
    # the same column as a K x 1 weight: the packer's scales and codes
    W = torch.from_numpy(x.reshape(-1, 1).copy()).cuda().contiguous()
    w = ops.pack_weight(W, "nvfp4")
    torch.cuda.synchronize()
    assert w.tensor_scale.cpu().numpy().view(np.uint32)[0] == int(g["s_T"][0], 16)
    assert w.scale_sp[0, 0].cpu().numpy().tolist() == [int(h, 16) for h in g["scales"]]
    pay = w.payload[0, 0].cpu().numpy()
    codes = np.empty(2 * pay.size, np.uint8)
    codes[0::2], codes[1::2] = pay & 0xF, pay >> 4
    for k in (0, 32, 64, 66):
        assert codes[k] == int(g["code%d" % k][0]), k
    compare_weight(w, O.pack_weight(x.T.copy(), "nvfp4"))
