"""Pins of the oracle's fused preparation (RMSNorm, 4:8 in-pairs mask,
backbone quantization and compaction, residual) against hand-derived values,
closed forms, brute force and the decomposition identities of the pages."""
import itertools
from fractions import Fraction

import numpy as np
import pytest

from oracle import formats as F
from oracle import sharq as O
from conftest import read_golden
from sparsity_sharq_prepare_amd import synth

F32 = np.float32


def hexbytes(row):
    return np.array([int(b, 16) for b in row], dtype=np.uint8)


# --------------------------------------------------------------------- RMSNorm
def test_pairwise_sum_order():
    # squares 2^24, 1, 1, 1: pairwise (2^24 + 1) + (1 + 1) = 2^24 + 2, while a
    # left-to-right fp32 sum stays at 2^24
    a = np.array([[2.0 ** 24, 1.0, 1.0, 1.0]], dtype=F32)
    assert O.pairwise_sum_f32(a)[0] == F32(2.0 ** 24 + 2)
    # zero padding to a power of two: (2^24 + 1) + (1 + 0) -> 2^24 + 0 ... = 2^24
    b = np.array([[2.0 ** 24, 1.0, 1.0]], dtype=F32)
    assert O.pairwise_sum_f32(b)[0] == F32(2.0 ** 24)
    # exact small sums
    c = np.arange(1, 101, dtype=F32)[None]
    assert O.pairwise_sum_f32(c)[0] == 5050


def test_rmsnorm_closed_forms():
    # x = (3, 4), eps = 0: mean square 12.5, y = x / sqrt(12.5) * gamma
    y = O.rmsnorm(np.array([[3.0, 4.0]], F32), np.array([1.0, 2.0], F32), 0.0)
    ref = np.array([3.0, 8.0]) / np.sqrt(12.5)
    assert np.allclose(y[0], ref, rtol=1e-6)
    # constant row c: y = c / sqrt(c^2 + eps) * gamma
    K = 4096
    for c in (0.5, 3.0, 100.0):
        g = np.linspace(0.5, 1.5, K).astype(F32)
        y = O.rmsnorm(np.full((1, K), c, F32), g, 1e-6)
        ref = c / np.sqrt(c * c + 1e-6) * g.astype(np.float64)
        assert np.allclose(y[0], ref, rtol=3e-7, atol=0)
    # random rows agree with an fp64 RMSNorm to a few fp32 ulps
    rng = np.random.default_rng(5)
    x = rng.standard_normal((4, 768)).astype(F32) * 7
    g = rng.uniform(0.5, 1.5, 768).astype(F32)
    y = O.rmsnorm(x, g, 1e-6)
    x64 = x.astype(np.float64)
    ref = x64 / np.sqrt((x64 ** 2).mean(axis=1, keepdims=True) + 1e-6) * g
    assert np.allclose(y, ref, rtol=1e-6, atol=0)
    # gamma None: no normalization
    assert np.array_equal(O.rmsnorm(x, None, 1e-6), x)


def test_rmsnorm_zero_row():
    y = O.rmsnorm(np.zeros((1, 64), F32), np.ones(64, F32), 1e-6)
    assert np.all(y == 0)


# ------------------------------------------------------------------------ mask
def brute_top2(scores):
    """Among the 6 pair sets, the one with the largest exact score sum, ties to
    the lexicographically first set."""
    best = None
    for s in itertools.combinations(range(4), 2):
        tot = sum(Fraction(float(scores[p])) for p in s)
        if best is None or tot > best[0]:
            best = (tot, s)
    return best[1]


def scores_to_row(scores):
    # a group of 8 whose pair p holds (score_p, score_p / 2)
    row = []
    for s in scores:
        row += [s, s / 2]
    return np.array([row], dtype=F32)


def test_mask_exhaustive_integer_scores():
    for scores in itertools.product(range(4), repeat=4):
        i0, i1 = O.pair_top2(scores_to_row(scores))
        assert (int(i0[0, 0]), int(i1[0, 0])) == brute_top2(scores), scores


def test_mask_random_scores_bruteforce():
    rng = np.random.default_rng(7)
    y = (rng.standard_normal((64, 256)) * np.exp(rng.uniform(-20, 20, (64, 256)))).astype(F32)
    y[:, ::7] = y[:, 1::7][:, : y[:, ::7].shape[1]]  # force ties between pairs
    i0, i1 = O.pair_top2(y)
    s = O.pair_scores(y)
    for t in range(64):
        for g in range(32):
            assert (int(i0[t, g]), int(i1[t, g])) == brute_top2(s[t, g])


def test_mask_structure_two_whole_pairs():
    case = synth.random_case(11, 8, 512, 16)
    y = O.rmsnorm(case.x_f32(), case.gamma, 1e-6)
    i0, i1 = O.pair_top2(y)
    M = O.mask_from_pairs(i0, i1)
    grp = M.reshape(8, 64, 4, 2)
    assert np.all(grp[..., 0] == grp[..., 1])           # whole pairs
    assert np.all(grp[..., 0].sum(-1) == 2)             # 2 of 4 pairs -> 4 of 8 values
    assert np.all(i0 < i1)
    # the pair with the group's largest |y| is always kept
    top = np.abs(y.reshape(8, 64, 4, 2)).max(-1).argmax(-1)
    assert np.all((top == i0) | (top == i1))


def test_meta_encoding_hand():
    # group 0 keeps pairs (1, 3) -> nibble 1 | 3 << 2 = 0xD; group 1 keeps (0, 2) -> 0x8
    row = np.zeros((1, 16), F32)
    row[0, 2], row[0, 7] = 5.0, 4.0          # pairs 1 and 3 of group 0
    row[0, 8], row[0, 13] = -3.0, 2.0        # pairs 0 and 2 of group 1
    i0, i1 = O.pair_top2(row)
    assert O.meta_bytes(i0, i1).tolist() == [[0x8D]]


# ------------------------------------------------------------ worked example
def worked_example_row():
    x = np.full((1, 32), F32(0.2), dtype=F32)
    x[0, 5] = 12.0
    return x


def test_worked_example_explainer_block():
    g = {r[0]: r[1:] for r in read_golden("worked_example_block.txt")}
    p = O.prepare(worked_example_row(), None, fmt="mxfp4")
    assert np.array_equal(p["bb_meta"][0], hexbytes(g["meta"]))
    assert np.array_equal(p["bb_scale"][0], hexbytes(g["bb_scale"]))
    assert np.array_equal(p["bb_codes"][0], hexbytes(g["bb_codes"]))
    assert np.array_equal(p["res_scale"][0], hexbytes(g["res_scale"]))
    assert np.array_equal(p["res_codes"][0], hexbytes(g["res_codes"]))
    c, e = O.mx_quantize(worked_example_row())
    assert np.array_equal(O.pack_nibbles(c)[0], hexbytes(g["plain_codes"]))
    # SharQ keeps the small values the plain quantizer loses
    Xt, Rt = O.act_dequant(p)
    assert Xt[0, 5] == 12.0 and np.all(Rt[0, np.arange(32) != 5] == 0.1875)


# --------------------------------------------------------- decomposition laws
@pytest.mark.parametrize("fmt", ["mxfp4", "nvfp4"])
def test_decomposition_identities(fmt):
    case = synth.random_case(3, 24, 1024, 8, fmt=fmt)
    p = O.prepare(case.x_f32(), case.gamma, 1e-6, fmt=fmt)
    y, M, Xt_sp, R = p["y"], p["mask"], p["Xt_sp"], p["R"]
    # review §3.3: R = X - X~_sp, and X = X~_sp + R holds exactly in fp32
    assert np.array_equal(Xt_sp + R, y)
    # masked-out positions carry y unchanged in the residual; X~_sp is 0 there
    assert np.array_equal(R[~M], y[~M])
    assert np.all(Xt_sp[~M] == 0)
    # R = (X - X_sp) + (X_sp - X~_sp)
    assert np.array_equal(R, (y - p["X_sp"]) + (p["X_sp"] - Xt_sp))
    # backbone block amax equals the amax of y (the group max pair is kept)
    if fmt == "mxfp4":
        _, e_plain = O.mx_quantize(y)
        assert np.array_equal(F.e8m0_decode_exponent(p["bb_scale"]), e_plain)
    # the stored layouts decode back to the fp32 backbone
    Xt64, Rt64 = O.act_dequant(p)
    assert np.array_equal(Xt64.astype(F32), Xt_sp)
    # the residual error is at most half the widest E2M1 gap (2) times the
    # element step, which is below amax / 3 of the block
    blk = 32 if fmt == "mxfp4" else 16
    amax = np.abs(R).reshape(24, -1, blk).max(-1).repeat(blk, -1).astype(np.float64)
    assert np.all(np.abs(R - Rt64) <= amax / 3)


def test_on_grid_backbone_gives_zero_residual():
    # y already on the FP4 grid inside the mask and zero outside -> R == 0,
    # residual codes 0, residual scale byte 0 (all-zero block: e = -127)
    row = np.zeros((1, 64), F32)
    row[0, [0, 1, 6, 7]] = [6.0, -3.0, 0.5, 1.5]
    row[0, [8, 9, 10, 11]] = [2.0, 4.0, -1.0, 0.0]
    row[0, 32:40] = [1.0, 1.0, 1.0, 1.0, 0.0, 0.0, 0.0, 0.0]
    p = O.prepare(row, None, fmt="mxfp4")
    assert np.all(p["R"] == 0)
    assert np.all(p["res_codes"] == 0) and np.all(p["res_scale"] == 0)


def test_all_zero_row():
    p = O.prepare(np.zeros((2, 64), F32), np.ones(64, F32), 1e-6, fmt="mxfp4")
    assert np.all(p["bb_meta"] == 0x44)       # ties everywhere -> pairs (0, 1)
    assert np.all(p["bb_codes"] == 0) and np.all(p["res_codes"] == 0)
    assert np.all(p["bb_scale"] == 0) and np.all(p["res_scale"] == 0)


# ---------------------------------------------------------------- NVFP4 (emu)
def test_nvfp4_hand_block():
    # tensor amax 2688 -> s_T = 2688 / 2688 = 1; block amax 6 -> u = 1 -> E4M3 0x38,
    # d = 1, codes are plain E2M1 of the values
    v = np.array([[2688.0] + [0.0] * 15 + [6.0, -3.0, 0.75, 1.25] + [0.0] * 12], F32)
    s = O.nv_tensor_scale(np.abs(v).max())
    assert s == 1.0
    codes, sc = O.nv_quantize(v, 16, s)
    assert sc.tolist() == [[0x7E, 0x38]]     # 2688 / 6 = 448 -> 0x7E
    assert codes[0, 16:20].tolist() == [7, 0xD, 2, 2]
    assert codes[0, 0] == 7                  # 2688 / (448 * 1) = 6
    # block amax 6.5 -> u = 1.0833 -> 1.125 (0x39); 6.5 / 1.125 = 5.78 -> 6 (code 7)
    v2 = np.array([[6.5] + [0.0] * 15], F32)
    c2, s2 = O.nv_quantize(v2, 16, F32(1.0))
    assert s2.tolist() == [[0x39]] and c2[0, 0] == 7
    # all-zero tensor -> s_T = 1, scale 0, signed zero codes
    c3, s3 = O.nv_quantize(np.array([[-0.0] + [0.0] * 15], F32), 16, O.nv_tensor_scale(0.0))
    assert s3.tolist() == [[0]] and c3[0, 0] == 8 and np.all(c3[0, 1:] == 0)


def test_nvfp4_residual_size_4p5_bits():
    # explainer: NVFP4 stores 16 E2M1 values with one E4M3 scale = 4.5 bits/value
    case = synth.random_case(4, 4, 512, 8, fmt="nvfp4")
    p = O.prepare(case.x_f32(), case.gamma, 1e-6, fmt="nvfp4")
    bits = (p["res_codes"].shape[1] + p["res_scale"].shape[1]) * 8 / 512
    assert bits == 4.5


# --------------------------------------------------------- N:M masks (2:4)
def test_nm_keep_matches_pair_rule_and_brute_force():
    rng = np.random.default_rng(17)
    y = rng.integers(0, 4, (40, 64)).astype(np.float32) * np.where(rng.random((40, 64)) < 0.5, -1, 1)
    # 4:8 in pairs is the general rule with units of 2
    assert np.array_equal(O.nm_keep(y, 4, 8, unit=2), O.mask_from_pairs(*O.pair_top2(y)))
    # 2:4: brute force over the 6 choices; the first (lexicographic) choice
    # with the largest sum of |y| (integer scores: ties are frequent)
    M = O.nm_keep(y, 2, 4)
    import itertools
    combos = list(itertools.combinations(range(4), 2))
    for t in range(y.shape[0]):
        for g in range(16):
            a = np.abs(y[t, 4 * g: 4 * g + 4])
            best = max(combos, key=lambda c: (a[c[0]] + a[c[1]], -combos.index(c)))
            exp = np.zeros(4, bool)
            exp[list(best)] = True
            assert np.array_equal(M[t, 4 * g: 4 * g + 4], exp), (t, g, a)
    assert np.all(M.reshape(40, 16, 4).sum(-1) == 2)


def test_prepare_24_worked_example_and_identities():
    # the explainer's block (one 12 among 0.2s) with the 2:4 backbone:
    # group 1 (k = 4..7) keeps k = 5 (the 12) and k = 4 (ties to the lower
    # index); every other group keeps its first two positions
    x = np.full((1, 32), np.float32(0.2), dtype=np.float32)
    x[0, 5] = 12.0
    p = O.prepare(x, None, fmt="mxfp4", mask="2:4")
    assert p["bb_meta"][0].tolist() == [0x44] * 4             # nibble 0 | 1 << 2 = 4 in every group
    # backbone scale 2^1 (amax 12): 0.2 / 2 -> 0, 12 / 2 = 6 -> code 7
    assert p["bb_scale"][0].tolist() == [128]
    assert p["bb_codes"][0].tolist() == [0x00, 0x70, 0, 0, 0, 0, 0, 0]
    # residual: 0 at k = 5, 0.2 elsewhere -> scale 2^-4, 0.2 * 16 = 3.2 -> code 5
    assert p["res_scale"][0].tolist() == [123]
    Xt, Rt = O.act_dequant(p)
    assert Xt[0, 5] == 12.0 and np.all(Xt[0, np.arange(32) != 5] == 0)
    assert np.all(Rt[0, np.arange(32) != 5] == 0.1875) and Rt[0, 5] == 0
    # y = X~_sp + R bit for bit; exactly 2 of every 4 kept
    case = synth.random_case(5, 6, 512, 8)
    q = O.prepare(case.x_f32(), case.gamma, 1e-6, "mxfp4", mask="2:4")
    assert np.array_equal(q["Xt_sp"] + q["R"], q["y"])
    assert np.all(q["mask"].reshape(6, -1, 4).sum(-1) == 2)
    with pytest.raises(ValueError):
        O.prepare(case.x_f32(), case.gamma, 1e-6, "nvfp4", mask="2:4")
