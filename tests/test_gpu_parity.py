"""GPU parity: the HIP library (through the C ABI) against the CPU oracle on
the same seeded inputs.  Codes, scales, metadata and tensor scales must be
bit-exact; fp32 GEMM outputs must lie within 1e-5 * sum_k |x~_k w~_k| of the
fp64 oracle."""
import numpy as np
import pytest
import torch

from oracle import sharq as O
from sparsity_sharq_prepare_amd import ops, synth

from gpu_util import (assert_bytes_equal, assert_gemm_close, compare_act, compare_weight, dev_gamma, dev_w, dev_x,
                      run_case, sample_pairs)

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True, scope="module")
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    yield


def oracle_prepare(case, fmt=None, eps=1e-6):
    return O.prepare(case.x_f32(), case.gamma, eps, fmt or case.fmt)


# ------------------------------------------------------------------ prepare
def test_prepare_tiny_config():
    case = synth.tiny_case()
    act = ops.prepare(dev_x(case), dev_gamma(case.gamma), 1e-6, "mxfp4")
    compare_act(act, oracle_prepare(case))


PREP_SHAPES = [  # (T, K, dtype, gamma): spans 64/128/256 threads per row, 1..16 chunks, ragged T
    (37, 256, "bf16", True), (5, 768, "bf16", True), (3, 32, "f32", True), (64, 4096, "bf16", False),
    (17, 14336, "bf16", True), (9, 18944, "bf16", True), (33, 2048, "f32", True), (2, 3584, "bf16", True),
    (1, 96, "bf16", True), (300, 512, "bf16", True),
    # one wave per row, rows looped per workgroup (ragged last block; fp32 rows not prefetched)
    (4099, 2048, "bf16", True), (2100, 4096, "f32", True),
]


@pytest.mark.parametrize("fmt", ["mxfp4", "nvfp4"])
@pytest.mark.parametrize("T,K,dtype,gamma", PREP_SHAPES)
def test_prepare_shapes(T, K, dtype, gamma, fmt):
    case = synth.random_case(T * 7 + K, T, K, 8, fmt=fmt, dtype=dtype, gamma=gamma)
    act = ops.prepare(dev_x(case), dev_gamma(case.gamma), 1e-6, fmt)
    compare_act(act, oracle_prepare(case))


@pytest.mark.parametrize("fmt", ["mxfp4", "nvfp4"])
def test_prepare_edge_rows(fmt):
    # zero row, worked-example row (one 12 among 0.2s), signed zeros, tiny and
    # large magnitudes, exact ties between pairs
    K = 64
    x = np.zeros((6, K), np.float32)
    x[1, :] = 0.2
    x[1, 5] = 12.0
    x[2, ::2] = -0.0
    x[2, 1::2] = 1e-30
    x[3, :] = np.float32(3.0e30) * np.cos(np.arange(K))
    x[4, :] = np.tile(np.array([1, -1, 1, -1, 2, 2, -2, -2], np.float32), K // 8)
    x[5, :] = np.float32(1e-38) * np.arange(K)
    case = synth.LinearCase("edge", fmt, "f32", 6, K, 8, x, None, np.zeros((K, 8), np.float32))
    act = ops.prepare(dev_x(case), None, 1e-6, fmt)
    compare_act(act, O.prepare(x, None, 1e-6, fmt))
    g = np.ones(K, np.float32)
    act = ops.prepare(dev_x(case), dev_gamma(g), 1e-6, fmt)
    compare_act(act, O.prepare(x, g, 1e-6, fmt))


def test_prepare_nvfp4_code_midpoints():
    # NVFP4 element codes at and next to the E2M1 rounding midpoints, where the
    # kernel's reciprocal-based fast path must defer to the correctly rounded
    # division: x = 2688 somewhere makes the backbone tensor scale exactly 1,
    # each 32-block's maximum 6 * 2^j makes its scale 2^j exactly, and the other
    # values sit on midpoints (and grid points) times 2^j, moved by 0, +-1,
    # +-2, +-4, +-8 and +-64 ulp
    rng = np.random.default_rng(7)
    T, K = 16, 512
    mids = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0], np.float32)
    steps = np.array([0, 1, -1, 2, -2, 4, -4, 8, -8, 64, -64], np.int32)
    base = mids[rng.integers(0, len(mids), (T, K))]
    bits = base.view(np.int32) + steps[rng.integers(0, len(steps), (T, K))]
    x = bits.view(np.float32) * np.where(rng.random((T, K)) < 0.5, -1, 1).astype(np.float32)
    j = rng.integers(-6, 7, (T, K // 32)).astype(np.float32)
    x = x * np.repeat(np.exp2(j), 32, axis=1).astype(np.float32)
    x[:, ::32] = np.float32(6.0) * np.exp2(j).astype(np.float32)       # block maxima
    x[0, 0] = np.float32(2688.0)                                        # tensor amax
    x = x.astype(np.float32)
    case = synth.LinearCase("midpoints", "nvfp4", "f32", T, K, 8, x, None, np.zeros((K, 8), np.float32))
    act = ops.prepare(dev_x(case), None, 1e-6, "nvfp4")
    ref = O.prepare(x, None, 1e-6, "nvfp4")
    compare_act(act, ref)
    # the construction reaches the intended scales: the backbone tensor scale
    # is exactly 1
    assert ref["tensor_scales"][0] == np.float32(1.0)


DECODE_IDS = [f"{K}x{D}" for K, D in synth.DECODE_SHAPES]
NVFP4_IDS = [f"{K}x{D}" for K, D in synth.NVFP4_SHAPES]


@pytest.mark.parametrize("i", range(3), ids=DECODE_IDS)
def test_prepare_decode_full(i):
    case = synth.decode_case(i)
    act = ops.prepare(dev_x(case), dev_gamma(case.gamma), 1e-6, "mxfp4")
    compare_act(act, oracle_prepare(case))


def test_prepare_prefill_full_and_deterministic():
    case = synth.prefill_case(D=256)          # the activation of the 4096 x 4096 x 14336 prefill
    X, g = dev_x(case), dev_gamma(case.gamma)
    a1 = ops.prepare(X, g, 1e-6, "mxfp4")
    s2 = torch.cuda.Stream()
    with torch.cuda.stream(s2):
        a2 = ops.prepare(X, g, 1e-6, "mxfp4", stream=s2)
    s2.synchronize()
    compare_act(a1, oracle_prepare(case))
    for k in ("bb_codes", "bb_meta", "bb_scale", "res_codes", "res_scale"):
        assert torch.equal(getattr(a1, k), getattr(a2, k)), k


# ------------------------------------------------------------------ packer
PACK_SHAPES = [(256, 256, "f32"), (256, 100, "bf16"), (160, 70, "bf16"), (4096, 4096, "bf16"), (96, 513, "f32")]


@pytest.mark.parametrize("fmt", ["mxfp4", "nvfp4"])
@pytest.mark.parametrize("K,D,dtype", PACK_SHAPES)
def test_pack_shapes(K, D, dtype, fmt):
    case = synth.random_case(K + D, 1, K, D, fmt=fmt, dtype=dtype)
    w = ops.pack_weight(dev_w(case.w, dtype), fmt)
    compare_weight(w, O.pack_weight(case.w_f32(), fmt))


def test_pack_grouped_and_full_decode_weight():
    case = synth.decode_cases()[1]             # 4096 x 14336
    w = ops.pack_weight(dev_w(case.w, "bf16"), "mxfp4")
    compare_weight(w, O.pack_weight(case.w_f32(), "mxfp4"))
    rng = np.random.default_rng(3)
    W = synth.f32_to_bf16_bits(rng.standard_normal((3, 256, 96)).astype(np.float32) * 0.02)
    for fmt in ("mxfp4", "nvfp4"):
        wg = ops.pack_weight(dev_w(W, "bf16"), fmt)
        for e in range(3):
            compare_weight(wg, O.pack_weight(synth.bf16_bits_to_f32(W[e]), fmt), group=e)


# ------------------------------------------------------------------ dual GEMM
def test_linear_tiny_config():
    case = synth.tiny_case()
    act, w, Y = run_case(case)
    compare_act(act, oracle_prepare(case))
    Yr, S = O.sharq_linear(oracle_prepare(case), O.pack_weight(case.w_f32()))
    assert_gemm_close(Y.cpu().numpy(), Yr, S)


LINEAR_SHAPES = [  # decode (T <= 16), batch (9-64 rows), skinny and tile paths, ragged rows and columns
    (1, 512, 200), (8, 512, 200), (13, 256, 64), (64, 384, 130), (65, 512, 300), (300, 512, 520),
    (256, 1024, 256), (700, 128, 40),
    # K % 512 != 0 on the tile path: 3, 5 and 6 steps of 128 (a partial last
    # group of four steps; 24-byte scale rows at K = 768)
    (100, 384, 72), (257, 640, 300), (333, 768, 250),
    # decode path (<= 8 rows): uneven steps per wave, the largest staged K, and
    # a K beyond it (general skinny path)
    (5, 1152, 72), (7, 16384, 48), (2, 18944, 40),
    # decode path with two MFMA tiles (9-16 rows): ragged rows, column
    # groups, the largest staged K (7168); beyond it the batch kernel with
    # two MFMA tiles (column groups of 1, 2 and 4, K past the decode
    # kernel's)
    (16, 4096, 300), (9, 1152, 72), (12, 2048, 4100), (11, 7168, 64), (16, 7296, 40),
    (9, 14336, 72), (10, 16512, 40), (13, 8192, 6500), (16, 14336, 13000),
    # 17-64 rows: the batch kernel (32 or 64 MFMA rows; column groups of 1,
    # 2 and 4; partial last K chunks; K beyond the decode kernel's; wide
    # outputs)
    (17, 512, 64), (32, 4096, 300), (40, 2048, 4100), (57, 1152, 200), (64, 7168, 48), (64, 7296, 40),
    (33, 14336, 72), (40, 16512, 48), (64, 16512, 40), (24, 640, 13000), (64, 384, 8200), (48, 18944, 130),
    (40, 1024, 13000), (20, 7296, 12800),
    # degenerate widths: one output column, the smallest GEMM K
    (3, 256, 1), (70, 512, 1), (1, 128, 16),
]


@pytest.mark.parametrize("T,K,D", LINEAR_SHAPES)
def test_linear_shapes(T, K, D):
    case = synth.random_case(T + 3 * K + D, T, K, D)
    act, w, Y = run_case(case)
    ref = oracle_prepare(case)
    compare_act(act, ref)
    Yr, S = O.sharq_linear(ref, O.pack_weight(case.w_f32()))
    assert_gemm_close(Y.cpu().numpy(), Yr, S)


@pytest.mark.parametrize("T,K,n", [(8, 256, 13), (200, 256, 205), (6, 256, 5), (12, 8192, 14), (30, 1024, 50),
                                   (20, 8192, 27)])
def test_linear_row_gather(T, K, n):
    # n gathered output rows: the two-tile decode kernel (13), the tile path
    # (205), the one-tile decode kernel (5), and the batch kernel with two
    # (14 rows at K = 8192), eight (50 rows) and four (27 rows at K = 8192)
    # MFMA tiles
    case = synth.random_case(99 + T, T, K, 96)
    act = ops.prepare(dev_x(case), dev_gamma(case.gamma), 1e-6)
    w = ops.pack_weight(dev_w(case.w, "bf16"))
    rows = np.random.default_rng(T).integers(0, T, n).astype(np.int32)
    Y = ops.linear(act, w, row_index=torch.from_numpy(rows).cuda())
    Yr, S = O.sharq_linear(oracle_prepare(case), O.pack_weight(case.w_f32()), rows=rows)
    assert_gemm_close(Y.cpu().numpy(), Yr, S)


@pytest.mark.parametrize("i", range(3), ids=DECODE_IDS)
def test_linear_decode_full_sampled(i):
    case = synth.decode_case(i)
    act, w, Y = run_case(case)
    ref = oracle_prepare(case)
    compare_act(act, ref)
    r, c = sample_pairs(case.T, case.D, 3000, seed=case.K)
    Yr, S = O.sharq_linear_sampled(ref, O.pack_weight(case.w_f32()), r, c)
    assert_gemm_close(Y.cpu().numpy()[r, c], Yr, S)


@pytest.mark.parametrize("i", range(3), ids=DECODE_IDS)
@pytest.mark.parametrize("T", [16, 40, 64])
def test_linear_decode_batch_full_sampled(T, i):
    # batched decode at the full Llama-3.1-8B shapes: 16 rows on the two-tile
    # decode kernel (the two-tile batch kernel at K = 14336), 40 and 64 rows
    # on the batch kernel (one and four column groups)
    case = synth.decode_case(i, T=T)
    act, w, Y = run_case(case)
    ref = oracle_prepare(case)
    compare_act(act, ref)
    r, c = sample_pairs(case.T, case.D, 3000, seed=case.K + T)
    Yr, S = O.sharq_linear_sampled(ref, O.pack_weight(case.w_f32()), r, c)
    assert_gemm_close(Y.cpu().numpy()[r, c], Yr, S)


def test_linear_prefill_full_sampled_and_deterministic():
    case = synth.prefill_case()
    act, w, Y = run_case(case)
    Y2 = ops.linear(act, w)
    torch.cuda.synchronize()
    assert torch.equal(Y, Y2)
    ref = oracle_prepare(case)
    r, c = sample_pairs(case.T, case.D, 3000, seed=1)
    cols = np.unique(c)
    wref = O.weight_cols(O.pack_weight(case.w_f32()[:, cols]), slice(None))
    ci = np.searchsorted(cols, c)
    Yr, S = O.sharq_linear_sampled(ref, wref, r, ci)
    assert_gemm_close(Y.cpu().numpy()[r, c], Yr, S)


@pytest.mark.parametrize("T,K,D", [(4096, 512, 4096), (4000, 1024, 3000)])
def test_linear_tile_widths_sampled(T, K, D):
    # 4096 x 4096: 256 tiles of 256 columns fill one round, so the 256-wide
    # tile is chosen; 4000 x 3000: 224-wide tiles with ragged rows and columns
    case = synth.random_case(T + K + D, T, K, D)
    act, w, Y = run_case(case)
    ref = oracle_prepare(case)
    r, c = sample_pairs(case.T, case.D, 2000, seed=2)
    cols = np.unique(c)
    wref = O.weight_cols(O.pack_weight(case.w_f32()[:, cols]), slice(None))
    ci = np.searchsorted(cols, c)
    Yr, S = O.sharq_linear_sampled(ref, wref, r, ci)
    assert_gemm_close(Y.cpu().numpy()[r, c], Yr, S)


# ------------------------------------------------------------------ NVFP4 (emulated)
@pytest.mark.parametrize("T,K,D", [(16, 256, 64), (130, 512, 200), (64, 3584, 300)])
def test_nvfp4_linear_shapes(T, K, D):
    case = synth.random_case(T + K + D + 1, T, K, D, fmt="nvfp4", spec=synth.QWEN_OUTLIERS)
    act, w, Y = run_case(case)
    ref = oracle_prepare(case)
    compare_act(act, ref)
    wref = O.pack_weight(case.w_f32(), "nvfp4")
    compare_weight(w, wref)
    Yr, S = O.sharq_linear(ref, wref)
    assert_gemm_close(Y.cpu().numpy(), Yr, S)


@pytest.mark.parametrize("i", range(2), ids=NVFP4_IDS)
def test_nvfp4_full_sampled(i):
    case = synth.nvfp4_cases(shapes=[synth.NVFP4_SHAPES[i]])[0]
    act, w, Y = run_case(case)
    ref = oracle_prepare(case)
    compare_act(act, ref)
    r, c = sample_pairs(case.T, case.D, 2000, seed=2)
    cols = np.unique(c)
    Wf = case.w_f32()
    # the tensor scale belongs to the whole weight: pack the sampled columns under it
    wsub = O.pack_weight(np.ascontiguousarray(Wf[:, cols]), "nvfp4", tensor_amax=np.abs(Wf).max())
    assert np.array_equal(w.tensor_scale.cpu().numpy(), wsub["tensor_scale"])
    compare_weight_cols(w, wsub, cols)
    Yr, S = O.sharq_linear_sampled(ref, wsub, r, np.searchsorted(cols, c))
    assert_gemm_close(Y.cpu().numpy()[r, c], Yr, S)


@pytest.mark.parametrize("T,K,D", [(250, 512, 32700)])
def test_nvfp4_tile_width_256_sampled(T, K, D):
    # on 256 CUs: 256 tiles of 256 columns fill one round while 292 tiles of
    # 224 would take two, so the 256-wide tile runs (ragged rows and columns);
    # the small shapes above all take the 224-wide tile
    case = synth.random_case(T + K + D + 7, T, K, D, fmt="nvfp4", spec=synth.QWEN_OUTLIERS)
    act, w, Y = run_case(case)
    ref = oracle_prepare(case)
    compare_act(act, ref)
    r, c = sample_pairs(case.T, case.D, 2000, seed=3)
    cols = np.unique(c)
    Wf = case.w_f32()
    wsub = O.pack_weight(np.ascontiguousarray(Wf[:, cols]), "nvfp4", tensor_amax=np.abs(Wf).max())
    compare_weight_cols(w, wsub, cols)
    Yr, S = O.sharq_linear_sampled(ref, wsub, r, np.searchsorted(cols, c))
    assert_gemm_close(Y.cpu().numpy()[r, c], Yr, S)


def compare_weight_cols(w, ref, cols):
    torch.cuda.synchronize()
    idx = torch.from_numpy(cols).cuda()
    for k in ("payload", "scale_sp", "scale_dn"):
        got = getattr(w, k)[0].index_select(0, idx).cpu().numpy()
        assert np.array_equal(got, ref[k]), k


# ------------------------------------------------------------------ grouped (MoE)
def test_grouped_small():
    rng = np.random.default_rng(8)
    E, T, K, D = 8, 64, 256, 160
    go, ri = synth.draw_routing(rng, T, E, 2)
    case = synth.random_case(8, T, K, 1)
    W = synth.f32_to_bf16_bits(rng.standard_normal((E, K, D)).astype(np.float32) * 0.02)
    act = ops.prepare(dev_x(case), dev_gamma(case.gamma), 1e-6)
    w = ops.pack_weight(dev_w(W, "bf16"))
    Y = ops.linear(act, w, group_offsets=torch.from_numpy(go).cuda(), row_index=torch.from_numpy(ri).cuda())
    ref = oracle_prepare(case)
    wps = [O.pack_weight(synth.bf16_bits_to_f32(W[e])) for e in range(E)]
    Yr, S = O.grouped_linear(ref, wps, go, ri)
    assert_gemm_close(Y.cpu().numpy(), Yr, S)


@pytest.mark.parametrize("K", [1024, 768])
@pytest.mark.parametrize("gather", [False, True])
def test_grouped_eight_wave_tile(gather, K):
    # the eight-wave grouped tile: experts of 0, 300 (two row tiles, the
    # second ragged), 17, 0 and 520 rows, a ragged column tile (D = 300),
    # expert-sorted rows or rows gathered from 400 activations; K = 768 ends
    # on a partial group of four steps
    rng = np.random.default_rng(21)
    E, D = 5, 300
    go = np.concatenate([[0], np.cumsum([0, 300, 17, 0, 520])]).astype(np.int32)
    R = int(go[-1])
    T = 400 if gather else R
    ri = rng.integers(0, T, R).astype(np.int32) if gather else None
    case = synth.random_case(21, T, K, 1)
    W = synth.f32_to_bf16_bits(rng.standard_normal((E, K, D)).astype(np.float32) * 0.02)
    act = ops.prepare(dev_x(case), dev_gamma(case.gamma), 1e-6)
    w = ops.pack_weight(dev_w(W, "bf16"))
    Y = ops.linear(act, w, group_offsets=torch.from_numpy(go).cuda(),
                   row_index=None if ri is None else torch.from_numpy(ri).cuda(), total_rows=R)
    ref = oracle_prepare(case)
    wps = [O.pack_weight(synth.bf16_bits_to_f32(W[e])) for e in range(E)]
    Yr, S = O.grouped_linear(ref, wps, go, ri)
    assert_gemm_close(Y.cpu().numpy(), Yr, S)


@pytest.mark.parametrize("K", [128, 640, 1024])
@pytest.mark.parametrize("gather", [False, True])
def test_grouped_persistent_many_tiles(gather, K):
    # 800 grouped tiles of 128 x 256, more than the persistent grid's
    # workgroups (two per CU), so workgroups run several tiles back to back:
    # experts of 0 to 6000 rows (empty ones first, in the middle and last),
    # one step per tile (K = 128), a partial last group of four steps
    # (K = 640) and two whole groups (K = 1024), rows expert-sorted or
    # gathered from 3000 activations
    rng = np.random.default_rng(K + 7 * gather)
    sizes = [0, 4000, 37, 0, 6000, 2900, 4500, 255, 1, 2300, 0]
    E, D = len(sizes), 1280
    go = np.concatenate([[0], np.cumsum(sizes)]).astype(np.int32)
    R = int(go[-1])
    T = 3000 if gather else R
    ri = rng.integers(0, T, R).astype(np.int32) if gather else None
    case = synth.random_case(40 + K, T, K, 1)
    W = synth.f32_to_bf16_bits(rng.standard_normal((E, K, D)).astype(np.float32) * 0.02)
    act = ops.prepare(dev_x(case), dev_gamma(case.gamma), 1e-6)
    w = ops.pack_weight(dev_w(W, "bf16"))
    Y = ops.linear(act, w, group_offsets=torch.from_numpy(go).cuda(),
                   row_index=None if ri is None else torch.from_numpy(ri).cuda(), total_rows=R)
    ref = oracle_prepare(case)
    wps = [O.pack_weight(synth.bf16_bits_to_f32(W[e])) for e in range(E)]
    Yr, S = O.grouped_linear(ref, wps, go, ri)
    assert_gemm_close(Y.cpu().numpy(), Yr, S)


def test_grouped_fewer_workgroups_than_xcds():
    # two experts of 100 and 30 rows, one column tile: a grid of 3
    # workgroups (the tile order is cut into 3 stretches, not 8)
    rng = np.random.default_rng(3)
    E, K, D = 2, 256, 96
    go = np.array([0, 100, 130], dtype=np.int32)
    case = synth.random_case(3, 130, K, 1)
    W = synth.f32_to_bf16_bits(rng.standard_normal((E, K, D)).astype(np.float32) * 0.02)
    act = ops.prepare(dev_x(case), dev_gamma(case.gamma), 1e-6)
    w = ops.pack_weight(dev_w(W, "bf16"))
    Y = ops.linear(act, w, group_offsets=torch.from_numpy(go).cuda())
    ref = oracle_prepare(case)
    wps = [O.pack_weight(synth.bf16_bits_to_f32(W[e])) for e in range(E)]
    Yr, S = O.grouped_linear(ref, wps, go, None)
    assert_gemm_close(Y.cpu().numpy(), Yr, S)


def test_grouped_more_than_256_experts():
    # 300 experts: the 256-row tile that locates its expert by a workgroup
    # prefix sum (the persistent tile's expert table holds 256)
    rng = np.random.default_rng(300)
    E, T, K, D = 300, 200, 256, 96
    go, ri = synth.draw_routing(rng, T, E, 3)
    case = synth.random_case(300, T, K, 1)
    W = synth.f32_to_bf16_bits(rng.standard_normal((E, K, D)).astype(np.float32) * 0.02)
    act = ops.prepare(dev_x(case), dev_gamma(case.gamma), 1e-6)
    w = ops.pack_weight(dev_w(W, "bf16"))
    Y = ops.linear(act, w, group_offsets=torch.from_numpy(go).cuda(), row_index=torch.from_numpy(ri).cuda())
    ref = oracle_prepare(case)
    wps = [O.pack_weight(synth.bf16_bits_to_f32(W[e])) for e in range(E)]
    Yr, S = O.grouped_linear(ref, wps, go, ri)
    assert_gemm_close(Y.cpu().numpy(), Yr, S)


@pytest.mark.parametrize("proj", ["up", "down"])
def test_grouped_moe_full_sampled(proj):
    mc = synth.moe_case(proj)
    X = torch.from_numpy(mc.x.view(np.int16)).view(torch.bfloat16).cuda()
    act = ops.prepare(X, dev_gamma(mc.gamma), 1e-6)
    w = ops.pack_weight(torch.from_numpy(mc.w.view(np.int16)).view(torch.bfloat16).cuda())
    go = torch.from_numpy(mc.group_offsets).cuda()
    ri = None if mc.row_index is None else torch.from_numpy(mc.row_index).cuda()
    Y = ops.linear(act, w, group_offsets=go, row_index=ri, total_rows=mc.total_rows)
    torch.cuda.synchronize()
    xa = mc.x_f32()
    ref = O.prepare(xa, mc.gamma, 1e-6)
    compare_act(act, ref)
    # sample outputs in a handful of experts; pack only those experts in the oracle
    rng = np.random.default_rng(5)
    experts = rng.choice(mc.n_experts, 6, replace=False)
    Yg = Y.cpu().numpy()
    for e in experts:
        a, b = int(mc.group_offsets[e]), int(mc.group_offsets[e + 1])
        wref = O.pack_weight(synth.bf16_bits_to_f32(mc.w[e]))
        compare_weight(w, wref, group=int(e))
        r = rng.integers(a, b, 200)
        c = rng.integers(0, mc.D, 200)
        rows = None if mc.row_index is None else mc.row_index
        Yr, S = O.sharq_linear_sampled(ref, wref, r, c, rows=rows)
        assert_gemm_close(Yg[r, c], Yr, S)


# ------------------------------------------------------------------ HIP graph replay
def test_graph_replay_matches_eager():
    # prepare + dual GEMM captured once, replayed several times with eager work
    # and synchronizations in between; every replay must equal the eager result
    case = synth.random_case(77, 8, 1024, 320)
    X, g = dev_x(case), dev_gamma(case.gamma)
    w = ops.pack_weight(dev_w(case.w, "bf16"))
    act = ops.empty_act("mxfp4", 8, 1024)
    Y = torch.empty((8, 320), dtype=torch.float32, device="cuda")
    ops.prepare(X, g, 1e-6, out=act)
    ops.linear(act, w, out=Y)
    torch.cuda.synchronize()
    Y_eager = Y.clone()
    codes_eager = act.res_codes.clone()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        ops.prepare(X, g, 1e-6, out=act)
        ops.linear(act, w, out=Y)
    for _ in range(4):
        Y.zero_()
        act.res_codes.zero_()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(Y, Y_eager)
        assert torch.equal(act.res_codes, codes_eager)
        ops.linear(act, w)             # eager work between replays
        torch.cuda.synchronize()


# ------------------------------------------------------------------ single-launch decode
FUSED_SHAPES = [  # (T, K, D, dtype, gamma): one launch for T <= 8, K <= 16384 and for
    # T <= 16, K <= 7168 (every decode kernel geometry: 1..16 K-splits, 1..8
    # column groups, J = 4 and 8), else the two launches
    (1, 256, 64, "bf16", True), (8, 512, 200, "bf16", True), (5, 1152, 72, "bf16", True),
    (3, 384, 40, "f32", True), (8, 2048, 96, "bf16", False), (7, 16384, 48, "bf16", True),
    (2, 14336, 130, "f32", True), (6, 768, 8200, "bf16", True), (8, 4096, 4100, "bf16", True),
    (2, 256, 40000, "bf16", True),
    (4, 16512, 64, "bf16", True),
    # 9-16 rows: two MFMA tiles per step in one launch up to K = 7168
    (9, 512, 96, "bf16", True), (16, 4096, 4100, "bf16", True), (12, 1152, 200, "f32", True),
    (16, 7168, 130, "bf16", False), (13, 256, 40000, "bf16", True),
    # 9-16 rows beyond K = 7168: the two launches
    (16, 7296, 64, "bf16", True),
]


@pytest.mark.parametrize("T,K,D,dtype,gamma", FUSED_SHAPES)
def test_prepare_linear_shapes(T, K, D, dtype, gamma):
    case = synth.random_case(T * 11 + K + D, T, K, D, dtype=dtype, gamma=gamma)
    X, g = dev_x(case), dev_gamma(case.gamma)
    w = ops.pack_weight(dev_w(case.w, dtype))
    act, Y = ops.prepare_linear(X, g, w)
    ref = oracle_prepare(case)
    compare_act(act, ref)
    Yr, S = O.sharq_linear(ref, O.pack_weight(case.w_f32()))
    assert_gemm_close(Y.cpu().numpy(), Yr, S)
    # the same bytes and values as the two separate calls, and again on a
    # second call (the workspace counters are back at zero)
    act2 = ops.prepare(X, g, 1e-6)
    Y2 = ops.linear(act2, w)
    act3, Y3 = ops.prepare_linear(X, g, w)
    torch.cuda.synchronize()
    for k in ("bb_codes", "bb_meta", "bb_scale", "res_codes", "res_scale"):
        assert torch.equal(getattr(act, k), getattr(act2, k)), k
        assert torch.equal(getattr(act3, k), getattr(act2, k)), k
    assert torch.equal(Y, Y2) and torch.equal(Y3, Y2)
    # workspace words: rows done (running), workgroups past the wait (0
    # between calls), base (= rows done once every call has finished), sticky error
    words = ops._prepare_linear_ws(X.device).view(torch.int32).cpu().tolist()
    assert words[1] == 0 and words[3] == 0 and words[0] == words[2]


@pytest.mark.parametrize("i", range(3), ids=DECODE_IDS)
def test_prepare_linear_decode_full_sampled(i):
    case = synth.decode_case(i)
    X, g = dev_x(case), dev_gamma(case.gamma)
    w = ops.pack_weight(dev_w(case.w, case.dtype))
    act, Y = ops.prepare_linear(X, g, w)
    ref = oracle_prepare(case)
    compare_act(act, ref)
    r, c = sample_pairs(case.T, case.D, 3000, seed=case.K + 1)
    Yr, S = O.sharq_linear_sampled(ref, O.pack_weight(case.w_f32()), r, c)
    assert_gemm_close(Y.cpu().numpy()[r, c], Yr, S)
    Y2 = ops.linear(ops.prepare(X, g, 1e-6), w)
    torch.cuda.synchronize()
    assert torch.equal(Y, Y2)


def test_prepare_linear_sequence_and_own_workspace():
    # calls of different shapes back to back on one workspace, then on a
    # caller-owned one; every output equals the two-launch result
    ws = torch.zeros(64, dtype=torch.uint8, device="cuda")
    outs = []
    for seed, (T, K, D) in enumerate([(8, 1024, 320), (1, 256, 64), (4, 2048, 1000), (8, 1024, 320)]):
        case = synth.random_case(500 + seed, T, K, D)
        X, g = dev_x(case), dev_gamma(case.gamma)
        w = ops.pack_weight(dev_w(case.w, case.dtype))
        for workspace in (None, ws):
            act, Y = ops.prepare_linear(X, g, w, workspace=workspace)
            outs.append((Y, ops.linear(ops.prepare(X, g, 1e-6), w)))
    torch.cuda.synchronize()
    for Y, Y2 in outs:
        assert torch.equal(Y, Y2)
    words = ws.view(torch.int32).cpu().tolist()
    assert words[1] == 0 and words[3] == 0 and words[0] == words[2] == 8 + 1 + 4 + 8
    # 16 rows (two MFMA tiles) on the same workspace: the base advances by 16
    case = synth.random_case(599, 16, 1024, 320)
    X, g = dev_x(case), dev_gamma(case.gamma)
    w = ops.pack_weight(dev_w(case.w, case.dtype))
    _, Y = ops.prepare_linear(X, g, w, workspace=ws)
    Y2 = ops.linear(ops.prepare(X, g, 1e-6), w)
    torch.cuda.synchronize()
    assert torch.equal(Y, Y2)
    words = ws.view(torch.int32).cpu().tolist()
    assert words[1] == 0 and words[3] == 0 and words[0] == words[2] == 21 + 16
    ops.prepare_linear_status(ws)


def test_prepare_linear_wait_give_up_is_loud():
    # a workspace whose base lies far ahead of its running count: the wait can
    # never be satisfied, so every GEMM workgroup gives up after its bounded
    # polling (the kernel ends normally), sets the sticky error word and writes
    # NaN into Y; later calls on that workspace keep writing NaN; a cleared
    # workspace works again
    T, K, D = 4, 512, 96
    case = synth.random_case(808, T, K, D)
    X, g = dev_x(case), dev_gamma(case.gamma)
    w = ops.pack_weight(dev_w(case.w, case.dtype))
    ws = torch.zeros(4, dtype=torch.int32, device="cuda")
    ws[2] = 0x40000000
    wsb = ws.view(torch.uint8)
    act, Y = ops.prepare_linear(X, g, w, workspace=wsb)
    torch.cuda.synchronize()
    assert bool(torch.isnan(Y).all())
    compare_act(act, oracle_prepare(case))          # the producers still wrote their rows
    from sparsity_sharq_prepare_amd import _lib
    with pytest.raises(_lib.SharqError) as ei:
        ops.prepare_linear_status(wsb)
    assert ei.value.status == _lib.SHARQ_ERR_HIP
    _, Y2 = ops.prepare_linear(X, g, w, workspace=wsb)   # sticky: NaN again, no wait
    torch.cuda.synchronize()
    assert bool(torch.isnan(Y2).all())
    ws.zero_()
    _, Y3 = ops.prepare_linear(X, g, w, workspace=wsb)
    Yref = ops.linear(ops.prepare(X, g, 1e-6), w)
    torch.cuda.synchronize()
    assert torch.equal(Y3, Yref)
    ops.prepare_linear_status(wsb)


def test_prepare_linear_graph_replay():
    case = synth.random_case(91, 8, 2048, 700)
    X, g = dev_x(case), dev_gamma(case.gamma)
    w = ops.pack_weight(dev_w(case.w, case.dtype))
    act = ops.empty_act("mxfp4", 8, 2048)
    Y = torch.empty((8, 700), dtype=torch.float32, device="cuda")
    ops.prepare_linear(X, g, w, act=act, out=Y)
    torch.cuda.synchronize()
    Y_eager, codes_eager = Y.clone(), act.bb_codes.clone()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        ops.prepare_linear(X, g, w, act=act, out=Y)
    for _ in range(4):
        Y.zero_()
        act.bb_codes.zero_()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(Y, Y_eager)
        assert torch.equal(act.bb_codes, codes_eager)
        ops.prepare_linear(X, g, w)     # eager work between replays
        torch.cuda.synchronize()


def test_prepare_linear_same_buffers_new_data():
    # consecutive calls write different activations into the same buffers
    # (36-byte scale rows: neighbouring rows share cache lines); every call
    # must see its own producers' bytes, never a cached copy of the last call's
    T, K, D = 7, 1152, 600
    cases = [synth.random_case(700 + i, T, K, D) for i in range(3)]
    w = ops.pack_weight(dev_w(cases[0].w, cases[0].dtype))
    refs = []
    for c in cases:
        X, g = dev_x(c), dev_gamma(c.gamma)
        a2 = ops.prepare(X, g, 1e-6)
        refs.append((X, g, a2, ops.linear(a2, w)))
    act = ops.empty_act("mxfp4", T, K)
    Y = torch.empty((T, D), dtype=torch.float32, device="cuda")
    for _ in range(3):
        for X, g, a2, Y2 in refs:
            ops.prepare_linear(X, g, w, act=act, out=Y)
            torch.cuda.synchronize()
            assert torch.equal(Y, Y2)
            for k in ("bb_codes", "bb_meta", "bb_scale", "res_codes", "res_scale"):
                assert torch.equal(getattr(act, k), getattr(a2, k)), k


# ------------------------------------------------------------------ edge cases
def test_linear_zero_rows_and_empty_experts():
    # a gathered linear of zero rows enqueues nothing (Y keeps its contents);
    # a grouped linear whose first, a middle and the last expert have no rows
    case = synth.random_case(31, 16, 512, 96)
    act = ops.prepare(dev_x(case), dev_gamma(case.gamma), 1e-6)
    w = ops.pack_weight(dev_w(case.w, case.dtype))
    Y = torch.full((4, 96), 7.0, device="cuda")
    ops.linear(act, w, row_index=torch.zeros(0, dtype=torch.int32, device="cuda"), total_rows=0, out=Y)
    torch.cuda.synchronize()
    assert bool(torch.all(Y == 7.0))
    rng = np.random.default_rng(12)
    E, K, D = 6, 256, 130
    go = np.concatenate([[0], np.cumsum([0, 37, 0, 64, 5, 0])]).astype(np.int32)
    case2 = synth.random_case(40, int(go[-1]), K, 1)
    W = synth.f32_to_bf16_bits(rng.standard_normal((E, K, D)).astype(np.float32) * 0.02)
    act2 = ops.prepare(dev_x(case2), dev_gamma(case2.gamma), 1e-6)
    w2 = ops.pack_weight(dev_w(W, "bf16"))
    Y2 = ops.linear(act2, w2, group_offsets=torch.from_numpy(go).cuda())
    ref = oracle_prepare(case2)
    wps = [O.pack_weight(synth.bf16_bits_to_f32(W[e])) for e in range(E)]
    Yr, S = O.grouped_linear(ref, wps, go)
    assert_gemm_close(Y2.cpu().numpy(), Yr, S)


@pytest.mark.parametrize("T", [5, 40, 300])
def test_strided_input_and_output(T):
    # X rows further apart than K (a column slice of a wider buffer) and Y rows
    # further apart than D: the same bytes and values as the contiguous call,
    # and Y's padding columns untouched (decode, skinny and tile paths)
    K, D = 512, 200
    case = synth.random_case(51 + T, T, K, D)
    X, g = dev_x(case), dev_gamma(case.gamma)
    Xw = torch.zeros((T, K + 64), dtype=X.dtype, device="cuda")
    Xw[:, 64:] = X
    act_s = ops.prepare(Xw[:, 64:], g, 1e-6)
    act = ops.prepare(X, g, 1e-6)
    w = ops.pack_weight(dev_w(case.w, case.dtype))
    Yw = torch.full((T, 256), -3.0, device="cuda")
    ops.linear(act_s, w, out=Yw[:, :D])
    Y = ops.linear(act, w)
    torch.cuda.synchronize()
    for k in ("bb_codes", "bb_meta", "bb_scale", "res_codes", "res_scale"):
        assert torch.equal(getattr(act_s, k), getattr(act, k)), k
    assert torch.equal(Yw[:, :D], Y)
    assert bool(torch.all(Yw[:, D:] == -3.0))
    compare_act(act, oracle_prepare(case))


# ------------------------------------------------------------------ plain baseline (unfused pipeline)
BASE_SHAPES = [  # (T, K, dtype, gamma): the prepare geometries (64..1024 threads per row, 1..16 chunks)
    (37, 256, "bf16", True), (5, 768, "bf16", False), (3, 32, "f32", True), (300, 4096, "bf16", True),
    (4099, 2048, "bf16", True), (17, 14336, "bf16", True), (2100, 4096, "f32", True), (9, 18944, "bf16", True),
]


@pytest.mark.parametrize("T,K,dtype,gamma", BASE_SHAPES)
def test_plain_rmsnorm_quantize(T, K, dtype, gamma):
    case = synth.random_case(7 * T + K, T, K, 8, dtype=dtype, gamma=gamma)
    y = ops.rmsnorm(dev_x(case), dev_gamma(case.gamma), 1e-6)
    codes, scales = ops.quantize_mx(y)
    ref = O.plain_prepare_mx(case.x_f32(), case.gamma)
    torch.cuda.synchronize()
    assert_bytes_equal("y bits", y.cpu().numpy().view(np.uint32), ref["y"].view(np.uint32))
    assert_bytes_equal("codes", codes.cpu().numpy(), ref["codes"])
    assert_bytes_equal("scales", scales.cpu().numpy(), ref["scales"])


def test_plain_quantize_edge_values_and_strided_rows():
    rng = np.random.default_rng(11)
    K = 128
    y = np.zeros((6, K), np.float32)
    y[0, 1::2] = -0.0                                          # signed zeros, all-zero blocks
    y[1] = rng.standard_normal(K).astype(np.float32) * np.float32(1e-40)   # subnormal blocks
    mags = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0], np.float32)   # E2M1 ties
    y[2] = mags[rng.integers(0, 7, K)] * np.where(rng.random(K) < 0.5, -1, 1).astype(np.float32)
    y[2, 0::32] = 6.0
    y[3] = rng.standard_normal(K).astype(np.float32) * np.float32(3e37)    # near the top of fp32
    y[4] = np.float32(1.0)
    y[4, 7] = np.float32(6.0000005)                            # amax just above 6: next scale
    y[5] = rng.standard_normal(K).astype(np.float32)
    wide = torch.zeros((6, K + 36), dtype=torch.float32, device="cuda")
    wide[:, :K] = torch.from_numpy(y).cuda()
    codes, scales = ops.quantize_mx(wide[:, :K])               # ldy = K + 36
    c, e = O.mx_quantize(y)
    torch.cuda.synchronize()
    assert_bytes_equal("codes", codes.cpu().numpy(), O.pack_nibbles(c))
    from oracle import formats as F
    assert_bytes_equal("scales", scales.cpu().numpy(), F.e8m0_encode_exponent(e))


DENSE_SHAPES = [  # (T, K, D): one and many row tiles, ragged rows and columns, both tile widths
    (1, 512, 200), (70, 512, 1), (300, 1024, 520), (257, 1536, 250), (4000, 512, 3000), (512, 2048, 4096),
]


@pytest.mark.parametrize("T,K,D", DENSE_SHAPES)
def test_plain_linear_dense(T, K, D):
    case = synth.random_case(T + 5 * K + D, T, K, D)
    y = ops.rmsnorm(dev_x(case), dev_gamma(case.gamma), 1e-6)
    codes, scales = ops.quantize_mx(y)
    w = ops.pack_weight(dev_w(case.w, "bf16"))
    Y = ops.linear_dense(codes, scales, w)
    ref = O.plain_prepare_mx(case.x_f32(), case.gamma)
    Yr, S = O.plain_linear_mx(ref["codes"], ref["scales"], O.pack_weight(case.w_f32()))
    assert_gemm_close(Y.cpu().numpy(), Yr, S)


def test_plain_linear_dense_prefill_sampled():
    case = synth.prefill_case()
    y = ops.rmsnorm(dev_x(case), dev_gamma(case.gamma), 1e-6)
    codes, scales = ops.quantize_mx(y)
    w = ops.pack_weight(dev_w(case.w, "bf16"))
    Y = ops.linear_dense(codes, scales, w)
    Y2 = ops.linear_dense(codes, scales, w)
    torch.cuda.synchronize()
    assert torch.equal(Y, Y2)
    ref_c, ref_s = codes.cpu().numpy(), scales.cpu().numpy()
    r, c = sample_pairs(case.T, case.D, 2000, seed=3)
    # the codes themselves are checked against the oracle on the sampled rows
    rows = np.unique(r)
    refp = O.plain_prepare_mx(case.x_f32()[rows], case.gamma)
    assert_bytes_equal("codes", ref_c[rows], refp["codes"])
    assert_bytes_equal("scales", ref_s[rows], refp["scales"])
    cols = np.unique(c)
    wref = O.pack_weight(case.w_f32()[:, cols])
    Yr, S = O.plain_linear_mx_sampled(ref_c, ref_s, wref, r, np.searchsorted(cols, c))
    assert_gemm_close(Y.cpu().numpy()[r, c], Yr, S)


# ------------------------------------------------------------------ 2:4 element-wise backbone (MXFP4)
def oracle_prepare_24(case, eps=1e-6):
    return O.prepare(case.x_f32(), case.gamma, eps, "mxfp4", mask="2:4")


M24_PREP = [  # (T, K, dtype, gamma): the prepare geometries, ragged T, no normalization
    (37, 256, "bf16", True), (5, 768, "bf16", True), (3, 32, "f32", True), (300, 4096, "bf16", True),
    (4099, 2048, "bf16", True), (17, 14336, "bf16", True), (64, 4096, "bf16", False), (2100, 4096, "f32", True),
]


@pytest.mark.parametrize("T,K,dtype,gamma", M24_PREP)
def test_prepare_24_shapes(T, K, dtype, gamma):
    case = synth.random_case(11 * T + K, T, K, 8, dtype=dtype, gamma=gamma)
    act = ops.prepare(dev_x(case), dev_gamma(case.gamma), 1e-6, "mxfp4_24")
    compare_act(act, oracle_prepare_24(case))


def test_prepare_24_edge_rows():
    # zero row, worked-example row, signed zeros, tiny and large magnitudes,
    # exact ties inside groups of 4
    K = 64
    x = np.zeros((6, K), np.float32)
    x[1, :] = 0.2
    x[1, 5] = 12.0
    x[2, ::2] = -0.0
    x[2, 1::2] = 1e-30
    x[3, :] = np.float32(3.0e30) * np.cos(np.arange(K))
    x[4, :] = np.tile(np.array([1, -1, 1, -1, 2, 2, -2, -2], np.float32), K // 8)
    x[5, :] = np.float32(1e-38) * np.arange(K)
    case = synth.LinearCase("edge", "mxfp4", "f32", 6, K, 8, x, None, np.zeros((K, 8), np.float32))
    act = ops.prepare(dev_x(case), None, 1e-6, "mxfp4_24")
    compare_act(act, O.prepare(x, None, 1e-6, "mxfp4", mask="2:4"))
    g = np.ones(K, np.float32)
    act = ops.prepare(dev_x(case), dev_gamma(g), 1e-6, "mxfp4_24")
    compare_act(act, O.prepare(x, g, 1e-6, "mxfp4", mask="2:4"))


M24_LINEAR = [  # decode (<= 16 rows; 17-64 in chunks of launches up to K = 16384), skinny (<= 64 rows
    # beyond), eight-wave tile (> 64 rows, any K % 128), ragged
    (1, 512, 200), (8, 512, 200), (5, 1152, 72), (7, 16384, 48), (13, 256, 64), (64, 384, 130),
    (40, 2048, 300), (33, 8192, 72), (20, 16512, 40),
    (65, 512, 300), (300, 512, 520), (700, 128, 40), (256, 1024, 256), (70, 512, 1),
    (100, 384, 72), (333, 768, 250),
]


@pytest.mark.parametrize("T,K,D", M24_LINEAR)
def test_linear_24_shapes(T, K, D):
    case = synth.random_case(T + 3 * K + D + 1, T, K, D)
    act = ops.prepare(dev_x(case), dev_gamma(case.gamma), 1e-6, "mxfp4_24")
    w = ops.pack_weight(dev_w(case.w, "bf16"))
    Y = ops.linear(act, w)
    ref = oracle_prepare_24(case)
    compare_act(act, ref)
    Yr, S = O.sharq_linear(ref, O.pack_weight(case.w_f32()))
    assert_gemm_close(Y.cpu().numpy(), Yr, S)


@pytest.mark.parametrize("i", range(3), ids=DECODE_IDS)
def test_linear_24_decode_full_sampled(i):
    case = synth.decode_case(i)
    act = ops.prepare(dev_x(case), dev_gamma(case.gamma), 1e-6, "mxfp4_24")
    w = ops.pack_weight(dev_w(case.w, "bf16"))
    Y = ops.linear(act, w)
    ref = oracle_prepare_24(case)
    compare_act(act, ref)
    r, c = sample_pairs(case.T, case.D, 3000, seed=case.K + 1)
    Yr, S = O.sharq_linear_sampled(ref, O.pack_weight(case.w_f32()), r, c)
    assert_gemm_close(Y.cpu().numpy()[r, c], Yr, S)


def test_linear_24_prefill_sampled():
    case = synth.prefill_case()
    act = ops.prepare(dev_x(case), dev_gamma(case.gamma), 1e-6, "mxfp4_24")
    w = ops.pack_weight(dev_w(case.w, "bf16"))
    Y = ops.linear(act, w)
    rows = np.random.default_rng(4).choice(case.T, 48, replace=False)
    refp = O.prepare(case.x_f32()[rows], case.gamma, 1e-6, "mxfp4", mask="2:4")
    g = act.as_numpy()
    for k in ("bb_codes", "bb_meta", "bb_scale", "res_codes", "res_scale"):
        assert_bytes_equal(k, g[k][rows], refp[k])
    r, c = sample_pairs(case.T, case.D, 2000, seed=5)
    ref = oracle_prepare_24(case)
    cols = np.unique(c)
    wref = O.pack_weight(case.w_f32()[:, cols])
    Yr, S = O.sharq_linear_sampled(ref, wref, r, np.searchsorted(cols, c))
    assert_gemm_close(Y.cpu().numpy()[r, c], Yr, S)


def test_grouped_24_small():
    rng = np.random.default_rng(18)
    E, T, K, D = 8, 64, 256, 160
    go, ri = synth.draw_routing(rng, T, E, 2)
    case = synth.random_case(18, T, K, 1)
    W = synth.f32_to_bf16_bits(rng.standard_normal((E, K, D)).astype(np.float32) * 0.02)
    act = ops.prepare(dev_x(case), dev_gamma(case.gamma), 1e-6, "mxfp4_24")
    w = ops.pack_weight(dev_w(W, "bf16"))
    Y = ops.linear(act, w, group_offsets=torch.from_numpy(go).cuda(), row_index=torch.from_numpy(ri).cuda())
    ref = oracle_prepare_24(case)
    wps = [O.pack_weight(synth.bf16_bits_to_f32(W[e])) for e in range(E)]
    Yr, S = O.grouped_linear(ref, wps, go, ri)
    assert_gemm_close(Y.cpu().numpy(), Yr, S)


# ------------------------------------------------------------------ largest supported K
@pytest.mark.parametrize("fmt", ["mxfp4", "nvfp4", "mxfp4_24"])
def test_prepare_and_linear_at_max_k(fmt):
    # K = 32768: 256 threads x 16 groups of 8 per row, the prepare kernels'
    # register limit; the GEMM runs the skinny path (K beyond the decode
    # kernel's staged maximum) and the tile path
    K = 32768
    for T, D in ((3, 40), (70, 96)):
        base = "nvfp4" if fmt == "nvfp4" else "mxfp4"
        case = synth.random_case(T + D, T, K, D, fmt=base)
        act = ops.prepare(dev_x(case), dev_gamma(case.gamma), 1e-6, fmt)
        w = ops.pack_weight(dev_w(case.w, "bf16"), base)
        Y = ops.linear(act, w)
        ref = O.prepare(case.x_f32(), case.gamma, 1e-6, base, mask="2:4" if fmt == "mxfp4_24" else "4:8")
        compare_act(act, ref)
        Yr, S = O.sharq_linear(ref, O.pack_weight(case.w_f32(), base))
        assert_gemm_close(Y.cpu().numpy(), Yr, S)
