"""The C-ABI library loads, exports every symbol include/sharq.h declares, and
rejects bad arguments on the host before touching the GPU (no compute calls:
every call here fails validation, so nothing is enqueued)."""
import ctypes
import os
import re

import pytest

from sparsity_sharq_prepare_amd import _lib as L

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

pytestmark = pytest.mark.skipif(not os.path.exists(L.LIB_PATH), reason="libsharq.so not built")


def header_functions():
    src = open(os.path.join(ROOT, "include", "sharq.h")).read()
    return sorted(set(re.findall(r"^(?:sharq_status|const char \*)\s*(sharq_\w+)\(", src, re.M)))


def test_exports_every_declared_symbol():
    names = header_functions()
    assert set(names) == set(L.EXPORTS)
    lib = L.lib()
    for n in names:
        assert hasattr(lib, n), n


def test_status_strings():
    assert L.status_name(0) == "SHARQ_OK"
    assert L.status_name(3) == "SHARQ_ERR_FORMAT_MISMATCH"


def test_sizes():
    # MXFP4 prep output = K/4 + K/16 + K/32 + K/2 + K/32 = 0.875 B per input element
    sz = L.act_sizes(L.SHARQ_MXFP4, 8, 4096)
    assert sz[:5] == [8 * 1024, 8 * 256, 8 * 128, 8 * 2048, 8 * 128] and sum(sz[:5]) == 0.875 * 8 * 4096
    assert sz[5] == 0 and sz[6] == 0
    nv = L.act_sizes(L.SHARQ_NVFP4_EMU, 8, 4096)
    assert nv[4] == 8 * 256 and nv[5] == 8 and nv[6] > 8 * 4
    w = L.weight_sizes(L.SHARQ_MXFP4, 4096, 14336, 1)
    assert w[0] == 14336 * 2048 and w[1] == w[2] == 14336 * 128 and w[3] == 0
    wn = L.weight_sizes(L.SHARQ_NVFP4_EMU, 3584, 18944, 2)
    assert wn[2] == 2 * 18944 * 224 and wn[3] == 8


@pytest.mark.parametrize("K", [0, 31, 48, -32])
def test_sizes_reject_bad_k(K):
    with pytest.raises(L.SharqError) as e:
        L.act_sizes(L.SHARQ_MXFP4, 8, K)
    assert e.value.status == L.SHARQ_ERR_UNSUPPORTED_SHAPE


def _fake_act(fmt=0, T=8, K=256, base=0x10000):
    return L.SharqAct(fmt, T, K, base, base + 0x1000, base + 0x2000, base + 0x3000, base + 0x4000,
                      base + 0x5000 if fmt else None)


def _fake_weight(fmt=0, K=256, D=64, G=1, base=0x20000):
    return L.SharqWeight(fmt, K, D, G, base, base + 0x1000, base + 0x1000 if fmt == 0 else base + 0x2000,
                         base + 0x3000 if fmt else None)


def test_linear_validation_errors():
    lib = L.lib()
    Y = 0x30000
    a, w = _fake_act(), _fake_weight()
    # format mismatch
    assert lib.sharq_linear(_fake_act(fmt=1), w, None, None, 8, Y, 64, None) == L.SHARQ_ERR_FORMAT_MISMATCH
    # K mismatch
    assert lib.sharq_linear(a, _fake_weight(K=512), None, None, 8, Y, 64, None) == L.SHARQ_ERR_FORMAT_MISMATCH
    # K not a multiple of 128 for the GEMM
    assert lib.sharq_linear(_fake_act(K=96), _fake_weight(K=96), None, None, 8, Y, 64, None) == \
        L.SHARQ_ERR_UNSUPPORTED_SHAPE
    # ldy < D, NULL Y, misaligned Y
    assert lib.sharq_linear(a, w, None, None, 8, Y, 32, None) == L.SHARQ_ERR_INVALID_ARGUMENT
    assert lib.sharq_linear(a, w, None, None, 8, None, 64, None) == L.SHARQ_ERR_INVALID_ARGUMENT
    assert lib.sharq_linear(a, w, None, None, 8, Y + 4, 64, None) == L.SHARQ_ERR_INVALID_ARGUMENT
    # more rows than T without a gather
    assert lib.sharq_linear(a, w, None, None, 9, Y, 64, None) == L.SHARQ_ERR_INVALID_ARGUMENT
    # grouped needs offsets; NVFP4 grouped is unsupported
    assert lib.sharq_linear(a, _fake_weight(G=4), None, None, 8, Y, 64, None) == L.SHARQ_ERR_INVALID_ARGUMENT
    assert lib.sharq_linear(_fake_act(fmt=1), _fake_weight(fmt=1, G=4), 0x40000, None, 8, Y, 64, None) == \
        L.SHARQ_ERR_UNSUPPORTED_SHAPE
    # buffers past the 32-bit buffer-descriptor range
    big_t = (1 << 33) // 4096
    assert lib.sharq_linear(_fake_act(T=big_t, K=4096), _fake_weight(K=4096), None, None, 8, Y, 64, None) == \
        L.SHARQ_ERR_UNSUPPORTED_SHAPE
    assert lib.sharq_linear(_fake_act(K=4096), _fake_weight(K=4096, D=big_t), None, None, 8, Y, big_t, None) == \
        L.SHARQ_ERR_UNSUPPORTED_SHAPE
    assert "bytes" in lib.sharq_last_error().decode()
    # ... and past 2 GiB: offsets with bit 31 set mark absent loads, so no
    # buffer may reach that far
    t2 = (1 << 32) // 4096                                 # T * K / 2 = 2 GiB
    assert lib.sharq_linear(_fake_act(T=t2, K=4096), _fake_weight(K=4096), None, None, 8, Y, 64, None) == \
        L.SHARQ_ERR_UNSUPPORTED_SHAPE
    # null activation buffer
    bad = _fake_act()
    bad.res_codes = None
    assert lib.sharq_linear(bad, w, None, None, 8, Y, 64, None) == L.SHARQ_ERR_INVALID_ARGUMENT
    assert "NULL" in lib.sharq_last_error().decode()


def test_prepare_validation_errors():
    lib = L.lib()
    X = 0x50000
    out = _fake_act()
    assert lib.sharq_prepare(None, 1, 8, 256, 256, None, 1e-6, out, None, 0, None) == L.SHARQ_ERR_INVALID_ARGUMENT
    assert lib.sharq_prepare(X, 7, 8, 256, 256, None, 1e-6, out, None, 0, None) == L.SHARQ_ERR_INVALID_ARGUMENT
    assert lib.sharq_prepare(X, 1, 8, 250, 256, None, 1e-6, _fake_act(K=250), None, 0, None) == \
        L.SHARQ_ERR_UNSUPPORTED_SHAPE
    # struct / call disagree
    assert lib.sharq_prepare(X, 1, 9, 256, 256, None, 1e-6, out, None, 0, None) == L.SHARQ_ERR_INVALID_ARGUMENT
    # ldx < K, unaligned rows, unaligned gamma, negative eps
    assert lib.sharq_prepare(X, 1, 8, 256, 128, None, 1e-6, out, None, 0, None) == L.SHARQ_ERR_INVALID_ARGUMENT
    assert lib.sharq_prepare(X, 1, 8, 256, 260, None, 1e-6, out, None, 0, None) == L.SHARQ_ERR_INVALID_ARGUMENT
    assert lib.sharq_prepare(X, 1, 8, 256, 256, 0x60004, 1e-6, out, None, 0, None) == L.SHARQ_ERR_INVALID_ARGUMENT
    assert lib.sharq_prepare(X, 1, 8, 256, 256, None, -1.0, out, None, 0, None) == L.SHARQ_ERR_INVALID_ARGUMENT
    # K beyond the register-resident maximum
    big = _fake_act(K=65536)
    assert lib.sharq_prepare(X, 1, 8, 65536, 65536, None, 1e-6, big, None, 0, None) == L.SHARQ_ERR_UNSUPPORTED_SHAPE
    # NVFP4 needs a workspace
    nv = _fake_act(fmt=1)
    assert lib.sharq_prepare(X, 1, 8, 256, 256, None, 1e-6, nv, None, 0, None) == L.SHARQ_ERR_WORKSPACE_TOO_SMALL


def test_pack_validation_errors():
    lib = L.lib()
    W = 0x70000
    w = _fake_weight()
    assert lib.sharq_pack_weight(None, 1, 256, 64, 1, 64, 0, w, None, 0, None) == L.SHARQ_ERR_INVALID_ARGUMENT
    assert lib.sharq_pack_weight(W, 1, 256, 64, 1, 32, 0, w, None, 0, None) == L.SHARQ_ERR_INVALID_ARGUMENT
    assert lib.sharq_pack_weight(W, 1, 512, 64, 1, 64, 0, w, None, 0, None) == L.SHARQ_ERR_INVALID_ARGUMENT
    assert lib.sharq_pack_weight(W, 1, 100, 64, 1, 64, 0, _fake_weight(K=100), None, 0, None) == \
        L.SHARQ_ERR_UNSUPPORTED_SHAPE
    g = _fake_weight(G=2)
    assert lib.sharq_pack_weight(W, 1, 256, 64, 2, 64, 100, g, None, 0, None) == L.SHARQ_ERR_INVALID_ARGUMENT
    nv = _fake_weight(fmt=1)
    assert lib.sharq_pack_weight(W, 1, 256, 64, 1, 64, 0, nv, None, 0, None) == L.SHARQ_ERR_WORKSPACE_TOO_SMALL
    nv_alias = _fake_weight(fmt=1)
    nv_alias.scale_dn = nv_alias.scale_sp
    assert lib.sharq_pack_weight(W, 1, 256, 64, 1, 64, 0, nv_alias, 0x80000, 1 << 20, None) == \
        L.SHARQ_ERR_INVALID_ARGUMENT


def test_prepare_linear_validation_errors():
    lib = L.lib()
    f = lib.sharq_prepare_linear
    X, Y, ws = 0x50000, 0x30000, 0x90000
    a, w = _fake_act(), _fake_weight()
    # NVFP4 preparation needs tensor-wide reductions first: not offered here
    assert f(X, 1, 8, 256, 256, None, 1e-6, _fake_act(fmt=1), _fake_weight(fmt=1), Y, 64, ws, 16, None) == \
        L.SHARQ_ERR_INVALID_ARGUMENT
    assert "MXFP4" in lib.sharq_last_error().decode()
    # plain linear only
    assert f(X, 1, 8, 256, 256, None, 1e-6, a, _fake_weight(G=2), Y, 64, ws, 16, None) == L.SHARQ_ERR_INVALID_ARGUMENT
    # workspace missing, too small, misaligned
    assert f(X, 1, 8, 256, 256, None, 1e-6, a, w, Y, 64, None, 0, None) == L.SHARQ_ERR_WORKSPACE_TOO_SMALL
    assert f(X, 1, 8, 256, 256, None, 1e-6, a, w, Y, 64, ws, 4, None) == L.SHARQ_ERR_WORKSPACE_TOO_SMALL
    assert f(X, 1, 8, 256, 256, None, 1e-6, a, w, Y, 64, ws, 8, None) == L.SHARQ_ERR_WORKSPACE_TOO_SMALL
    # the status query checks its workspace argument before any copy
    assert lib.sharq_prepare_linear_status(None, 16, None) == L.SHARQ_ERR_WORKSPACE_TOO_SMALL
    assert lib.sharq_prepare_linear_status(ws, 8, None) == L.SHARQ_ERR_WORKSPACE_TOO_SMALL
    assert lib.sharq_prepare_linear_status(ws + 4, 16, None) == L.SHARQ_ERR_INVALID_ARGUMENT
    assert f(X, 1, 8, 256, 256, None, 1e-6, a, w, Y, 64, ws + 4, 16, None) == L.SHARQ_ERR_INVALID_ARGUMENT
    # activation / weight K differ; act describes other rows; K % 128 != 0
    assert f(X, 1, 8, 256, 256, None, 1e-6, a, _fake_weight(K=512), Y, 64, ws, 16, None) == \
        L.SHARQ_ERR_FORMAT_MISMATCH
    assert f(X, 1, 4, 256, 256, None, 1e-6, a, w, Y, 64, ws, 16, None) == L.SHARQ_ERR_INVALID_ARGUMENT
    assert f(X, 1, 8, 96, 96, None, 1e-6, _fake_act(K=96), _fake_weight(K=96), Y, 64, ws, 16, None) == \
        L.SHARQ_ERR_UNSUPPORTED_SHAPE
    # prepare-side checks: unknown dtype, ldx < K; linear-side: ldy < D
    assert f(X, 7, 8, 256, 256, None, 1e-6, a, w, Y, 64, ws, 16, None) == L.SHARQ_ERR_INVALID_ARGUMENT
    assert f(X, 1, 8, 256, 128, None, 1e-6, a, w, Y, 64, ws, 16, None) == L.SHARQ_ERR_INVALID_ARGUMENT
    assert f(X, 1, 8, 256, 256, None, 1e-6, a, w, Y, 32, ws, 16, None) == L.SHARQ_ERR_INVALID_ARGUMENT


def test_prepare_no_alloc_validation_errors():
    # the allocation-free prepare: the usual prepare checks, and NVFP4 shapes
    # whose scratch exceeds the static 1 MiB rejected before any device work
    lib = L.lib()
    f = lib.sharq_prepare_no_alloc
    X = 0x50000
    assert f(X, 1, 8, 256, 256, None, ctypes.c_float(1e-6), None, None) == L.SHARQ_ERR_INVALID_ARGUMENT
    assert f(X, 7, 8, 256, 256, None, ctypes.c_float(1e-6), _fake_act(), None) == L.SHARQ_ERR_INVALID_ARGUMENT
    assert f(X, 1, 100000, 2048, 2048, None, ctypes.c_float(1e-6), _fake_act(fmt=1, T=100000, K=2048), None) == \
        L.SHARQ_ERR_UNSUPPORTED_SHAPE
    assert "scratch" in lib.sharq_last_error().decode()


def test_plain_baseline_validation_errors():
    lib = L.lib()
    X, Y, c, s = 0x50000, 0x30000, 0x60000, 0x70000
    # rmsnorm: unknown dtype, K % 32, ldy < K, misaligned Y rows, NULL
    assert lib.sharq_rmsnorm(X, 7, 8, 256, 256, None, 1e-6, Y, 256, None) == L.SHARQ_ERR_INVALID_ARGUMENT
    assert lib.sharq_rmsnorm(X, 1, 8, 48, 48, None, 1e-6, Y, 48, None) == L.SHARQ_ERR_UNSUPPORTED_SHAPE
    assert lib.sharq_rmsnorm(X, 1, 8, 256, 256, None, 1e-6, Y, 128, None) == L.SHARQ_ERR_INVALID_ARGUMENT
    assert lib.sharq_rmsnorm(X, 1, 8, 256, 256, None, 1e-6, Y, 258, None) == L.SHARQ_ERR_INVALID_ARGUMENT
    assert lib.sharq_rmsnorm(None, 1, 8, 256, 256, None, 1e-6, Y, 256, None) == L.SHARQ_ERR_INVALID_ARGUMENT
    assert lib.sharq_rmsnorm(X, 1, 0, 256, 256, None, 1e-6, Y, 256, None) == L.SHARQ_ERR_UNSUPPORTED_SHAPE
    # quantize: K % 32, ldy < K, misaligned outputs
    assert lib.sharq_quantize_mx(Y, 8, 48, 48, c, s, None) == L.SHARQ_ERR_UNSUPPORTED_SHAPE
    assert lib.sharq_quantize_mx(Y, 8, 256, 128, c, s, None) == L.SHARQ_ERR_INVALID_ARGUMENT
    assert lib.sharq_quantize_mx(Y, 8, 256, 256, c + 8, s, None) == L.SHARQ_ERR_INVALID_ARGUMENT
    assert lib.sharq_quantize_mx(Y, 8, 256, 256, None, s, None) == L.SHARQ_ERR_INVALID_ARGUMENT
    # dense GEMM: K % 512, NVFP4 weight, grouped weight, ldy < D
    f = lib.sharq_linear_dense
    assert f(c, s, 8, _fake_weight(K=256), Y, 64, None) == L.SHARQ_ERR_UNSUPPORTED_SHAPE
    assert "512" in lib.sharq_last_error().decode()
    assert f(c, s, 8, _fake_weight(fmt=1, K=512), Y, 64, None) == L.SHARQ_ERR_FORMAT_MISMATCH
    assert f(c, s, 8, _fake_weight(K=512, G=2), Y, 64, None) == L.SHARQ_ERR_INVALID_ARGUMENT
    assert f(c, s, 8, _fake_weight(K=512), Y, 32, None) == L.SHARQ_ERR_INVALID_ARGUMENT
    assert f(c, s, 0, _fake_weight(K=512), Y, 64, None) == L.SHARQ_ERR_UNSUPPORTED_SHAPE
    assert f(None, s, 8, _fake_weight(K=512), Y, 64, None) == L.SHARQ_ERR_INVALID_ARGUMENT


def test_mxfp4_24_format_rules():
    lib = L.lib()
    sz = (ctypes.c_size_t * 7)()
    assert lib.sharq_act_sizes(L.SHARQ_MXFP4_24, 8, 256, sz) == L.SHARQ_OK
    assert list(sz) == [8 * 64, 8 * 32, 8 * 8, 8 * 128, 8 * 8, 0, 0]       # metadata K/8 per row
    w5 = (ctypes.c_size_t * 5)()
    assert lib.sharq_weight_sizes(L.SHARQ_MXFP4_24, 256, 64, 1, w5) == L.SHARQ_ERR_INVALID_ARGUMENT
    Y = 0x30000
    a24 = _fake_act(fmt=L.SHARQ_MXFP4_24)
    # 2:4 activations multiply MXFP4 weights, not NVFP4 ones
    assert lib.sharq_linear(a24, _fake_weight(fmt=1), None, None, 8, Y, 64, None) == L.SHARQ_ERR_FORMAT_MISMATCH
    # the single-launch decode offers the 4:8 backbone only
    assert lib.sharq_prepare_linear(0x50000, 1, 8, 256, 256, None, 1e-6, a24, _fake_weight(), Y, 64, 0x90000, 16,
                                    None) == L.SHARQ_ERR_INVALID_ARGUMENT


def test_prepare_k_limit():
    lib = L.lib()
    K = 32768 + 128
    a = _fake_act(K=K)
    assert lib.sharq_prepare(0x50000, 1, 8, K, K, None, 1e-6, a, None, 0, None) == L.SHARQ_ERR_UNSUPPORTED_SHAPE
    assert "maximum" in lib.sharq_last_error().decode()
    assert lib.sharq_rmsnorm(0x50000, 1, 8, K, K, None, 1e-6, 0x30000, K, None) == L.SHARQ_ERR_UNSUPPORTED_SHAPE


def test_timeline_entry_points_of_the_normal_build():
    # the tile-timeline entry points exist in every build; outside the
    # SHARQ_TIMELINE build they report no records and refuse clear / read
    # (host-side answers: nothing touches the GPU)
    lib = L.lib()
    n = ctypes.c_size_t(7)
    assert lib.sharq_timeline_records(ctypes.byref(n)) == L.SHARQ_OK
    assert n.value == 0
    assert lib.sharq_timeline_records(None) == L.SHARQ_ERR_INVALID_ARGUMENT
    assert lib.sharq_timeline_clear() == L.SHARQ_ERR_INVALID_ARGUMENT
    assert "timeline" in lib.sharq_last_error().decode()
    buf = (ctypes.c_uint64 * 8)()
    assert lib.sharq_timeline_read(buf, 8) == L.SHARQ_ERR_INVALID_ARGUMENT
