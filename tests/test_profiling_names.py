"""The profile summaries average a kernel's counters over the dispatches whose
names the selection patterns pick: the instances the bench reports on, and
not the plain baseline's dense tile or the single-launch decode form."""
from sparsity_sharq_prepare_amd.profiling import selects

SIG = "(unsigned char const*, unsigned char const*, int, float*, long)"


def test_decode_selects_the_two_launch_4_8_gemm():
    assert selects("linear_mx_decode", "void sharq::linear_mx_decode<16, 1, 8, false, false>" + SIG)
    assert selects("linear_mx_decode", "void sharq::linear_mx_decode<8, 1, 4, false, false>" + SIG)
    assert not selects("linear_mx_decode", "void sharq::linear_mx_decode<16, 1, 8, true, false>" + SIG)   # fused
    assert not selects("linear_mx_decode", "void sharq::linear_mx_decode<16, 1, 8, false, true>" + SIG)   # 2:4


def test_tile_selects_the_dual_gemm_instances_only():
    for name in ("linear_mx_tile8<8, 224, false, false, false, false>", "linear_mx_tile8<8, 256, false, true, false, true>",
                 "linear_mx_tile8<8, 224, false, false, true, false>"):
        assert selects("linear_mx_tile", "void sharq::" + name + SIG), name
    for name in ("linear_mx_tile8<8, 224, true, false, false, false>", "linear_mx_tile8<8, 256, true, false, false, false>"):
        assert not selects("linear_mx_tile", "void sharq::" + name + SIG), name
    assert not selects("linear_mx_tile", "void sharq::linear_mx_decode<16, 1, 8, false, false>" + SIG)


def test_other_kernels():
    assert selects("linear_nv_tile", "sharq::linear_nv_tile" + SIG)
    assert selects("prepare_mx_kernel", "void sharq::prepare_mx_kernel<64, 8, true, true, false>" + SIG)
    assert not selects("prepare_mx_kernel", "void sharq::prepare_nv_phase1<256, 16, true>" + SIG)
