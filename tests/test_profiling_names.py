"""The profile summaries average a kernel's counters over the dispatches whose
names the selection patterns pick: the instances the bench reports on, and
not the plain baseline's dense tile, the single-launch decode form, the 2:4
backbone or the two-tile (9-16 row) decode kernel."""
from sparsity_sharq_prepare_amd.profiling import selects

SIG = "(unsigned char const*, unsigned char const*, int, float*, long)"


def test_decode_selects_the_two_launch_4_8_one_tile_gemm():
    assert selects("linear_mx_decode", "void sharq::linear_mx_decode<16, 1, 8, false, false, 1>" + SIG)
    assert selects("linear_mx_decode", "void sharq::linear_mx_decode<8, 1, 4, false, false, 1>" + SIG)
    assert not selects("linear_mx_decode", "void sharq::linear_mx_decode<16, 1, 8, true, false, 1>" + SIG)   # fused
    assert not selects("linear_mx_decode", "void sharq::linear_mx_decode<16, 1, 8, false, true, 1>" + SIG)   # 2:4
    assert not selects("linear_mx_decode", "void sharq::linear_mx_decode<4, 2, 8, false, false, 2>" + SIG)   # 16 rows


def test_tile_selects_the_dual_gemm_instances_only():
    for name in ("linear_mx_tile8<256, 224, false, false, false, false>",
                 "linear_mx_tile8<128, 256, false, true, false, true>",
                 "linear_mx_tile8<256, 224, false, false, true, false>"):
        assert selects("linear_mx_tile", "void sharq::" + name + SIG), name
    for name in ("linear_mx_tile8<256, 224, true, false, false, false>",
                 "linear_mx_tile8<256, 256, true, false, false, false>"):
        assert not selects("linear_mx_tile", "void sharq::" + name + SIG), name
    assert not selects("linear_mx_tile", "void sharq::linear_mx_decode<16, 1, 8, false, false, 1>" + SIG)


def test_other_kernels():
    assert selects("linear_nv_tile", "sharq::linear_nv_tile" + SIG)
    assert selects("prepare_mx_kernel", "void sharq::prepare_mx_kernel<64, 8, true, true, false>" + SIG)
    assert not selects("prepare_mx_kernel", "void sharq::prepare_nv_phase1<256, 16, true>" + SIG)


def test_source_hash_ignores_comments_and_whitespace():
    from sparsity_sharq_prepare_amd.profiling import code_text
    a = "int f(int x) {  // doubles x\n  return 2 * x; /* no overflow\n check */ }\n"
    b = "int f(int x) {\n\treturn 2*x;\n}"
    c = "int f(int x) { return 3 * x; }"
    assert code_text(a) == code_text(b)
    assert code_text(a) != code_text(c)
    # a '//' inside a string literal would also start a comment here; the
    # kernel sources have no such literal
    assert code_text("a = 1; // x\nb = 2;") == "a=1;b=2;"
