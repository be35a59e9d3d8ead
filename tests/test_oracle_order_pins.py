"""Pins of the oracle's fp32 operation order where the pages leave it open:
the RMSNorm of the fused preparation (review §3.5) and the two-level NVFP4
scaling (review §3.1; explainer, block-scale section) at a tensor scale other
than 1.  The expected bits come from hand derivations in
``tests/golden/rmsnorm_order_row.txt`` and ``nvfp4_scale_order_row.txt``; each
fixture also records the bits the other plausible orders give, so a slip in
the oracle's order turns these tests red.

The derivations are re-checked here in exact rational arithmetic with an
explicit round-to-nearest-even to fp32 (``rne32``), which shares nothing with
the oracle's numpy code."""
import struct
from fractions import Fraction as Fr

import numpy as np

from oracle import sharq as O
from conftest import read_golden

F32 = np.float32


def rne32(q) -> Fr:
    """The fp32 value nearest to the rational q, ties to the even significand
    (normal and subnormal range; no overflow handling needed here)."""
    q = Fr(q)
    if q == 0:
        return Fr(0)
    a = abs(q)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    if Fr(2) ** e > a:
        e -= 1
    if Fr(2) ** (e + 1) <= a:
        e += 1
    ulp = Fr(2) ** (max(e, -126) - 23)
    n = a / ulp
    m = n.numerator // n.denominator
    rem = n - m
    if rem > Fr(1, 2) or (rem == Fr(1, 2) and m % 2 == 1):
        m += 1
    return (m * ulp) if q > 0 else -(m * ulp)


def bits_of(v) -> int:
    return struct.unpack("<I", struct.pack("<f", float(v)))[0]


def from_bits(h: str) -> Fr:
    return Fr(float(np.frombuffer(struct.pack("<I", int(h, 16)), dtype=F32)[0]))


E2M1 = [Fr(0), Fr(1, 2), Fr(1), Fr(3, 2), Fr(2), Fr(3), Fr(4), Fr(6)]


def e4m3_values():
    out = []
    for c in range(127):
        E, M = c >> 3, c & 7
        out.append(Fr(M, 512) if E == 0 else (1 + Fr(M, 8)) * Fr(2) ** (E - 7))
    return out


E4M3 = e4m3_values()


def nearest_code(u: Fr, table) -> int:
    """Index of the nearest table value to u >= 0, ties to the even index,
    saturating at the last entry (the E2M1 / E4M3 rounding rules)."""
    best = 0
    for c in range(1, len(table)):
        mid = (table[c - 1] + table[c]) / 2
        if u > mid or (u == mid and c % 2 == 0):
            best = c
    return best


def golden_map(name):
    return {r[0]: r[1:] for r in read_golden(name)}


# ------------------------------------------------------------------- RMSNorm
def rmsnorm_row(g):
    K = int(g["K"][0])
    x = np.zeros((1, K), F32)
    gamma = np.ones(K, F32)
    x[0, [int(k) for k in g["x_three"]]] = 3.0
    x[0, [int(k) for k in g["x_two"]]] = 2.0
    x[0, 5], x[0, 18] = float(g["x5"][0]), float(g["x18"][0])
    gamma[5] = float(from_bits(g["gamma5"][0]))
    gamma[18] = float(from_bits(g["gamma18"][0]))
    return x, gamma


def test_rmsnorm_order_fixture_derivation():
    # the hand derivation itself, in exact arithmetic: S, r, inv, and the three
    # orders at k = 5 and k = 18
    g = golden_map("rmsnorm_order_row.txt")
    x, gamma = rmsnorm_row(g)
    assert sum(Fr(float(v)) ** 2 for v in x[0]) == 288
    inv = rne32(Fr(1, 3))
    assert bits_of(inv) == int(g["inv"][0], 16)
    for k, yk, alt in ((5, "y5", "alt5"), (18, "y18", "alt18")):
        xv, gv = Fr(float(x[0, k])), Fr(float(gamma[k]))
        reading = rne32(rne32(xv * inv) * gv)
        other1 = rne32(xv * rne32(inv * gv))
        other2 = rne32(rne32(xv / 3) * gv)
        assert bits_of(reading) == int(g[yk][0], 16)
        assert [bits_of(other1), bits_of(other2)] == [int(h, 16) for h in g[alt]]
        assert len({reading, other1, other2}) == 3
    assert bits_of(rne32(3 * inv)) == int(g["y_three"][0], 16)
    assert bits_of(rne32(2 * inv)) == int(g["y_two"][0], 16)


def test_rmsnorm_order_oracle_matches_fixture():
    g = golden_map("rmsnorm_order_row.txt")
    x, gamma = rmsnorm_row(g)
    y = O.rmsnorm(x, gamma, float(g["eps"][0]))
    yb = y.view(np.uint32)[0]
    assert yb[5] == int(g["y5"][0], 16)
    assert yb[18] == int(g["y18"][0], 16)
    assert np.all(yb[[int(k) for k in g["x_three"]]] == int(g["y_three"][0], 16))
    assert np.all(yb[[int(k) for k in g["x_two"]]] == int(g["y_two"][0], 16))
    # the fused preparation normalizes with the same bits
    p = O.prepare(x, gamma, float(g["eps"][0]), fmt="mxfp4")
    assert np.array_equal(p["y"].view(np.uint32), y.view(np.uint32))


# --------------------------------------------------------------------- NVFP4
def nvfp4_row(g):
    K = int(g["K"][0])
    x = np.zeros((1, K), F32)
    x[0, 0] = float(g["x0"][0])
    x[0, 32] = float(from_bits(g["x32"][0]))
    x[0, 64] = float(g["x64"][0])
    x[0, 66] = float(from_bits(g["x66"][0]))
    return x


def test_nvfp4_order_fixture_derivation():
    g = golden_map("nvfp4_scale_order_row.txt")
    x = nvfp4_row(g)
    xs = [Fr(float(v)) for v in x[0]]
    sT = rne32(Fr(1000) / 2688)
    assert bits_of(sT) == int(g["s_T"][0], 16)
    codes, alt_codes = [], []
    for b in range(3):
        amax = max(abs(v) for v in xs[32 * b: 32 * b + 32])
        codes.append(nearest_code(rne32(rne32(amax / 6) / sT), E4M3))
        alt_codes.append(nearest_code(rne32(amax / rne32(6 * sT)), E4M3))
    assert codes == [int(h, 16) for h in g["scales"]]
    assert alt_codes == [int(h, 16) for h in g["scale_alt"]]
    # element codes under the reading, and the other division order at k = 66
    for k in (0, 32, 64, 66):
        dec = E4M3[codes[k // 32]]
        t = rne32(xs[k] / rne32(dec * sT))
        assert nearest_code(t, E2M1) == int(g["code%d" % k][0])
    dec = E4M3[codes[2]]
    t_alt = rne32(rne32(xs[66] / sT) / dec)
    assert nearest_code(t_alt, E2M1) == int(g["code66_alt"][0])
    assert int(g["code66_alt"][0]) != int(g["code66"][0])


def test_nvfp4_order_oracle_quantizer_and_packer():
    g = golden_map("nvfp4_scale_order_row.txt")
    x = nvfp4_row(g)
    sT = O.nv_tensor_scale(np.abs(x).max())
    assert np.array([sT], F32).view(np.uint32)[0] == int(g["s_T"][0], 16)
    codes, sc = O.nv_quantize(x, 32, sT)
    assert sc[0].tolist() == [int(h, 16) for h in g["scales"]]
    for k in (0, 32, 64, 66):
        assert codes[0, k] == int(g["code%d" % k][0]), k
    # the packer quantizes a weight column the same way (blocks of 32 along K,
    # tensor scale from amax(W))
    wp = O.pack_weight(x.T.copy(), "nvfp4")
    assert np.array(wp["tensor_scale"], F32).view(np.uint32)[0] == int(g["s_T"][0], 16)
    assert wp["scale_sp"][0].tolist() == [int(h, 16) for h in g["scales"]]
    for k in (0, 32, 64, 66):
        assert wp["codes"][0, k] == int(g["code%d" % k][0]), k


def test_nvfp4_order_oracle_prepare_backbone():
    g = golden_map("nvfp4_scale_order_row.txt")
    x = nvfp4_row(g)
    p = O.prepare(x, None, fmt="nvfp4")
    assert np.array([p["tensor_scales"][0]], F32).view(np.uint32)[0] == int(g["s_T"][0], 16)
    assert p["bb_scale"][0].tolist() == [int(h, 16) for h in g["scales"]]
    assert p["bb_meta"][0].tolist() == [int(h, 16) for h in g["bb_meta"]]
    bb = p["bb_codes"][0].reshape(-1, 2)
    for grp in (0, 4, 8):
        assert bb[grp].tolist() == [int(h, 16) for h in g["bb_group%d" % grp]], grp


# ------------------------------------------------- RMSNorm scalar chain, K = 96
def nearest_f32_sqrt(v: Fr) -> Fr:
    """The fp32 value nearest to sqrt(v), found among the neighbours of a
    double-precision estimate by exact comparison of squared midpoints."""
    c = np.float32(np.sqrt(float(v)))
    cands = [c]
    for _ in range(3):
        cands.append(np.nextafter(cands[-1], np.float32(np.inf), dtype=F32))
        cands.insert(0, np.nextafter(cands[0], np.float32(-np.inf), dtype=F32))
    for i in range(1, len(cands) - 1):
        r = Fr(float(cands[i]))
        lo = (Fr(float(cands[i - 1])) + r) / 2
        hi = (r + Fr(float(cands[i + 1]))) / 2
        if lo * lo < v < hi * hi:
            return r
    raise AssertionError("sqrt estimate not bracketed")


def nearest_f32_rsqrt(v: Fr) -> Fr:
    c = np.float32(1.0 / np.sqrt(float(v)))
    cands = [np.nextafter(c, np.float32(-np.inf), dtype=F32), c, np.nextafter(c, np.float32(np.inf), dtype=F32)]
    return min((Fr(float(r)) for r in cands), key=lambda r: abs(r * r * v - 1))


def chain_row(g):
    K = int(g["K"][0])
    x = np.full((1, K), 3.0, F32)
    gamma = np.ones(K, F32)
    x[0, [int(k) for k in g["x_four"]]] = 4.0
    x[0, [int(k) for k in g["x_two"]]] = 2.0
    x[0, 5] = float(g["x5"][0])
    gamma[5] = float(from_bits(g["gamma5"][0]))
    return x, gamma, float(from_bits(g["eps"][0]))


def test_rmsnorm_chain_fixture_derivation():
    g = golden_map("rmsnorm_chain_row.txt")
    x, gamma, eps = chain_row(g)
    K = x.shape[1]
    S = sum(Fr(float(v)) ** 2 for v in x[0])
    assert S == 1004
    ms = rne32(S / K)
    v = rne32(ms + Fr(eps))
    r = nearest_f32_sqrt(v)
    inv = rne32(1 / r)
    for name, val in (("ms", ms), ("v", v), ("r", r), ("inv", inv)):
        assert bits_of(val) == int(g[name][0], 16), name
    gv = Fr(float(gamma[5]))
    y5 = rne32(rne32(7 * inv) * gv)
    assert bits_of(y5) == int(g["y5"][0], 16)
    # the other chains
    ms_r = rne32(S * rne32(Fr(1, K)))
    inv_r = rne32(1 / nearest_f32_sqrt(rne32(ms_r + Fr(eps))))
    inv_c = nearest_f32_rsqrt(v)
    inv_e = rne32(1 / rne32(nearest_f32_sqrt(ms) + Fr(eps)))
    alts = [bits_of(rne32(rne32(7 * i) * gv)) for i in (inv_r, inv_c, inv_e)]
    assert alts == [int(h, 16) for h in g["alt5"]]
    assert int(g["y5"][0], 16) not in alts
    for name, xv in (("y_four", 4), ("y_two", 2), ("y_three", 3)):
        assert bits_of(rne32(xv * inv)) == int(g[name][0], 16), name


def test_rmsnorm_chain_oracle_matches_fixture():
    g = golden_map("rmsnorm_chain_row.txt")
    x, gamma, eps = chain_row(g)
    yb = O.rmsnorm(x, gamma, eps).view(np.uint32)[0]
    assert yb[5] == int(g["y5"][0], 16)
    assert np.all(yb[[int(k) for k in g["x_four"]]] == int(g["y_four"][0], 16))
    assert yb[21] == int(g["y_two"][0], 16)
    threes = np.ones(x.shape[1], bool)
    threes[[5, 21] + [int(k) for k in g["x_four"]]] = False
    assert np.all(yb[threes] == int(g["y_three"][0], 16))
