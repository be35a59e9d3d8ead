"""Pins of the oracle's number formats against the format definitions
(hand-derived fixtures and brute-force nearest-value searches)."""
import itertools
import math

import numpy as np
import pytest

from oracle import formats as F
from conftest import read_golden

E2M1_GRID = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]


def brute_e2m1(v: float) -> int:
    """Nearest grid value by exhaustive distance search; among equally near
    candidates the even code wins; sign bit from the input."""
    a = abs(v)
    best = min(range(8), key=lambda c: (abs(a - E2M1_GRID[c]), c % 2, c))
    return best | (8 if math.copysign(1.0, v) < 0 else 0)


def test_e2m1_golden_points():
    for val, code in read_golden("e2m1_points.txt"):
        got = int(F.e2m1_encode(np.array([float(val)]))[0])
        assert got == int(code, 16), (val, got, code)


def test_e2m1_bruteforce_dense_f32():
    # every float32 in [-8, 8] on a lattice of mantissa patterns, plus all
    # midpoints and their float32 neighbours
    rng = np.random.default_rng(1)
    vals = rng.uniform(-8, 8, 20000).astype(np.float32)
    mids = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0], dtype=np.float32)
    near = np.concatenate([mids, np.nextafter(mids, np.float32(0)), np.nextafter(mids, np.float32(9))])
    vals = np.concatenate([vals, near, -near, np.array(E2M1_GRID, np.float32), [np.float32(-0.0)]])
    got = F.e2m1_encode(vals)
    exp = np.array([brute_e2m1(float(v)) for v in vals], dtype=np.uint8)
    assert np.array_equal(got, exp)


def test_e2m1_decode_roundtrip():
    codes = np.arange(16, dtype=np.uint8)
    vals = F.e2m1_decode(codes)
    assert list(vals[:8]) == E2M1_GRID
    assert list(-vals[8:]) == E2M1_GRID
    # encoding an exact grid value gives its code back (except -0 -> 8)
    assert np.array_equal(F.e2m1_encode(vals), codes)


def brute_e8m0(amax: float) -> int:
    for e in range(-127, 128):
        if amax <= 6.0 * 2.0 ** e:
            return e
    return 127


def test_e8m0_bruteforce():
    rng = np.random.default_rng(2)
    vals = [0.0, 1e-45, 1e-40, 2.0 ** -126, 6 * 2.0 ** -128, 1.0, 1.5, 1.5000001, 3.0, 6.0, 6.0000005,
            12.0, 0.2, 1e38, 3.4e38]
    vals += list(rng.lognormal(0, 20, 2000).astype(np.float32))
    for e in range(-127, 126):
        b = np.float32(6.0 * 2.0 ** e)
        vals += [b, np.nextafter(b, np.float32(np.inf)), np.nextafter(b, np.float32(0))]
    vals = np.array(vals, dtype=np.float32)
    vals = vals[np.isfinite(vals)]
    got = F.e8m0_exponent(vals)
    exp = np.array([brute_e8m0(float(v)) for v in vals])
    assert np.array_equal(got, exp)


def test_e8m0_examples():
    # the explainer's block with a single 12: 12 = 6 * 2^1 -> e = 1
    assert F.e8m0_exponent(np.float32(12.0)) == 1
    # 0.2 needs 6 * 2^-4 = 0.375 (6 * 2^-5 = 0.1875 < 0.2)
    assert F.e8m0_exponent(np.float32(0.2)) == -4
    assert F.e8m0_exponent(np.float32(0.0)) == -127
    assert F.e8m0_encode_exponent(np.int32(-127)) == 0
    assert F.e8m0_encode_exponent(np.int32(127)) == 254


def test_e4m3_golden_points():
    for val, code in read_golden("e4m3_points.txt"):
        got = int(F.e4m3_encode(np.array([float(val)]))[0])
        assert got == int(code, 16), (val, hex(got), code)


def test_e4m3_table_and_bruteforce():
    tab = F.e4m3_value_table()
    assert tab[0x38] == 1.0 and tab[0x7E] == 448.0 and tab[0x01] == 2.0 ** -9 and tab[0x08] == 2.0 ** -6
    assert np.all(np.diff(tab) > 0)
    rng = np.random.default_rng(3)
    vals = np.concatenate([rng.uniform(0, 500, 3000), rng.lognormal(-3, 3, 3000),
                           0.5 * (tab[1:] + tab[:-1]), tab])
    got = F.e4m3_encode(vals)
    exp = np.array([min(range(127), key=lambda c: (abs(v - tab[c]), c % 2, c)) for v in vals])
    assert np.array_equal(got, exp)


def test_nvfp4_bits_per_value():
    # explainer: 16 E2M1 values + one E4M3 scale = 72 bits = 4.5 bits / value
    K = 16 * 37
    codes_bytes = K // 2
    scale_bytes = K // 16
    assert (codes_bytes + scale_bytes) * 8 / K == 4.5
