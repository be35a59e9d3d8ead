"""CPU oracle -- number formats (TEST INFRASTRUCTURE ONLY).

Plain, slow definitions of the three codecs the SharQ hot path uses.  Only
``tests/``, ``__graft_entry__.smoke()`` and ``bench.py``'s cpu_baseline leg may
import this package; the product path never does.

Sources (pages about "SharQ: Bridging Activation Sparsity and FP4 Quantization
for LLM Inference"):

* review  = the xllm-io paper review (xllm-io.github.io/paper-review), §3.1:
  group-symmetric block quantization uses the scale max|x| / alpha_B of the
  group; NVFP4 is FP4 values + a local block scale + a second, global scale.
* review §5.3: MXFP4 uses a power-of-two scale over a larger group.
* explainer = the kasblo.com explainer, section on outliers dominating the
  FP4 block scale: NVFP4 shares one FP8-E4M3 scale among 16 E2M1 values
  (72 bits per 16 values, 4.5 bits per value).

Readings taken where the pages are silent (each is listed in the design notes):

* E2M1 (FP4): sign bit + 2 exponent bits + 1 mantissa bit, magnitudes
  {0, 0.5, 1, 1.5, 2, 3, 4, 6} for codes 0..7; code = sign << 3 | magnitude
  code.  Values are rounded to the nearest grid value, a value half-way between
  two grid values goes to the one with the even code, values beyond 6 saturate
  to 6, and the sign bit is copied from the input (so -0.1 -> code 0x8).
* E8M0 (MXFP4 block scale): the scale 2**e uses the smallest integer e with
  amax <= 6 * 2**e (amax / alpha rounded *up* to a power of two, so no value
  clips), clamped to [-127, 127]; an all-zero block gets e = -127.  The stored
  byte is e + 127.
* E4M3 (NVFP4 block scale): OCP FP8 E4M3 (bias 7, subnormals m * 2**-9, largest
  finite 448, 0x7F is NaN and never produced); positive inputs are rounded to
  the nearest finite value, ties to the even code, saturating at 448.
"""
from __future__ import annotations

import numpy as np

# magnitude of E2M1 code 0..7
E2M1_MAGNITUDES = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0], dtype=np.float64)
E2M1_MAX = 6.0          # alpha of the FP4 element format
E4M3_MAX = 448.0
E8M0_MIN_EXP = -127
E8M0_MAX_EXP = 127


# ----------------------------------------------------------------------------
# E2M1
# ----------------------------------------------------------------------------
def e2m1_encode(v) -> np.ndarray:
    """E2M1 code (uint8, 0..15) of each (already scaled) value ``v``.

    The magnitude code counts how many decision points between neighbouring
    grid values |v| has passed.  A decision point is the midpoint of two
    neighbours; |v| equal to a midpoint passes it only when the upper neighbour
    has the even code (round half to even).  Beyond the last midpoint (5) every
    value maps to 6 (saturation)."""
    v = np.asarray(v)
    a = np.abs(v.astype(np.float64))
    code = np.zeros(a.shape, dtype=np.uint8)
    for c in range(1, 8):
        mid = 0.5 * (E2M1_MAGNITUDES[c - 1] + E2M1_MAGNITUDES[c])
        passed = (a >= mid) if c % 2 == 0 else (a > mid)
        code += passed.astype(np.uint8)
    sign = np.signbit(v).astype(np.uint8) << 3
    return code | sign


def e2m1_decode(code) -> np.ndarray:
    """Signed value (float64) of each E2M1 code."""
    code = np.asarray(code, dtype=np.uint8)
    mag = E2M1_MAGNITUDES[code & 7]
    return np.where(code & 8, -mag, mag)


# ----------------------------------------------------------------------------
# E8M0
# ----------------------------------------------------------------------------
def e8m0_exponent(amax) -> np.ndarray:
    """Smallest integer e with amax <= 6 * 2**e, clamped to [-127, 127] (int32).

    With amax = m * 2**E, m in [0.5, 1): amax <= 6 * 2**e  <=>  m * 2**(E-e) <= 6,
    which needs E - e <= 3 when m <= 0.75 and E - e <= 2 when m > 0.75."""
    amax = np.asarray(amax, dtype=np.float64)
    m, E = np.frexp(amax)
    e = E - 3 + (m > 0.75).astype(np.int64)
    e = np.where(amax == 0.0, E8M0_MIN_EXP, e)
    return np.clip(e, E8M0_MIN_EXP, E8M0_MAX_EXP).astype(np.int32)


def e8m0_encode_exponent(e) -> np.ndarray:
    return (np.asarray(e, dtype=np.int32) + 127).astype(np.uint8)


def e8m0_decode_exponent(code) -> np.ndarray:
    return np.asarray(code, dtype=np.int32) - 127


# ----------------------------------------------------------------------------
# E4M3 (OCP FP8)
# ----------------------------------------------------------------------------
def e4m3_value_table() -> np.ndarray:
    """Value of every positive finite E4M3 code 0x00..0x7E (float64)."""
    vals = np.empty(127, dtype=np.float64)
    for code in range(127):
        E, M = code >> 3, code & 7
        vals[code] = M * 2.0 ** -9 if E == 0 else (1.0 + M / 8.0) * 2.0 ** (E - 7)
    return vals


_E4M3 = e4m3_value_table()


def e4m3_decode(code) -> np.ndarray:
    code = np.asarray(code, dtype=np.uint8)
    return _E4M3[code & 0x7F]


def e4m3_encode(u) -> np.ndarray:
    """E4M3 code (uint8) of non-negative ``u``: nearest finite value, ties to
    the even code, saturating at 448 (code 0x7E)."""
    u = np.asarray(u, dtype=np.float64)
    code = np.zeros(u.shape, dtype=np.uint8)
    for c in range(1, 127):
        mid = 0.5 * (_E4M3[c - 1] + _E4M3[c])
        passed = (u >= mid) if c % 2 == 0 else (u > mid)
        code += passed.astype(np.uint8)
    return code
