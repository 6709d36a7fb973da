"""Exact e4m3 (OCP ``e4m3fn``) decode table and encoder.  Test infrastructure only.

The pages say only "FP8" (deepseek.csdn.net, "technical features";
pomoai.com, "core functions").  Reading taken: the OCP e4m3fn format, 1 sign
bit, 4 exponent bits with bias 7, 3 mantissa bits, no infinities, NaN only at
exponent 15 with mantissa 7 (codes 0x7F and 0xFF), largest finite 448.

Decode rule for a code with sign s, exponent e and mantissa f:

    e == 0            ->  (-1)^s * f * 2^-9              (subnormal)
    e == 15, f == 7   ->  NaN
    otherwise         ->  (-1)^s * (8 + f) * 2^(e - 10)

Every value is a dyadic rational with at most 4 significant bits, so the
float64 table below is exact.
"""

import numpy as np

E4M3_MAX = 448.0
_MIN_NORMAL_EXP = -6  # smallest normal is 2^-6
_SUBNORMAL_QUANTUM = 2.0 ** -9


def _decode_one(code):
    s = (code >> 7) & 1
    e = (code >> 3) & 0xF
    f = code & 0x7
    if e == 15 and f == 7:
        return float("nan")
    if e == 0:
        mag = f * _SUBNORMAL_QUANTUM
    else:
        mag = (8 + f) * 2.0 ** (e - 10)
    return -mag if s else mag


_TABLE = np.array([_decode_one(c) for c in range(256)], dtype=np.float64)
_TABLE.setflags(write=False)


def decode_table():
    """Return the read-only float64 table of all 256 e4m3 codes."""
    return _TABLE


def decode(codes):
    """Decode an array of uint8 e4m3 codes to float64 (exact)."""
    codes = np.asarray(codes, dtype=np.uint8)
    return _TABLE[codes]


def encode(values):
    """Round float values to e4m3 codes: nearest, ties to even, saturating.

    Inputs are taken exactly (float32 inputs are widened to float64, which
    is exact).  |v| >= 448 maps to +-448 (code 0x7E / 0xFE) instead of
    overflowing; the sign bit is kept, so -0.0 maps to 0x80.  NaN maps to
    0x7F.  The rounding is done in exact binary arithmetic: the magnitude is
    scaled by a power of two so that one e4m3 step becomes 1.0, and np.rint
    (round half to even) picks the integer.
    """
    v = np.asarray(values, dtype=np.float64)
    sign = np.signbit(v).astype(np.uint8) << 7
    a = np.abs(v)
    nan = np.isnan(a)
    a = np.where(nan, 0.0, a)
    a = np.minimum(a, E4M3_MAX)

    # Exponent of the e4m3 binade holding a (normals), clamped to the
    # subnormal binade below 2^-6.  frexp gives a = m * 2^x with m in [0.5, 1).
    _, x = np.frexp(a)
    e_unb = np.maximum(x - 1, _MIN_NORMAL_EXP)  # unbiased exponent
    # One step of the 3-bit mantissa in this binade is 2^(e_unb - 3).
    steps = np.ldexp(a, -(e_unb - 3))  # exact: scaling by a power of two
    q = np.rint(steps)  # ties to even
    # q is in [0, 16]; q == 16 means the value rounded up into the next binade.
    # Normal code = (e_unb + 7) << 3 | (q - 8); subnormal (q < 8 in the lowest
    # binade) = q.  Both are covered by biasing: code = (e_unb + 6) * 8 + q,
    # which also handles q == 16 (carry into the exponent field).
    code = (e_unb + 6) * 8 + q.astype(np.int64)
    code = np.where(a == 0.0, 0, code)
    code = np.minimum(code, 0x7E)  # 448 is the largest finite value
    out = code.astype(np.uint8) | sign
    out = np.where(nan, np.uint8(0x7F), out)
    return out.astype(np.uint8)
