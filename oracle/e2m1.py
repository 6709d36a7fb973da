"""Exact FP4 (e2m1) codec and nibble packing.  Test infrastructure only.

The pages name FP4 beside FP8 and BF16 as a GEMM format ("DeepGEMM: making
LLM matrix multiplication fly", pomoai.com, core functions, first point; its
caveats warn that FP4 may cost accuracy) and say nothing more.  Reading
taken: the 4-bit float e2m1 (1 sign bit, 2 exponent bits with bias 1,
1 mantissa bit, no infinities or NaN), whose magnitudes are
0, 0.5, 1, 1.5, 2, 3, 4 and 6.

Decode rule for a 4-bit code with sign s, exponent e and mantissa f:

    e == 0  ->  (-1)^s * f * 2^-1                 (subnormal)
    e >  0  ->  (-1)^s * (2 + f) * 2^(e - 2)

Two codes share a byte: element 2i in the low nibble, element 2i + 1 in the
high nibble.
"""

import numpy as np

E2M1_MAX = 6.0


def _decode_one(code):
    s = (code >> 3) & 1
    e = (code >> 1) & 3
    f = code & 1
    mag = f * 0.5 if e == 0 else (2 + f) * 2.0 ** (e - 2)
    return -mag if s else mag


_TABLE = np.array([_decode_one(c) for c in range(16)], dtype=np.float64)
_TABLE.setflags(write=False)


def decode_table():
    """The read-only float64 table of the 16 e2m1 codes."""
    return _TABLE


def encode(values):
    """Round values to e2m1 codes (uint8, 0..15): nearest, ties to even,
    saturating at +-6; the sign bit is kept (-0.0 -> 0x8).  NaN raises.

    Exact binary arithmetic: in the binade of |v| (exponent clamped to
    [0, 2], the lowest one also holding the subnormals) one step is
    2^(e - 1); np.rint (half to even) picks the step count q, and the code
    magnitude is 2e + q (q = 4 carries into the next binade)."""
    v = np.asarray(values, dtype=np.float64)
    if np.isnan(v).any():
        raise ValueError("e2m1 has no NaN")
    sign = np.signbit(v).astype(np.uint8) << 3
    a = np.minimum(np.abs(v), E2M1_MAX)
    _, x = np.frexp(a)                      # a = m * 2^x, m in [0.5, 1)
    e = np.clip(x - 1, 0, 2)
    q = np.rint(np.ldexp(a, -(e - 1)))      # exact scaling by a power of two
    mag = (2 * e + q).astype(np.uint8)
    return mag | sign


def pack(codes):
    """Pack codes [..., K] (K even) into bytes [..., K/2], low nibble first."""
    c = np.asarray(codes, dtype=np.uint8)
    if c.shape[-1] % 2:
        raise ValueError("K must be even")
    return (c[..., 0::2] & 0xF) | ((c[..., 1::2] & 0xF) << 4)


def unpack(packed):
    """Inverse of pack: bytes [..., K/2] -> codes [..., K]."""
    p = np.asarray(packed, dtype=np.uint8)
    out = np.empty(p.shape[:-1] + (2 * p.shape[-1],), dtype=np.uint8)
    out[..., 0::2] = p & 0xF
    out[..., 1::2] = p >> 4
    return out


def decode_packed(packed):
    """Packed bytes [..., K/2] -> float64 values [..., K] (exact)."""
    return _TABLE[unpack(packed)]
