"""Pins of the oracle's FP4 (e2m1) pieces against facts outside the oracle.

* the decode table against the e2m1 value set {0, 0.5, 1, 1.5, 2, 3, 4, 6}
  (the OCP 4-bit float format), signs in the top bit;
* the encoder against a brute-force nearest search with ties to the even
  code, on every midpoint and on random values, plus saturation;
* the packing against hand-packed bytes;
* the quantisers: each block's largest magnitude lands on +-6, dequantised
  values stay within half an e2m1 step, the scale is amax / 6;
* the GEMM against exact-rational brute force, a closed form (ones give K),
  and the pinned FP8 oracle on the same values (every e2m1 value is also an
  e4m3 value, so both oracles must agree exactly).
"""

from fractions import Fraction

import numpy as np
import pytest

from oracle import e2m1, e4m3, fp4_gemm_nt_ref, gemm_nt_ref, quantize_a_1x128_fp4, quantize_b_128x128_fp4

SET = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]


def test_decode_table_is_the_e2m1_value_set():
    t = e2m1.decode_table()
    assert list(t[:8]) == SET
    assert list(-t[8:]) == SET
    assert np.signbit(t[8])  # code 8 is -0


def brute_encode(v):
    """Nearest of the 16 codes; on a tie the code with an even mantissa
    (bit 0 clear); beyond 6 the largest magnitude."""
    t = e2m1.decode_table()
    best = None
    for c in range(16):
        if (c >> 3) != (1 if np.signbit(v) else 0):
            continue
        d = abs(t[c] - min(abs(v), 6.0) * (-1 if np.signbit(v) else 1))
        key = (d, c & 1)
        if best is None or key < best[0]:
            best = (key, c)
    return best[1]


def test_encoder_against_brute_force():
    mids = [(a + b) / 2 for a, b in zip(SET, SET[1:])]
    vals = SET + mids + [6.5, 100.0, 1e-9, 0.2499, 0.2501]
    rng = np.random.default_rng(3)
    vals += list(rng.uniform(-7, 7, 2000)) + list(rng.normal(0, 1, 2000))
    vals += [-x for x in vals]
    got = e2m1.encode(np.array(vals))
    want = np.array([brute_encode(v) for v in vals], np.uint8)
    assert np.array_equal(got, want)
    # every code decodes and encodes back to itself
    assert np.array_equal(e2m1.encode(e2m1.decode_table()), np.arange(16, dtype=np.uint8))
    with pytest.raises(ValueError):
        e2m1.encode([np.nan])


def test_packing_low_nibble_first():
    codes = np.array([[1, 7, 15, 0, 2, 3]], np.uint8)  # 0.5, 6, -6, 0, 1, 1.5
    packed = e2m1.pack(codes)
    assert packed.tolist() == [[0x71, 0x0F, 0x32]]
    assert np.array_equal(e2m1.unpack(packed), codes)
    assert e2m1.decode_packed(packed).tolist() == [[0.5, 6.0, -6.0, 0.0, 1.0, 1.5]]


def _half_step(v):
    a = np.abs(v)
    return np.where(a < 2, 0.25, np.where(a < 4, 0.5, 1.0))


@pytest.mark.parametrize("which", ["a", "b"])
def test_quantisers_block_rule(which):
    rng = np.random.default_rng(5)
    x = rng.normal(0, 1, (200, 384)).astype(np.float32)
    x[7, 128:256] = 0.0  # an all-zero block: amax floored
    if which == "a":
        p, s = quantize_a_1x128_fp4(x)
        s_el = np.repeat(s, 128, axis=1)
        amax = np.abs(x).reshape(200, 3, 128).max(axis=-1)
    else:
        p, s = quantize_b_128x128_fp4(x)
        s_el = np.repeat(np.repeat(s, 128, axis=0)[:200], 128, axis=1)
        amax = np.stack([np.abs(x[r:r + 128]).reshape(-1, 3, 128).max(axis=(0, 2)) for r in (0, 128)])
    assert p.shape == (200, 192) and p.dtype == np.uint8
    v = e2m1.decode_packed(p)
    scaled = x.astype(np.float64) / s_el
    # within half a step of x / s (a hair more for the fp32 division)
    assert np.all(np.abs(v - np.minimum(np.abs(scaled), 6) * np.sign(scaled)) <= _half_step(scaled) * (1 + 1e-6))
    assert np.allclose(s, np.maximum(amax, 1e-4) / 6.0, rtol=2.0 ** -23)
    # the element of largest magnitude in each block is +-6
    if which == "a":
        top = np.take_along_axis(np.abs(v).reshape(200, 3, 128), np.argmax(np.abs(x).reshape(200, 3, 128), -1)[..., None], -1)
        live = amax >= 1e-4
        assert np.all(top[..., 0][live] == 6.0)
        assert np.all(v[7, 128:256] == 0.0)


def test_gemm_against_exact_brute_force():
    rng = np.random.default_rng(9)
    m, n, k = 3, 5, 256
    ca = rng.integers(0, 16, (m, k)).astype(np.uint8)
    cb = rng.integers(0, 16, (n, k)).astype(np.uint8)
    sa = rng.uniform(0.1, 2, (m, 2)).astype(np.float32)
    sb = rng.uniform(0.1, 2, (1, 2)).astype(np.float32)
    r = fp4_gemm_nt_ref(e2m1.pack(ca), sa, e2m1.pack(cb), sb)
    t = e2m1.decode_table()
    for i in range(m):
        for j in range(n):
            exact, ab = Fraction(0), 0.0
            for s in range(2):
                part = sum(Fraction(t[ca[i, kk]]) * Fraction(t[cb[j, kk]]) for kk in range(128 * s, 128 * s + 128))
                term = part * Fraction(float(sa[i, s])) * Fraction(float(sb[0, s]))
                exact += term
                ab += abs(float(term))
            # slab sums are exact in fp64; the scaled sum of two terms rounds
            # at most three times
            assert abs(Fraction(r[i, j]) - exact) <= Fraction(3 * 2.0 ** -53 * ab)


def test_gemm_closed_form_and_fp8_agreement():
    m, n, k = 4, 130, 384
    ones = np.full((m, k), 2, np.uint8)  # code 2 = 1.0
    r = fp4_gemm_nt_ref(e2m1.pack(ones), np.ones((m, 3), np.float32),
                        e2m1.pack(np.full((n, k), 2, np.uint8)), np.ones((2, 3), np.float32))
    assert np.all(r == k)
    rng = np.random.default_rng(11)
    ca = rng.integers(0, 16, (m, k)).astype(np.uint8)
    cb = rng.integers(0, 16, (n, k)).astype(np.uint8)
    sa = rng.uniform(0.1, 2, (m, 3)).astype(np.float32)
    sb = rng.uniform(0.1, 2, (2, 3)).astype(np.float32)
    r4 = fp4_gemm_nt_ref(e2m1.pack(ca), sa, e2m1.pack(cb), sb)
    t = e2m1.decode_table()
    r8 = gemm_nt_ref(e4m3.encode(t[ca]), sa, e4m3.encode(t[cb]), sb)
    assert np.array_equal(r4, r8)
