"""Pins for the oracle GEMMs.

* exact-rational brute force on tiny shapes (fractions.Fraction, codes
  decoded by torch's float8_e4m3fn conversion, not by the oracle's table);
* with unit scales the result equals a plain whole-K matmul bit for bit;
* closed forms: all-ones operands give K, per-slab and per-block scales give
  128 * sum_kb sa[m,kb] * sb[n//128,kb];
* invariants: scaling a row of sa scales that row of the result exactly,
  the _at variants agree with the full ones bit for bit;
* grouped layouts against the brute force: each row uses its own expert's B,
  padding rows and rows past masked_m have no result, masked_m is clamped;
* the K-grouped layout against the brute force on each group's K columns,
  its groups summing to the dense result, unit scales giving a plain matmul
  per K slice, an empty group giving zero, and bad group sizes rejected;
* the BF16 GEMM: its bf16 decode against torch's, exact-rational brute force,
  and closed forms (ones give K, a one-hot row selects a column of B);
* SiLU against torch's and the identity silu(x) - silu(-x) = x; FC1 + SwiGLU
  with the up half fixed to give exactly 1 (then h = silu(gate)), and with
  the gate half fixed to give exactly 0 (then h = 0); the requantised h
  dequantises to within half an e4m3 step of h, each block's largest |h|
  lands on +-448, and rows past the count stay empty.
"""

from fractions import Fraction

import numpy as np
import pytest
import torch

from oracle import (gemm_nt_ref, gemm_nt_ref_at, grouped_contiguous_ref,
                    grouped_masked_ref, k_grouped_ref, k_grouped_ref_at, tolerance_check,
                    bf16_gemm_nt_ref, bf16_to_f64, masked_swiglu_ref, masked_swiglu_quant_ref, silu,
                    contiguous_swiglu_ref, contiguous_swiglu_quant_ref)
from oracle.gemm import grouped_contiguous_ref_at, grouped_masked_ref_at
from oracle.e4m3 import decode_table

SPECIAL = np.array([0x7E, 0xFE, 0x01, 0x81, 0x00, 0x80, 0x07, 0x08, 0x38, 0x5F], dtype=np.uint8)


def lib_decode(codes):
    t = torch.from_numpy(np.ascontiguousarray(codes, np.uint8)).view(torch.float8_e4m3fn)
    return t.to(torch.float64).numpy()


def random_codes(rng, shape):
    c = rng.integers(0, 256, size=shape).astype(np.uint8)
    c[(c & 0x7F) == 0x7F] = 0x3F  # no NaN codes in operands
    flat = c.reshape(-1)
    pick = rng.random(flat.size) < 0.2
    flat[pick] = rng.choice(SPECIAL, pick.sum())
    return c


def random_scales(rng, shape):
    return (np.exp2(rng.uniform(-12, 2, shape)) * rng.uniform(1, 2, shape)).astype(np.float32)


def brute(qa, sa, qb, sb):
    """Exact rational result and the sum of |terms| per entry."""
    m, k = qa.shape
    n = qb.shape[0]
    da, db = lib_decode(qa), lib_decode(qb)
    r = np.zeros((m, n), dtype=object)
    mag = np.zeros((m, n))
    for i in range(m):
        for j in range(n):
            tot = Fraction(0)
            ab = 0.0
            for kb in range(k // 128):
                sl = 0
                for kk in range(kb * 128, (kb + 1) * 128):
                    sl += Fraction(da[i, kk]) * Fraction(db[j, kk])
                term = sl * Fraction(float(sa[i, kb])) * Fraction(float(sb[j // 128, kb]))
                tot += term
                ab += abs(float(term))
            r[i, j] = tot
            mag[i, j] = ab
    return r, mag


def assert_close_to_exact(got, exact, mag, kslabs):
    bound = (kslabs + 1) * 2.0 ** -53 * mag
    for idx in np.ndindex(got.shape):
        assert abs(Fraction(float(got[idx])) - exact[idx]) <= Fraction(float(bound[idx])) + 0, idx


@pytest.mark.parametrize("m,n,k", [(3, 5, 128), (5, 2, 256), (4, 4, 384), (1, 3, 256)])
def test_dense_brute_force(m, n, k):
    rng = np.random.default_rng(m * 100 + n * 10 + k)
    qa, qb = random_codes(rng, (m, k)), random_codes(rng, (n, k))
    sa, sb = random_scales(rng, (m, k // 128)), random_scales(rng, (1, k // 128))
    exact, mag = brute(qa, sa, qb, sb)
    assert_close_to_exact(gemm_nt_ref(qa, sa, qb, sb), exact, mag, k // 128)


def test_dense_brute_force_two_b_blocks():
    # N spans two 128-row scale blocks (the second partial): column n must use sb[n // 128]
    rng = np.random.default_rng(11)
    m, n, k = 2, 131, 256
    qa, qb = random_codes(rng, (m, k)), random_codes(rng, (n, k))
    sa, sb = random_scales(rng, (m, 2)), random_scales(rng, (2, 2))
    cols = [0, 1, 127, 128, 130]
    got = gemm_nt_ref(qa, sa, qb, sb)[:, cols]
    da, db = lib_decode(qa), lib_decode(qb)
    for i in range(m):
        for jj, j in enumerate(cols):
            tot, ab = Fraction(0), 0.0
            for kb in range(2):
                sl = sum(Fraction(da[i, kk]) * Fraction(db[j, kk]) for kk in range(kb * 128, kb * 128 + 128))
                term = sl * Fraction(float(sa[i, kb])) * Fraction(float(sb[j // 128, kb]))
                tot += term
                ab += abs(float(term))
            assert abs(Fraction(float(got[i, jj])) - tot) <= Fraction(3 * 2.0 ** -53 * ab)


def test_unit_scales_equal_plain_matmul_bitwise():
    rng = np.random.default_rng(3)
    m, n, k = 33, 70, 1024
    qa, qb = random_codes(rng, (m, k)), random_codes(rng, (n, k))
    r = gemm_nt_ref(qa, np.ones((m, 8), np.float32), qb, np.ones((1, 8), np.float32))
    ref = torch.from_numpy(lib_decode(qa)) @ torch.from_numpy(lib_decode(qb)).T
    assert np.array_equal(r, ref.numpy())


def test_ones_closed_forms():
    m, n, k = 4, 320, 1024
    qa = np.full((m, k), 0x38, np.uint8)  # 1.0
    qb = np.full((n, k), 0x38, np.uint8)
    r = gemm_nt_ref(qa, np.ones((m, 8), np.float32), qb, np.ones((3, 8), np.float32))
    assert np.all(r == k)
    r = gemm_nt_ref(qa, np.full((m, 8), 0.5, np.float32), qb, np.full((3, 8), 3.0, np.float32))
    assert np.all(r == 1.5 * k)
    rng = np.random.default_rng(4)
    sa, sb = random_scales(rng, (m, 8)), random_scales(rng, (3, 8))
    r = gemm_nt_ref(qa, sa, qb, sb)
    expect = 128.0 * np.einsum("mk,bk->mb", sa.astype(np.float64), sb.astype(np.float64))
    np.testing.assert_allclose(r, expect[:, np.arange(n) // 128], rtol=1e-15)


def test_row_scale_linearity_exact():
    rng = np.random.default_rng(9)
    m, n, k = 6, 40, 512
    qa, qb = random_codes(rng, (m, k)), random_codes(rng, (n, k))
    sa, sb = random_scales(rng, (m, 4)), random_scales(rng, (1, 4))
    r1 = gemm_nt_ref(qa, sa, qb, sb)
    sa2 = sa.copy()
    sa2[2] *= 2
    r2 = gemm_nt_ref(qa, sa2, qb, sb)
    assert np.array_equal(r2[2], 2 * r1[2])
    assert np.array_equal(np.delete(r2, 2, 0), np.delete(r1, 2, 0))


def test_at_variant_matches_full_bitwise():
    rng = np.random.default_rng(10)
    m, n, k = 50, 300, 768
    qa, qb = random_codes(rng, (m, k)), random_codes(rng, (n, k))
    sa, sb = random_scales(rng, (m, 6)), random_scales(rng, (3, 6))
    full = gemm_nt_ref(qa, sa, qb, sb)
    rows = rng.integers(0, m, 500)
    cols = rng.integers(0, n, 500)
    assert np.array_equal(gemm_nt_ref_at(qa, sa, qb, sb, rows, cols), full[rows, cols])


def test_contiguous_against_brute_force():
    rng = np.random.default_rng(12)
    g, m, n, k = 3, 7, 4, 256
    qa = random_codes(rng, (m, k))
    sa = random_scales(rng, (m, 2))
    qb = random_codes(rng, (g, n, k))
    sb = random_scales(rng, (g, 1, 2))
    idx = np.array([2, 0, -1, 1, 2, 5, 0], dtype=np.int32)  # -1 and 5: no result
    r, valid = grouped_contiguous_ref(qa, sa, qb, sb, idx)
    assert list(valid) == [True, True, False, True, True, False, True]
    assert np.all(np.isnan(r[~valid]))
    for row in np.nonzero(valid)[0]:
        e = idx[row]
        exact, mag = brute(qa[row:row + 1], sa[row:row + 1], qb[e], sb[e])
        assert_close_to_exact(r[row:row + 1], exact, mag, 2)
    rows = np.array([0, 2, 3, 5, 6, 6])
    cols = np.array([1, 0, 3, 2, 0, 3])
    at = grouped_contiguous_ref_at(qa, sa, qb, sb, idx, rows, cols)
    assert np.array_equal(np.isnan(at), np.isnan(r[rows, cols]))
    ok = ~np.isnan(at)
    assert np.array_equal(at[ok], r[rows, cols][ok])


def test_contiguous_equals_per_group_dense():
    rng = np.random.default_rng(13)
    g, n, k = 4, 64, 384
    idx = np.repeat(np.arange(g, dtype=np.int32), [5, 0, 9, 3])
    m = idx.size
    qa, sa = random_codes(rng, (m, k)), random_scales(rng, (m, 3))
    qb, sb = random_codes(rng, (g, n, k)), random_scales(rng, (g, 1, 3))
    r, valid = grouped_contiguous_ref(qa, sa, qb, sb, idx)
    assert valid.all()
    for e in range(g):
        rows = idx == e
        if rows.any():
            # a different, independent route: the dense oracle on that expert's rows
            # against brute force on one sampled row
            i = np.nonzero(rows)[0][0]
            exact, mag = brute(qa[i:i + 1], sa[i:i + 1], qb[e][:3], sb[e])
            assert_close_to_exact(r[i:i + 1, :3], exact, mag, 3)


def test_masked_against_brute_force_and_clamping():
    rng = np.random.default_rng(14)
    g, max_m, n, k = 4, 5, 3, 256
    qa, sa = random_codes(rng, (g, max_m, k)), random_scales(rng, (g, max_m, 2))
    qb, sb = random_codes(rng, (g, n, k)), random_scales(rng, (g, 1, 2))
    masked_m = np.array([2, 0, 9, -3], dtype=np.int32)  # 9 clamps to 5, -3 to 0
    r, valid = grouped_masked_ref(qa, sa, qb, sb, masked_m)
    assert valid.sum(axis=1).tolist() == [2, 0, 5, 0]
    assert np.all(np.isnan(r[~valid])) and not np.any(np.isnan(r[valid]))
    for e, cnt in [(0, 2), (2, 5)]:
        exact, mag = brute(qa[e, :cnt], sa[e, :cnt], qb[e], sb[e])
        assert_close_to_exact(r[e, :cnt], exact, mag, 2)
    gs = np.array([0, 0, 1, 2, 2, 3])
    rs = np.array([1, 2, 0, 4, 0, 0])
    cs = np.array([0, 1, 2, 2, 1, 0])
    at = grouped_masked_ref_at(qa, sa, qb, sb, masked_m, gs, rs, cs)
    full = r[gs, rs, cs]
    assert np.array_equal(np.isnan(at), np.isnan(full))
    assert np.array_equal(at[~np.isnan(at)], full[~np.isnan(full)])


def test_tolerance_rule():
    r = np.array([1.0, -2.0, 1e-6, 100.0])
    rms = float(np.sqrt(np.mean(r * r)))
    assert tolerance_check(r.copy(), r)["ok"]
    d = r * (1 + 7e-3)
    assert tolerance_check(d, r)["ok"]
    d = r.copy()
    d[1] *= 1.05  # err 0.1 > 8e-3*2 + 1e-3*rms (rms ~ 50)
    assert not tolerance_check(d, r)["ok"]
    d = r.copy()
    d[2] = 1e-3 * rms * 0.9  # near-zero element: absolute term covers it
    assert tolerance_check(d, r)["ok"]
    d[2] = np.nan
    res = tolerance_check(d, r)
    assert not res["ok"] and res["n_bad"] == 1


# ---- K-grouped layout (groups concatenated along K)

def test_k_grouped_against_brute_force():
    # three groups of 1, 0 and 2 slabs over K = 512 (the last slab unused)
    rng = np.random.default_rng(21)
    m, n, k = 3, 4, 512
    qa, qb = random_codes(rng, (m, k)), random_codes(rng, (n, k))
    sa, sb = random_scales(rng, (m, 4)), random_scales(rng, (1, 4))
    sizes = [128, 0, 256]
    got = k_grouped_ref(qa, sa, qb, sb, sizes)
    assert got.shape == (3, m, n)
    assert np.all(got[1] == 0.0)  # an empty group is the empty sum
    exact0, mag0 = brute(qa[:, 0:128], sa[:, 0:1], qb[:, 0:128], sb[:, 0:1])
    assert_close_to_exact(got[0], exact0, mag0, 1)
    exact2, mag2 = brute(qa[:, 128:384], sa[:, 1:3], qb[:, 128:384], sb[:, 1:3])
    assert_close_to_exact(got[2], exact2, mag2, 2)


def test_k_grouped_sums_to_dense():
    # linearity: the groups' results add up to the dense result over the
    # K columns they cover (up to fp64 rounding of the regrouped sum)
    rng = np.random.default_rng(22)
    m, n, k = 9, 140, 1280
    qa, qb = random_codes(rng, (m, k)), random_codes(rng, (n, k))
    sa, sb = random_scales(rng, (m, 10)), random_scales(rng, (2, 10))
    sizes = [384, 128, 0, 512]  # 8 of the 10 slabs
    got = k_grouped_ref(qa, sa, qb, sb, sizes).sum(axis=0)
    dense = gemm_nt_ref(qa[:, :1024], sa[:, :8], qb[:, :1024], sb[:, :8])
    da, db = lib_decode(qa[:, :1024]), lib_decode(qb[:, :1024])
    scale_mag = np.abs(da) @ np.abs(db).T * sa[:, :8].max() * sb[:, :8].max()
    assert np.all(np.abs(got - dense) <= 1e-14 * scale_mag + 0.0)


def test_k_grouped_unit_scales_equal_plain_matmul():
    rng = np.random.default_rng(23)
    m, n, k = 17, 33, 768
    qa, qb = random_codes(rng, (m, k)), random_codes(rng, (n, k))
    sizes = [256, 512]
    got = k_grouped_ref(qa, np.ones((m, 6), np.float32), qb, np.ones((1, 6), np.float32), sizes)
    da, db = torch.from_numpy(lib_decode(qa)), torch.from_numpy(lib_decode(qb))
    assert np.array_equal(got[0], (da[:, :256] @ db[:, :256].T).numpy())
    assert np.array_equal(got[1], (da[:, 256:] @ db[:, 256:].T).numpy())


def test_k_grouped_at_matches_full_and_rejects_bad_sizes():
    rng = np.random.default_rng(24)
    m, n, k = 6, 130, 640
    qa, qb = random_codes(rng, (m, k)), random_codes(rng, (n, k))
    sa, sb = random_scales(rng, (m, 5)), random_scales(rng, (2, 5))
    sizes = [128, 384, 0]
    full = k_grouped_ref(qa, sa, qb, sb, sizes)
    g = rng.integers(0, 3, 40)
    r = rng.integers(0, m, 40)
    c = rng.integers(0, n, 40)
    assert np.array_equal(k_grouped_ref_at(qa, sa, qb, sb, sizes, g, r, c), full[g, r, c])
    for bad in ([100], [-128], [512, 256]):
        with pytest.raises(ValueError):
            k_grouped_ref(qa, sa, qb, sb, bad)



# ---- BF16 NT GEMM

def _bf16_bits_from_torch(x):
    return torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def test_bf16_decode_matches_library():
    rng = np.random.default_rng(31)
    bits = rng.integers(0, 1 << 16, 4096).astype(np.uint16)
    bits = bits[(bits & 0x7F80) != 0x7F80]  # no inf / NaN
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(bf16_to_f64(bits), ref)


def test_bf16_gemm_against_brute_force():
    rng = np.random.default_rng(32)
    m, n, k = 3, 4, 64
    a = _bf16_bits_from_torch(rng.standard_normal((m, k)).astype(np.float32) * 3)
    b = _bf16_bits_from_torch(rng.standard_normal((n, k)).astype(np.float32))
    got = bf16_gemm_nt_ref(a, b)
    ta = torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    tb = torch.from_numpy(b.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    for i in range(m):
        for j in range(n):
            exact = sum(Fraction(ta[i, kk]) * Fraction(tb[j, kk]) for kk in range(k))
            mag = sum(abs(ta[i, kk] * tb[j, kk]) for kk in range(k))
            assert abs(Fraction(float(got[i, j])) - exact) <= Fraction(k * 2.0 ** -53 * mag)


def test_bf16_gemm_closed_forms():
    # ones give K; a one-hot row of A picks the matching column of B
    k = 256
    one = np.full((2, k), 0x3F80, np.uint16)
    assert np.all(bf16_gemm_nt_ref(one, one) == k)
    rng = np.random.default_rng(33)
    b = _bf16_bits_from_torch(rng.standard_normal((5, k)).astype(np.float32))
    a = np.zeros((1, k), np.uint16)
    a[0, 17] = 0x3F80
    assert np.array_equal(bf16_gemm_nt_ref(a, b)[0], bf16_to_f64(b[:, 17]))



# ---- FC1 + SwiGLU (masked layout)

def test_silu_against_library_and_identity():
    x = np.linspace(-30, 30, 2001)
    ref = torch.nn.functional.silu(torch.from_numpy(x)).numpy()
    assert np.allclose(silu(x), ref, rtol=1e-15, atol=1e-300)
    assert np.allclose(silu(x) - silu(-x), x, rtol=1e-15, atol=1e-15)
    assert silu(0.0) == 0.0


def _swiglu_case(up_code, gate_code=None, seed=41):
    rng = np.random.default_rng(seed)
    g, max_m, i, k = 2, 5, 128, 256
    qa = random_codes(rng, (g, max_m, k))
    sa = random_scales(rng, (g, max_m, k // 128))
    qb = random_codes(rng, (g, 2 * i, k))
    sb = random_scales(rng, (g, 2, k // 128))
    if gate_code is not None:
        qb[:, :i, :] = gate_code
    # up half: A row . up row must be a known constant: put the code only at
    # K position 0 of every up row and make every A row's K position 0 give
    # one, with unit scales on slab 0 and zero codes elsewhere in the up rows
    qb[:, i:, :] = 0x00
    qb[:, i:, 0] = up_code
    qa[:, :, 0] = 0x38  # 1.0
    sa[:, :, 0] = 1.0
    sb[:, 1, 0] = 1.0
    masked_m = np.array([3, 5], np.int32)
    return qa, sa, qb, sb, masked_m, i


def test_swiglu_with_unit_up_is_silu_of_gate():
    qa, sa, qb, sb, mm, i = _swiglu_case(up_code=0x38)  # up = 1.0 exactly
    h, valid = masked_swiglu_ref(qa, sa, qb, sb, mm)
    r, _ = grouped_masked_ref(qa, sa, qb, sb, mm)
    gate = r[..., :i]
    ref = torch.nn.functional.silu(torch.from_numpy(np.nan_to_num(gate))).numpy()
    assert np.allclose(h[valid], ref[valid], rtol=1e-14, atol=0)
    assert np.all(np.isnan(h[~valid]))
    assert h.shape == (2, 5, i)


def test_swiglu_with_zero_gate_is_zero():
    qa, sa, qb, sb, mm, i = _swiglu_case(up_code=0x48, gate_code=0x00)  # gate = 0, up = 4
    h, valid = masked_swiglu_ref(qa, sa, qb, sb, mm)
    assert np.all(h[valid] == 0.0)


def test_swiglu_requantised_bounds():
    rng = np.random.default_rng(43)
    g, max_m, i, k = 3, 40, 256, 384
    qa = random_codes(rng, (g, max_m, k))
    sa = random_scales(rng, (g, max_m, k // 128))
    qb = random_codes(rng, (g, 2 * i, k))
    sb = random_scales(rng, (g, 4, k // 128))
    mm = np.array([40, 0, 17], np.int32)
    hq, hs, valid = masked_swiglu_quant_ref(qa, sa, qb, sb, mm)
    h, _ = masked_swiglu_ref(qa, sa, qb, sb, mm)
    assert hq.shape == (g, max_m, i) and hs.shape == (g, max_m, i // 128)
    assert np.all(hq[~valid] == 0) and np.all(np.isnan(hs[~valid]))
    vals = decode_table()[hq].astype(np.float64)
    hv = h[valid].reshape(-1, i // 128, 128)
    qv = vals[valid].reshape(-1, i // 128, 128)
    sv = hs[valid].astype(np.float64)
    deq = qv * sv[..., None]
    # e4m3: 3 mantissa bits (half step 2^-4 relative), subnormal step 2^-9
    bound = np.maximum(np.abs(hv) * 2.0 ** -4, sv[..., None] * 2.0 ** -10) * (1 + 2.0 ** -20)
    assert np.all(np.abs(deq - hv) <= bound)
    # the largest |h| of a block maps onto the saturation value
    top = np.take_along_axis(np.abs(qv), np.argmax(np.abs(hv), axis=-1)[..., None], -1)
    assert np.all(top == 448.0)
    # and the scale is that element's magnitude over 448
    amax = np.max(np.abs(hv), axis=-1)
    assert np.allclose(sv, amax / 448.0, rtol=2.0 ** -22)


def _swiglu_contig_case(up_code, gate_code=None, seed=47):
    # the unit-up construction of _swiglu_case on the contiguous layout:
    # expert tags with padding (-1) and an out-of-range tag (2 experts)
    rng = np.random.default_rng(seed)
    g, i, k = 2, 128, 256
    tags = np.array([0, 0, 0, -1, 1, 1, 5, 1, -1, 0], np.int32)
    m = tags.size
    qa = random_codes(rng, (m, k))
    sa = random_scales(rng, (m, k // 128))
    qb = random_codes(rng, (g, 2 * i, k))
    sb = random_scales(rng, (g, 2, k // 128))
    if gate_code is not None:
        qb[:, :i, :] = gate_code
    qb[:, i:, :] = 0x00
    qb[:, i:, 0] = up_code
    qa[:, 0] = 0x38  # 1.0
    sa[:, 0] = 1.0
    sb[:, 1, 0] = 1.0
    return qa, sa, qb, sb, tags, i


def test_contiguous_swiglu_with_unit_up_is_silu_of_gate():
    qa, sa, qb, sb, tags, i = _swiglu_contig_case(up_code=0x38)  # up = 1.0 exactly
    h, valid = contiguous_swiglu_ref(qa, sa, qb, sb, tags)
    assert valid.tolist() == [True, True, True, False, True, True, False, True, False, True]
    # the gate half from the plain dense GEMM of each valid row with its expert
    for r in np.nonzero(valid)[0]:
        gate = gemm_nt_ref(qa[r:r + 1], sa[r:r + 1], qb[tags[r], :i], sb[tags[r], :1])[0]
        ref = torch.nn.functional.silu(torch.from_numpy(gate)).numpy()
        assert np.allclose(h[r], ref, rtol=1e-14, atol=0)
    assert np.all(np.isnan(h[~valid]))
    assert h.shape == (tags.size, i)


def test_contiguous_swiglu_with_zero_gate_is_zero():
    qa, sa, qb, sb, tags, i = _swiglu_contig_case(up_code=0x48, gate_code=0x00)  # gate = 0, up = 4
    h, valid = contiguous_swiglu_ref(qa, sa, qb, sb, tags)
    assert np.all(h[valid] == 0.0)


def test_contiguous_swiglu_matches_the_masked_layout():
    # the same rows and weights laid out both ways give the same h
    rng = np.random.default_rng(53)
    g, i, k = 3, 128, 384
    counts = [5, 0, 9]
    qb = random_codes(rng, (g, 2 * i, k))
    sb = random_scales(rng, (g, 2, k // 128))
    rows = [random_codes(rng, (c, k)) for c in counts]
    srows = [random_scales(rng, (c, k // 128)) for c in counts]
    max_m = max(counts)
    qa_m = np.zeros((g, max_m, k), np.uint8)
    sa_m = np.ones((g, max_m, k // 128), np.float32)
    for e in range(g):
        qa_m[e, :counts[e]], sa_m[e, :counts[e]] = rows[e], srows[e]
    h_m, _ = masked_swiglu_ref(qa_m, sa_m, qb, sb, np.array(counts, np.int32))
    qa_c = np.concatenate(rows)
    sa_c = np.concatenate(srows)
    tags = np.concatenate([np.full(c, e, np.int32) for e, c in enumerate(counts)])
    h_c, valid = contiguous_swiglu_ref(qa_c, sa_c, qb, sb, tags)
    assert valid.all()
    assert np.array_equal(h_c, np.concatenate([h_m[e, :counts[e]] for e in range(g)]))


def test_contiguous_swiglu_requantised_bounds():
    rng = np.random.default_rng(59)
    g, i, k = 3, 256, 384
    tags = np.array([0] * 7 + [-1] * 3 + [2] * 11 + [1] * 4, np.int32)
    m = tags.size
    qa = random_codes(rng, (m, k))
    sa = random_scales(rng, (m, k // 128))
    qb = random_codes(rng, (g, 2 * i, k))
    sb = random_scales(rng, (g, 4, k // 128))
    hq, hs, valid = contiguous_swiglu_quant_ref(qa, sa, qb, sb, tags)
    h, _ = contiguous_swiglu_ref(qa, sa, qb, sb, tags)
    assert hq.shape == (m, i) and hs.shape == (m, i // 128)
    assert np.all(hq[~valid] == 0) and np.all(np.isnan(hs[~valid]))
    vals = decode_table()[hq].astype(np.float64)
    hv = h[valid].reshape(-1, i // 128, 128)
    qv = vals[valid].reshape(-1, i // 128, 128)
    sv = hs[valid].astype(np.float64)
    deq = qv * sv[..., None]
    bound = np.maximum(np.abs(hv) * 2.0 ** -4, sv[..., None] * 2.0 ** -10) * (1 + 2.0 ** -20)
    assert np.all(np.abs(deq - hv) <= bound)
    top = np.take_along_axis(np.abs(qv), np.argmax(np.abs(hv), axis=-1)[..., None], -1)
    assert np.all(top == 448.0)
    amax = np.max(np.abs(hv), axis=-1)
    assert np.allclose(sv, amax / 448.0, rtol=2.0 ** -22)
