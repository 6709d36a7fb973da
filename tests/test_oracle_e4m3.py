"""Pins for the oracle's e4m3 decode table and encoder.

The table is checked against an independent library conversion (torch's
float8_e4m3fn on the CPU) and against format facts (largest finite 448,
smallest subnormal 2^-9, smallest normal 2^-6, NaN codes).  The encoder is
checked against torch's round-to-nearest-even cast wherever that cast does not
overflow, on all exact midpoints and on random values in every binade.
"""

import numpy as np
import pytest
import torch

from oracle import decode, decode_table, encode


def torch_decode_all():
    return torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).to(torch.float64).numpy()


def torch_encode(v):
    return torch.from_numpy(np.asarray(v, np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def test_table_matches_library_conversion():
    t = decode_table()
    ref = torch_decode_all()
    assert np.array_equal(np.isnan(t), np.isnan(ref))
    ok = ~np.isnan(ref)
    assert np.array_equal(t[ok], ref[ok])
    # signed zero preserved
    assert np.signbit(t[0x80]) and not np.signbit(t[0x00])


def test_table_format_facts():
    t = decode_table()
    assert t[0x7E] == 448.0 and t[0xFE] == -448.0
    assert t[0x01] == 2.0 ** -9
    assert t[0x07] == 7 * 2.0 ** -9
    assert t[0x08] == 2.0 ** -6
    assert t[0x38] == 1.0
    assert t[0x40] == 2.0 and t[0x3C] == 1.5
    assert np.isnan(t[0x7F]) and np.isnan(t[0xFF])
    assert np.sum(np.isnan(t)) == 2
    pos = t[0x00:0x7F]
    assert np.all(np.diff(pos) > 0)  # strictly increasing
    assert np.array_equal(t[0x80:0xFF], -pos)


def test_round_trip_all_codes():
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], dtype=np.uint8)
    assert np.array_equal(encode(decode(codes)), codes)


def test_encoder_matches_library_on_midpoints():
    t = decode_table()
    pos = t[0x00:0x7F]
    mids = (pos[:-1] + pos[1:]) / 2  # exact in fp32 (<= 5 significant bits)
    vals = np.concatenate([mids, -mids]).astype(np.float32)
    assert np.array_equal(vals.astype(np.float64), np.concatenate([mids, -mids]))
    assert np.array_equal(encode(vals), torch_encode(vals))
    # a few by hand: ties go to the even mantissa
    assert encode(np.float32(1.0625)) == 0x38  # between 1.0 and 1.125 -> 1.0
    assert encode(np.float32(1.1875)) == 0x3A  # between 1.125 and 1.25 -> 1.25
    assert encode(np.float32(2.0 ** -10)) == 0x00  # half the smallest subnormal -> 0
    assert encode(np.float32(464.0)) == 0x7E


def test_encoder_matches_library_random_binades():
    rng = np.random.default_rng(123)
    e = rng.uniform(-14, np.log2(464.0), 200000)
    v = (np.exp2(e) * rng.choice([-1.0, 1.0], e.size)).astype(np.float32)
    v = v[np.abs(v) <= 464.0]
    assert np.array_equal(encode(v), torch_encode(v))


def test_encoder_saturates_instead_of_nan():
    v = np.array([465.0, 1e6, 3e38, -465.0, -1e30], dtype=np.float32)
    assert list(encode(v)) == [0x7E, 0x7E, 0x7E, 0xFE, 0xFE]
    assert encode(np.float32(np.nan)) == 0x7F
    assert encode(np.float32(-0.0)) == 0x80


@pytest.mark.parametrize("x", [0.0, 1e-30, 2.0 ** -9, 3 * 2.0 ** -10, 0.015625, 447.9, 448.0])
def test_encoder_scalar_cases(x):
    assert encode(np.float32(x)) == torch_encode(np.float32(x))
