"""Pins for the oracle quantisers (1x128 for A, 128x128 for B).

Checked against an independent construction: the scale computed in fp32 by
torch, the codes by torch's float8_e4m3fn cast after clamping to +-448; and
against the invariants the scaling rule fixes: the block's largest element
lands on +-448, every code is within half an e4m3 step of x/s, partial row
blocks use only their own rows, an all-zero block gives zero codes.
"""

import numpy as np
import torch

from oracle import decode, quantize_a_1x128, quantize_b_128x128


def torch_codes(x, s):
    xs = torch.from_numpy(x) / torch.from_numpy(s)
    return xs.clamp(-448.0, 448.0).to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def test_quant_a_against_library():
    rng = np.random.default_rng(5)
    x = rng.standard_normal((37, 384), dtype=np.float32) * np.float32(3.0)
    q, s = quantize_a_1x128(x)
    assert q.shape == (37, 384) and s.shape == (37, 3) and s.dtype == np.float32
    xt = torch.from_numpy(x).view(37, 3, 128)
    amax = xt.abs().amax(dim=2).clamp_min(torch.tensor(1e-4, dtype=torch.float32))
    s_ref = (amax / 448.0).numpy()
    assert np.array_equal(s, s_ref)
    codes = torch_codes(x.reshape(37, 3, 128), s_ref[:, :, None]).reshape(37, 384)
    assert np.array_equal(q, codes)


def test_quant_b_against_library_with_tail():
    rng = np.random.default_rng(6)
    n, k = 200, 256  # two row blocks, the second holds 72 rows
    x = rng.standard_normal((n, k), dtype=np.float32) * np.float32(0.02)
    q, s = quantize_b_128x128(x)
    assert s.shape == (2, 2)
    for bi, (r0, r1) in enumerate([(0, 128), (128, 200)]):
        for kb in range(2):
            blk = x[r0:r1, kb * 128:(kb + 1) * 128]
            amax = np.float32(np.abs(blk).max())
            s_ref = np.float32(max(amax, np.float32(1e-4)) / np.float32(448.0))
            assert s[bi, kb] == s_ref
            assert np.array_equal(q[r0:r1, kb * 128:(kb + 1) * 128],
                                  torch_codes(blk, np.full(blk.shape, s_ref, np.float32)))


def test_amax_element_maps_to_448_and_error_bound():
    rng = np.random.default_rng(7)
    x = rng.standard_normal((16, 512), dtype=np.float32)
    q, s = quantize_a_1x128(x)
    xb = x.reshape(16, 4, 128)
    qb = q.reshape(16, 4, 128)
    idx = np.abs(xb).argmax(axis=2)
    top = np.take_along_axis(qb, idx[:, :, None], 2)[:, :, 0]
    assert np.all((top == 0x7E) | (top == 0xFE))
    # |decode(q) * s - x| <= half an e4m3 step of x/s, times s
    y = (xb / s[:, :, None]).astype(np.float64)
    _, ex = np.frexp(np.abs(y))
    step = np.exp2(np.maximum(ex - 1, -6) - 3)
    err = np.abs(decode(qb) - y)
    assert np.all(err <= step / 2 + 1e-12)


def test_zero_block_and_floor():
    x = np.zeros((2, 256), dtype=np.float32)
    x[1, 200] = 1.0
    q, s = quantize_a_1x128(x)
    assert np.all(q[0] == 0) and np.all(q[1, :128] == 0)
    assert s[0, 0] == np.float32(np.float32(1e-4) / np.float32(448))
    assert q[1, 200] == 0x7E and s[1, 1] == np.float32(np.float32(1.0) / np.float32(448))


def test_quant_a_rows_are_independent():
    rng = np.random.default_rng(8)
    x = rng.standard_normal((20, 256), dtype=np.float32)
    q, s = quantize_a_1x128(x)
    q5, s5 = quantize_a_1x128(x[5:9])
    assert np.array_equal(q[5:9], q5) and np.array_equal(s[5:9], s5)
