"""The algorithmic byte and flop accounting used for roofline figures.

Pinned to the pages: the decode-shape row of the performance table in
"DeepSeek open-source week day 3" gives 206 TFLOPS together with 1688 GB/s
for M=64 N=2112 K=7168, so bytes = flops * 1688e9 / 206e12 up to the pages'
rounding.  The configuration sizes quoted for the workloads follow from the
shapes.
"""

import json
import os

import numpy as np

import workloads as W

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "pages_perf_table.json")


def test_byte_convention_matches_pages_decode_row():
    g = json.load(open(GOLDEN))["dense_decode"]
    flops, nbytes = W.algorithmic_work("dense", m=g["m"], n=g["n"], k=g["k"])
    assert flops == 2.0 * 64 * 2112 * 7168
    implied = flops * (g["gb_per_s"] * 1e9) / (g["tflops"] * 1e12)
    # 206 is given to 3 significant digits: +-0.25% on the ratio
    assert abs(nbytes - implied) / implied < 0.003
    # counting D as fp32 instead of bf16 would break the pin
    assert abs(nbytes + 2 * 64 * 2112 - implied) / implied > 0.003


def test_named_workload_sizes():
    f, b = W.workload_work("dense_128x512x1024")
    assert (f, b) == (2.0 * 128 * 512 * 1024, 131072 + 4096 + 524288 + 128 + 131072)
    f, b = W.workload_work("dense_large_4096x7168x16384")
    assert b == 245395456 and f == 2.0 * 4096 * 7168 * 16384
    f, b = W.workload_work("moe_contiguous_4x8192_n4096_k7168")
    assert b == 628256768
    f, b = W.workload_work("fp4_dense_4096x7168x16384")
    # the FP8 large shape's bytes with A and B at half a byte per element
    assert f == 2.0 * 4096 * 7168 * 16384 and b == 245395456 - (4096 + 7168) * 16384 // 2
    f, b = W.workload_work("moe_masked_16x256_n4096_k7168")
    assert b == 502088928 and f == 2.0 * 2067 * 4096 * 7168
    # the fused FC1 + SwiGLU on the same inputs: D (2 bytes x 4096) becomes h
    # codes (1 byte x 2048) plus one fp32 scale per 128 of them
    f2, b2 = W.workload_work("moe_swiglu_16x256_i2048_k7168")
    assert f2 == f and b2 == b - 2067 * 4096 * 2 + 2067 * 2048 + 2067 * 16 * 4
    # the same exchange on the contiguous layout's 32768 tagged rows
    f, b = W.workload_work("moe_contiguous_4x8192_n4096_k7168")
    f2, b2 = W.workload_work("moe_swiglu_contig_4x8192_i2048_k7168")
    assert f2 == f and b2 == b - 32768 * 4096 * 2 + 32768 * 2048 + 32768 * 16 * 4


def test_masked_draw_recipe():
    mm = np.random.default_rng(0).integers(0, 257, 16)
    assert int(mm.sum()) == 2067
    inp = W.draw_masked(2, 8, 16, 128, seed=0)
    assert inp["a"].shape == (2, 8, 128) and inp["b"].shape == (2, 16, 128)


def test_contiguous_indices_padding():
    idx = W.contiguous_indices([5, 0, 130])
    assert idx.size == 128 + 0 + 256
    assert (idx[:5] == 0).all() and (idx[5:128] == -1).all()
    assert (idx[128:258] == 2).all() and (idx[258:] == -1).all()
