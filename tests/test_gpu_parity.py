"""GPU parity: the library's GEMMs against the oracle, element by element.

Operands are drawn by `workloads`, quantised on the CPU by the oracle, and
the same bytes are given to the GPU, so these tests check the GEMM alone.
Sizes span several tiles of every configuration and ragged tails in M and N
(N=2112 has a 64-row partial scale block).  The acceptance rule is
|d - r| <= 8e-3 |r| + 1e-3 rms(r) over valid elements; every element without
a result must keep the 0xFFFF sentinel, and the guard band past D must stay
untouched.
"""

import os

import numpy as np
import pytest

import fp8_block_scaled_nt_amd as dg
import oracle
import workloads as W
from tests import gpu_harness as H

pytestmark = pytest.mark.gpu

DENSE_CONFIGS = ["dense_256x256_w8_s2", "dense_256x128_w8_s3", "dense_128x256_w8_s3", "dense_128x128_w4_s3",
                 "dense_128x128_w4_s2", "dense_64x64_w4_s3", "dense_64x64_w4_s8", "dense_64x32_w4_s4", "dense_256x224_w8_s2",
                 "dense_128x256_w4_s3_wide", "dense_256x256_w8_s2_pp", "dense_256x128_w4_s2",
                 "dense_256x128_w4_s3", "dense_128x256_w4_s3", "dense_128x256_w4_s2_sb",
                 "dense_64x32_w4_s4_pair", "dense_64x32_w4_s6_triple", "dense_64x64_w4_s4_pair"]


def dense_case(m, n, k, seed, b_std=1.0):
    x = W.draw_dense(m, n, k, seed=seed, b_std=b_std)
    qa, sa = oracle.quantize_a_1x128(x["a"])
    qb, sb = oracle.quantize_b_128x128(x["b"])
    return qa, sa, qb, sb


def check_dense(gpu, qa, sa, qb, sb, label):
    print(f"[case] {label}", flush=True)
    d, flat = H.run_dense(qa, sa, qb, sb, gpu)
    r = oracle.gemm_nt_ref(qa, sa, qb, sb)
    res = oracle.tolerance_check(H.d_float(d), r)
    assert res["ok"], (label, res)
    assert H.guard_untouched(flat, d.numel()), label
    return d


@pytest.mark.parametrize("m,n,k", [
    (128, 512, 1024),   # the small dense workload
    (1, 16, 128),
    (17, 40, 256),
    (200, 176, 384),
    (64, 2112, 512),
    (300, 520, 640),
    (513, 257, 256),
    # each branch of the tile rules below the large shapes: 64 x 32 for M <= 64
    # up to N 8192 with short K, 64 x 64 for wider N or longer K; M <= 128 with
    # short K: 64 x 32 up to 64 tiles of 128 x 128, 64 x 64 up to 128; 51-72
    # tiles: 128 x 128 with 3 stages; short K over at most one tile per CU: the
    # same tile unsplit
    (64, 7000, 2048),
    (64, 5000, 3072),
    (48, 9000, 512),
    (128, 7168, 1536),
    (128, 12000, 1536),
    (384, 2112, 1024),
    (384, 8192, 1024),
])
def test_dense_default_selection(gpu, m, n, k):
    check_dense(gpu, *dense_case(m, n, k, seed=m + n + k), label=f"dense {m}x{n}x{k}")


@pytest.mark.parametrize("cfg", DENSE_CONFIGS)
@pytest.mark.parametrize("m,n,k", [(300, 520, 640), (64, 200, 384), (520, 300, 256)])
def test_dense_every_config(gpu, cfg, m, n, k, monkeypatch):
    monkeypatch.setenv("DG_FORCE_CONFIG", cfg)
    check_dense(gpu, *dense_case(m, n, k, seed=7), label=f"{cfg} {m}x{n}x{k}")


def test_dense_small_workload_matches(gpu):
    x = W.draw("dense_128x512x1024")
    qa, sa = oracle.quantize_a_1x128(x["a"])
    qb, sb = oracle.quantize_b_128x128(x["b"])
    d = check_dense(gpu, qa, sa, qb, sb, "dense_128x512x1024 seed 0")
    # run-to-run determinism (split-K partials are added in a fixed order)
    d2, _ = H.run_dense(qa, sa, qb, sb, gpu)
    assert np.array_equal(H.d_bits(d), H.d_bits(d2))


def test_dense_unit_scale_exact_values(gpu):
    # all-ones operands with unit scales: every output is exactly k
    m, n, k = 96, 144, 1024
    qa = np.full((m, k), 0x38, np.uint8)
    qb = np.full((n, k), 0x38, np.uint8)
    d, _ = H.run_dense(qa, np.ones((m, 8), np.float32), qb, np.ones((2, 8), np.float32), gpu)
    assert np.all(H.d_float(d) == k)


@pytest.mark.parametrize("cfg", [None, "contig_128x256_w8_s3", "contig_128x128_w4_s3", "contig_128x128_w4_s2",
                                 "contig_128x256_w8_s2", "contig_128x256_w4_s3", "contig_128x256_w4_s2",
                                 "contig_128x256_w4_s2_sb", "contig_64x64_w4_s3"])
def test_contiguous(gpu, cfg, monkeypatch):
    if cfg:
        monkeypatch.setenv("DG_FORCE_CONFIG", cfg)
    group_rows = [200, 0, 77, 128, 5]
    n, k = 384, 512
    x = W.draw_contiguous(group_rows, n, k, seed=3)
    idx = x["m_indices"].copy()
    idx[5] = 99  # an out-of-range tag inside expert 0's block: no result
    qa, sa = oracle.quantize_a_1x128(x["a"])
    qbs = [oracle.quantize_b_128x128(x["b"][g]) for g in range(len(group_rows))]
    qb = np.stack([q for q, _ in qbs])
    sb = np.stack([s for _, s in qbs])
    print(f"[case] contiguous {cfg} rows={group_rows}", flush=True)
    d, flat = H.run_contiguous(qa, sa, qb, sb, idx, gpu)
    r, valid = oracle.grouped_contiguous_ref(qa, sa, qb, sb, idx)
    res = oracle.tolerance_check(H.d_float(d), r, valid[:, None])
    assert res["ok"], res
    bits = H.d_bits(d)
    assert np.all(bits[~valid] == H.SENTINEL)
    assert H.guard_untouched(flat, d.numel())


def test_contiguous_block_expert_same_for_64_row_tiles(gpu, monkeypatch):
    # A 128-row block whose rows carry two valid tags (outside the alignment
    # contract): its expert is the largest tag, and rows with another tag get
    # no result.  A 64-row tile scans the whole block, so it must agree with
    # the 128-row tile bit for bit.
    group_rows = [128, 128, 256]
    n, k = 320, 384
    x = W.draw_contiguous(group_rows, n, k, seed=9)
    idx = x["m_indices"].copy()
    idx[64:128] = 1  # block 0: rows 0-63 tag 0, rows 64-127 tag 1 -> expert 1
    qa, sa = oracle.quantize_a_1x128(x["a"])
    qbs = [oracle.quantize_b_128x128(x["b"][g]) for g in range(len(group_rows))]
    qb = np.stack([q for q, _ in qbs])
    sb = np.stack([s for _, s in qbs])
    out = {}
    for cfg in ["contig_128x128_w4_s2", "contig_64x64_w4_s3"]:
        monkeypatch.setenv("DG_FORCE_CONFIG", cfg)
        print(f"[case] contiguous mixed block {cfg}", flush=True)
        d, _ = H.run_contiguous(qa, sa, qb, sb, idx, gpu)
        out[cfg] = H.d_bits(d)
    assert np.array_equal(out["contig_128x128_w4_s2"], out["contig_64x64_w4_s3"])
    bits = out["contig_64x64_w4_s3"]
    assert np.all(bits[:64] == H.SENTINEL)  # tag 0 in a block whose expert is 1
    r, valid = oracle.grouped_contiguous_ref(qa, sa, qb, sb, idx)
    got = bits[64:].view(np.uint16).astype(np.uint32) << 16
    res = oracle.tolerance_check(got.view(np.float32).astype(np.float64), r[64:], valid[64:, None])
    assert res["ok"], res


@pytest.mark.parametrize("cfg,max_m", [(None, 96), (None, 256), ("masked_256x128_w4_s2", 300),
                                       ("masked_256x128_w4_s3", 200), ("masked_64x64_w4_s3", 130),
                                       ("masked_256x256_w8_s2", 300), ("masked_256x256_w8_s2_pp", 300),
                                       ("masked_256x256_w8_s2_pp", 200), ("masked_256x128_w8_s2", 300),
                                       ("masked_256x128_w8_s2", 100), ("masked_128x256_w8_s3", 300),
                                       ("masked_128x256_w8_s3", 100)])
def test_masked(gpu, cfg, max_m, monkeypatch):
    if cfg:
        monkeypatch.setenv("DG_FORCE_CONFIG", cfg)
    g, n, k = 6, 272, 384
    masked_m = np.array([0, 1, 17, max_m, max_m + 50, max_m // 2 + 3], dtype=np.int32)
    x = W.draw_masked(g, max_m, n, k, seed=4, masked_m=masked_m)
    qas = [oracle.quantize_a_1x128(x["a"][i]) for i in range(g)]
    qa = np.stack([q for q, _ in qas])
    sa = np.stack([s for _, s in qas])
    qbs = [oracle.quantize_b_128x128(x["b"][i]) for i in range(g)]
    qb = np.stack([q for q, _ in qbs])
    sb = np.stack([s for _, s in qbs])
    print(f"[case] masked {cfg} max_m={max_m}", flush=True)
    d, flat = H.run_masked(qa, sa, qb, sb, masked_m, gpu)
    r, valid = oracle.grouped_masked_ref(qa, sa, qb, sb, masked_m)
    res = oracle.tolerance_check(H.d_float(d), r, valid[:, :, None])
    assert res["ok"], res
    bits = H.d_bits(d)
    assert np.all(bits[~valid] == H.SENTINEL)
    assert H.guard_untouched(flat, d.numel())


@pytest.mark.parametrize("cfg", [None, "masked_64x64_w4_s3", "masked_256x256_w8_s2_pp", "masked_128x256_w8_s3"])
def test_masked_many_experts(gpu, cfg, monkeypatch):
    """150 experts, more than two 64-expert chunks of the valid-tile walk:
    empty experts, experts past max_m and runs of empty experts across the
    chunk boundaries; the valid tiles are far fewer than the grid."""
    if cfg:
        monkeypatch.setenv("DG_FORCE_CONFIG", cfg)
    g, max_m, n, k = 150, 80, 144, 256
    rng = np.random.default_rng(31)
    masked_m = rng.integers(0, max_m + 1, g).astype(np.int32)
    masked_m[rng.integers(0, g, 40)] = 0
    masked_m[60:70] = 0
    masked_m[127:131] = 0
    masked_m[63], masked_m[64], masked_m[128] = max_m + 7, 1, 65
    masked_m[-1] = max_m
    x = W.draw_masked(g, max_m, n, k, seed=32, masked_m=masked_m)
    qas = [oracle.quantize_a_1x128(x["a"][i]) for i in range(g)]
    qa = np.stack([q for q, _ in qas])
    sa = np.stack([s for _, s in qas])
    qbs = [oracle.quantize_b_128x128(x["b"][i]) for i in range(g)]
    qb = np.stack([q for q, _ in qbs])
    sb = np.stack([s for _, s in qbs])
    print(f"[case] masked many experts {cfg}", flush=True)
    d, flat = H.run_masked(qa, sa, qb, sb, masked_m, gpu)
    r, valid = oracle.grouped_masked_ref(qa, sa, qb, sb, masked_m)
    res = oracle.tolerance_check(H.d_float(d), r, valid[:, :, None])
    assert res["ok"], res
    assert np.all(H.d_bits(d)[~valid] == H.SENTINEL)
    assert H.guard_untouched(flat, d.numel())


def test_masked_expected_m_steers_schedule_only(gpu):
    # expected_m 0 (unknown) and 150 keep the ping-pong schedule, 1..80 the
    # interleaved one; each is checked against the oracle, and all give the
    # same bits (both promote every slab in the same order)
    g, max_m, n, k = 5, 256, 512, 640
    masked_m = np.array([40, 0, 256, 7, 129], dtype=np.int32)
    x = W.draw_masked(g, max_m, n, k, seed=21, masked_m=masked_m)
    qas = [oracle.quantize_a_1x128(x["a"][i]) for i in range(g)]
    qa = np.stack([q for q, _ in qas])
    sa = np.stack([s for _, s in qas])
    qbs = [oracle.quantize_b_128x128(x["b"][i]) for i in range(g)]
    qb = np.stack([q for q, _ in qbs])
    sb = np.stack([s for _, s in qbs])
    r, valid = oracle.grouped_masked_ref(qa, sa, qb, sb, masked_m)
    bits = []
    for em in (0, 32, 80, 81, 150):
        print(f"[case] masked expected_m={em}", flush=True)
        d, flat = H.run_masked(qa, sa, qb, sb, masked_m, gpu, expected_m=em)
        res = oracle.tolerance_check(H.d_float(d), r, valid[:, :, None])
        assert res["ok"], (em, res)
        assert H.guard_untouched(flat, d.numel())
        bits.append(H.d_bits(d))
    for b in bits[1:]:
        assert np.array_equal(b, bits[0])


@pytest.mark.parametrize("max_m,counts", [
    (256, [40, 0, 256, 7, 129, 128, 1, 90]),   # experts past 128 rows: second row of 128-row tiles
    (128, [128, 0, 64, 1, 127, 33, 100, 12]),  # max_m 128: the 128-row tile whatever the hint
])
def test_masked_tile_rule_wide(gpu, max_m, counts):
    # 8 experts x 16 column tiles cover half the CUs, so hints up to 48 (and
    # max_m <= 128) take the 128-row tile, up to 80 the 256-row interleaved
    # schedule, else ping-pong: every choice matches the oracle with the
    # same bits
    g, n, k = 8, 4096, 256
    masked_m = np.array(counts, dtype=np.int32)
    x = W.draw_masked(g, max_m, n, k, seed=23, masked_m=masked_m)
    qas = [oracle.quantize_a_1x128(x["a"][i]) for i in range(g)]
    qa = np.stack([q for q, _ in qas])
    sa = np.stack([s for _, s in qas])
    qbs = [oracle.quantize_b_128x128(x["b"][i]) for i in range(g)]
    qb = np.stack([q for q, _ in qbs])
    sb = np.stack([s for _, s in qbs])
    r, valid = oracle.grouped_masked_ref(qa, sa, qb, sb, masked_m)
    bits = []
    for em in (0, 16, 48, 64, 100):
        print(f"[case] masked wide max_m={max_m} expected_m={em}", flush=True)
        d, flat = H.run_masked(qa, sa, qb, sb, masked_m, gpu, expected_m=em)
        res = oracle.tolerance_check(H.d_float(d), r, valid[:, :, None])
        assert res["ok"], (em, res)
        assert np.all(H.d_bits(d)[~valid] == H.SENTINEL)
        assert H.guard_untouched(flat, d.numel())
        bits.append(H.d_bits(d))
    for b in bits[1:]:
        assert np.array_equal(b, bits[0])


def test_too_many_tiles_is_rejected(gpu):
    # each operand stays below 4 GiB, but 2^24 x 2^24 outputs are 2^32 tiles:
    # the host rejects the call before touching the (fake) pointers
    import ctypes
    lib = dg.lib()
    fake = ctypes.c_void_p(0x10000)
    big = 1 << 24
    assert lib.dg_fp8_gemm_nt(fake, fake, fake, fake, fake, big, big, 128, None) == 2
    assert b"too many output tiles" in lib.dg_last_error_message()
    out = ctypes.c_size_t(0)
    assert lib.dg_dense_workspace_size(0, big, big, 128, ctypes.byref(out)) == 2


def test_unknown_forced_config_is_an_error(gpu, monkeypatch):
    monkeypatch.setenv("DG_FORCE_CONFIG", "no_such_config")
    qa, sa, qb, sb = dense_case(64, 64, 128, seed=1)
    with pytest.raises(Exception, match="DG_FORCE_CONFIG"):
        H.run_dense(qa, sa, qb, sb, gpu)


def test_dense_long_k_pipeline(gpu):
    # many slabs: the prologue, the steady state and the drain of the load pipeline
    for cfg in DENSE_CONFIGS:
        import os
        os.environ["DG_FORCE_CONFIG"] = cfg
        try:
            check_dense(gpu, *dense_case(136, 264, 128 * 13, seed=5), label=f"{cfg} long k")
            check_dense(gpu, *dense_case(136, 264, 128 * 2, seed=6), label=f"{cfg} k=256")
            check_dense(gpu, *dense_case(136, 264, 128, seed=7), label=f"{cfg} k=128")
        finally:
            del os.environ["DG_FORCE_CONFIG"]


@pytest.mark.parametrize("m,n,k,splits", [
    (64, 2112, 7168, None),   # the decode shape, default split choice
    (17, 200, 1280, "3"),     # 10 slabs over 3 splits: 4 + 4 + 2
    (1, 64, 512, "4"),
    (64, 130, 896, "7"),      # one slab per split
    (100, 192, 768, "2"),     # two tile rows
    (64, 130, 1408, "11"),    # more splits than one batch of the reducer's partial loads
])
@pytest.mark.parametrize("cfg", ["dense_64x64_w4_s8", "dense_64x32_w4_s4", "dense_128x128_w4_s2",
                                 "dense_128x256_w4_s2_sb", "dense_64x32_w4_s6_triple", "dense_64x32_w4_s4_pair"])
def test_dense_split_k(gpu, m, n, k, splits, cfg, monkeypatch):
    if splits:
        monkeypatch.setenv("DG_SPLIT_K", splits)
    monkeypatch.setenv("DG_FORCE_CONFIG", cfg)
    qa, sa, qb, sb = dense_case(m, n, k, seed=m * 3 + k, b_std=0.02)
    d = check_dense(gpu, qa, sa, qb, sb, label=f"split-K {cfg} {m}x{n}x{k} splits={splits}")
    # bit-for-bit reproducible, and the arrival counters are reset for the next call
    d2, _ = H.run_dense(qa, sa, qb, sb, gpu)
    assert np.array_equal(H.d_bits(d), H.d_bits(d2))


@pytest.mark.parametrize("m,n,k", [
    (1024, 896, 2048),   # 16 big tiles: 128 x 128 tiles, 8 splits of 2 slabs
    (512, 1792, 1536),   # 56 tiles of 128 x 128 over 6 splits
    (2304, 2304, 512),   # 81 big tiles: 128 x 128, no split (324 tiles, 2 slabs each)
    (128, 2112, 1024),   # 17 tiles of 128 x 128: 64 x 64 tiles, 3 stages, split-K
    (256, 512, 1280),    # n <= 1024: 64 x 32 tiles, split-K
    (384, 2112, 768),    # 51 tiles of 128 x 128: 3 stages
    (200, 4096, 384),    # a partial 64-row tile row, 3 slabs
])
def test_dense_default_mid_shapes(gpu, m, n, k):
    # shapes whose 256 x 256 tiles would leave most CUs idle take 128 x 128
    # tiles (with three stages when they are few), 64 x 64 or 64 x 32 tiles
    # when m <= 256 and the 128 x 128 tiles are fewer than 65, and split-K
    # while still too few
    qa, sa, qb, sb = dense_case(m, n, k, seed=m + n + k)
    d = check_dense(gpu, qa, sa, qb, sb, label=f"default mid shape {m}x{n}x{k}")
    d2, _ = H.run_dense(qa, sa, qb, sb, gpu)
    assert np.array_equal(H.d_bits(d), H.d_bits(d2))


@pytest.mark.parametrize("cfg", ["dense_64x64_w4_s8", "dense_64x32_w4_s4", "dense_128x128_w4_s2",
                                 "dense_64x32_w4_s6_triple"])
def test_split_k_back_to_back_shapes(gpu, cfg, monkeypatch):
    # calls with different split counts and tile counts in a row share the workspace
    monkeypatch.setenv("DG_FORCE_CONFIG", cfg)
    for splits, (m, n, k) in [("5", (64, 512, 1280)), ("2", (40, 1024, 512)), ("7", (64, 512, 1792))]:
        monkeypatch.setenv("DG_SPLIT_K", splits)
        check_dense(gpu, *dense_case(m, n, k, seed=11), label=f"back-to-back splits={splits}")


@pytest.mark.parametrize("cfg", [None, "kgrouped_256x256_w8_s2", "kgrouped_128x128_w4_s2", "kgrouped_128x256_w4_s2_sb"])
@pytest.mark.parametrize("m,n,sizes,k_total", [
    (300, 520, [256, 0, 640, 128], 1280),   # ragged tiles, an empty group, two unused slabs
    (64, 2112, [1024, 512], 1536),           # skinny M, N with a 64-row partial scale block
    (520, 300, [128], 128),                  # one group, one slab
    (512, 1024, [384, 640], 1024),           # 32 workgroups of 128 x 256 tiles: the XCD remap is active
])
def test_k_grouped(gpu, cfg, m, n, sizes, k_total, monkeypatch):
    if cfg:
        monkeypatch.setenv("DG_FORCE_CONFIG", cfg)
    x = W.draw_kgrouped(sizes, m, n, seed=m + n + k_total, k_total=k_total)
    qa, sa = oracle.quantize_a_1x128(x["a"])
    qb, sb = oracle.quantize_b_128x128(x["b"])
    print(f"[case] k-grouped {cfg} {m}x{n} sizes={sizes} k={k_total}", flush=True)
    d, flat = H.run_kgrouped(qa, sa, qb, sb, sizes, gpu)
    r = oracle.k_grouped_ref(qa, sa, qb, sb, sizes)
    got = H.d_float(d)
    for g in range(len(sizes)):
        if sizes[g] == 0:
            assert np.all(H.d_bits(d)[g] == 0), "an empty group must be written as +0"
        else:
            res = oracle.tolerance_check(got[g], r[g])
            assert res["ok"], (g, res)
    assert H.guard_untouched(flat, d.numel())


def test_k_grouped_device_side_clamping(gpu):
    # sizes are device values: negative counts as 0, a remainder below 128
    # is dropped, and the last group is cut off at K
    m, n, k_total = 96, 200, 768
    x = W.draw_kgrouped([k_total], m, n, seed=5)
    qa, sa = oracle.quantize_a_1x128(x["a"])
    qb, sb = oracle.quantize_b_128x128(x["b"])
    print("[case] k-grouped clamping", flush=True)
    d, flat = H.run_kgrouped(qa, sa, qb, sb, [-128, 300, 1024], gpu)
    r = oracle.k_grouped_ref(qa, sa, qb, sb, [0, 256, 512])
    got = H.d_float(d)
    assert np.all(H.d_bits(d)[0] == 0)
    for g in (1, 2):
        res = oracle.tolerance_check(got[g], r[g])
        assert res["ok"], (g, res)
    assert H.guard_untouched(flat, d.numel())



def bf16_bits(x):
    import torch
    return torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


@pytest.mark.parametrize("cfg", [None, "bf16_256x256_w8_s2", "bf16_128x128_w4_s2", "bf16_64x32_w4_s4",
                                 "bf16_64x64_w4_s3", "bf16_64x32_w4_s4_pair"])
@pytest.mark.parametrize("m,n,k", [(300, 520, 640), (64, 2112, 1024), (1, 16, 64), (520, 300, 128),
                                   (200, 2112, 512)])
def test_bf16_gemm(gpu, cfg, m, n, k, monkeypatch):
    if cfg:
        monkeypatch.setenv("DG_FORCE_CONFIG", cfg)
    x = W.draw_dense(m, n, k, seed=m + 2 * n + k)
    a, b = bf16_bits(x["a"]), bf16_bits(x["b"])
    print(f"[case] bf16 {cfg} {m}x{n}x{k}", flush=True)
    d, flat = H.run_bf16(a, b, gpu)
    r = oracle.bf16_gemm_nt_ref(a, b)
    res = oracle.tolerance_check(H.d_float(d), r)
    assert res["ok"], res
    assert H.guard_untouched(flat, d.numel())


@pytest.mark.parametrize("m,n,k", [(64, 4200, 512), (64, 9000, 256), (64, 5000, 3072), (100, 5000, 1024),
                                   (128, 7168, 2048)])
def test_bf16_default_tile_regions(gpu, m, n, k):
    """Each branch of the BF16 small-M tile rules at its default choice:
    64 x 32 up to N 8192 with short K, 64 x 64 for wider N, longer K, or
    M up to 128 with K up to 2048."""
    x = W.draw_dense(m, n, k, seed=m + 3 * n + k)
    a, b = bf16_bits(x["a"]), bf16_bits(x["b"])
    print(f"[case] bf16 default {m}x{n}x{k}", flush=True)
    d, flat = H.run_bf16(a, b, gpu)
    res = oracle.tolerance_check(H.d_float(d), oracle.bf16_gemm_nt_ref(a, b))
    assert res["ok"], res
    assert H.guard_untouched(flat, d.numel())


@pytest.mark.parametrize("cfg", ["bf16_64x32_w4_s4", "bf16_64x32_w4_s4_pair"])
def test_bf16_gemm_forced_split_k(gpu, cfg, monkeypatch):
    monkeypatch.setenv("DG_FORCE_CONFIG", cfg)
    monkeypatch.setenv("DG_SPLIT_K", "5")
    m, n, k = 48, 200, 1280
    x = W.draw_dense(m, n, k, seed=3)
    a, b = bf16_bits(x["a"]), bf16_bits(x["b"])
    print("[case] bf16 split-K 5", flush=True)
    d, flat = H.run_bf16(a, b, gpu)
    res = oracle.tolerance_check(H.d_float(d), oracle.bf16_gemm_nt_ref(a, b))
    assert res["ok"], res
    d2, _ = H.run_bf16(a, b, gpu)
    assert np.array_equal(H.d_bits(d), H.d_bits(d2))


@pytest.mark.parametrize("cfg,m,n,k", [
    ("dense_256x256_w8_s2", 1024, 1024, 512),   # 16 tiles: the grid is a multiple of 8, the XCD remap is active
    ("dense_128x256_w4_s2_sb", 1024, 1024, 512),
    ("dense_256x256_w8_s2", 768, 2048, 384),    # 24 tiles
    ("dense_128x256_w4_s2_sb", 768, 2048, 384),  # 48 tiles
    ("dense_128x256_w4_s2_sb", 1000, 2000, 640),  # ragged rows and columns, 64 tiles
    ("dense_256x224_w8_s2", 1024, 1792, 512),   # 32 tiles, every wave column split across two B scale blocks
])
def test_dense_default_tiles_with_xcd_remap(gpu, cfg, m, n, k, monkeypatch):
    """The large-shape default tiles, element by element, at shapes whose
    workgroup count is a multiple of the 8 XCDs, so that the XCD-aware block
    remap and the grouped raster are not the identity."""
    monkeypatch.setenv("DG_FORCE_CONFIG", cfg)
    check_dense(gpu, *dense_case(m, n, k, seed=13), label=f"{cfg} {m}x{n}x{k}")


def test_contiguous_default_tile_with_xcd_remap(gpu, monkeypatch):
    """contig_128x256_w4_s2_sb (the 4-expert default) on 8 experts x 128 rows,
    N 512: 16 workgroups, a multiple of the 8 XCDs; every element against the
    oracle."""
    monkeypatch.setenv("DG_FORCE_CONFIG", "contig_128x256_w4_s2_sb")
    group_rows = [128] * 8
    n, k = 512, 512
    x = W.draw_contiguous(group_rows, n, k, seed=14)
    qa, sa = oracle.quantize_a_1x128(x["a"])
    qbs = [oracle.quantize_b_128x128(x["b"][g]) for g in range(len(group_rows))]
    qb = np.stack([q for q, _ in qbs])
    sb = np.stack([s for _, s in qbs])
    print("[case] contig_128x256_w4_s2_sb 8x128 rows", flush=True)
    d, flat = H.run_contiguous(qa, sa, qb, sb, x["m_indices"], gpu)
    r, valid = oracle.grouped_contiguous_ref(qa, sa, qb, sb, x["m_indices"])
    assert valid.all()
    res = oracle.tolerance_check(H.d_float(d), r)
    assert res["ok"], res
    assert H.guard_untouched(flat, d.numel())
