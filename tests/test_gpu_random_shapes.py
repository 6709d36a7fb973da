"""Seeded random shapes for every entry point, against the oracle.

Each case draws its sizes from a fixed seed (ragged M and N, K anywhere in
its allowed steps, empty and clamped groups), quantises with the oracle and
runs the library at its default configuration.  The checks are those of
the per-entry-point parity tests: the acceptance rule on valid outputs,
sentinels elsewhere, untouched guard bands."""

import os

import numpy as np
import pytest

import oracle
import workloads as W
from tests import gpu_harness as H

pytestmark = pytest.mark.gpu

# DG_TEST_SEED draws another set of shapes (the default set is the one the
# suite runs)
RNG_SEED = int(os.environ.get("DG_TEST_SEED", "20261203"))


def shapes(kind, count):
    rng = np.random.default_rng(RNG_SEED + sum(map(ord, kind)))
    out = []
    for _ in range(count):
        m = int(rng.integers(1, 700))
        n = int(rng.integers(1, 700))
        kslabs = int(rng.integers(1, 9))
        out.append((m, n, kslabs))
    return out


@pytest.mark.parametrize("m,n,kslabs", shapes("dense", 12))
def test_random_dense(gpu, m, n, kslabs):
    k = 128 * kslabs
    x = W.draw_dense(m, n, k, seed=m * 7 + n)
    qa, sa = oracle.quantize_a_1x128(x["a"])
    qb, sb = oracle.quantize_b_128x128(x["b"])
    print(f"[case] random dense {m}x{n}x{k}", flush=True)
    d, flat = H.run_dense(qa, sa, qb, sb, gpu)
    res = oracle.tolerance_check(H.d_float(d), oracle.gemm_nt_ref(qa, sa, qb, sb))
    assert res["ok"], res
    assert H.guard_untouched(flat, d.numel())


def small_m_shapes(count):
    """Decode-like shapes: m 1..16 and N x K with 3100-4000 units of a 64x32
    tile and a 128-wide slab, the range the skinny kernel was written for."""
    rng = np.random.default_rng(RNG_SEED + 16)
    out = []
    for _ in range(count):
        m = int(rng.integers(1, 17))
        n = int(rng.integers(1000, 4200))
        tiles = (n + 31) // 32
        lo, hi = -(-3100 // tiles), 4000 // tiles
        out.append((m, n, int(rng.integers(lo, hi + 1))))
    return out


@pytest.mark.parametrize("m,n,kslabs", small_m_shapes(6))
@pytest.mark.parametrize("cfg", [None, "skinny_64x32_w16_stagea", "dense_64x32_w4_s4", "dense_64x32_w4_s6_triple"])
def test_random_small_m(gpu, m, n, kslabs, cfg, monkeypatch):
    if cfg:
        monkeypatch.setenv("DG_FORCE_CONFIG", cfg)
    k = 128 * kslabs
    x = W.draw_dense(m, n, k, seed=m * 11 + n)
    qa, sa = oracle.quantize_a_1x128(x["a"])
    qb, sb = oracle.quantize_b_128x128(x["b"])
    print(f"[case] random small m {m}x{n}x{k} {cfg}", flush=True)
    d, flat = H.run_dense(qa, sa, qb, sb, gpu)
    res = oracle.tolerance_check(H.d_float(d), oracle.gemm_nt_ref(qa, sa, qb, sb))
    assert res["ok"], res
    assert H.guard_untouched(flat, d.numel())


@pytest.mark.parametrize("m,n,kslabs", shapes("fp4", 8))
def test_random_fp4(gpu, m, n, kslabs):
    k = 256 * ((kslabs + 1) // 2)
    x = W.draw_dense(m, n, k, seed=m * 5 + n)
    pa, sa = oracle.quantize_a_1x128_fp4(x["a"])
    pb, sb = oracle.quantize_b_128x128_fp4(x["b"])
    print(f"[case] random fp4 {m}x{n}x{k}", flush=True)
    d, flat = H.run_fp4(pa, sa, pb, sb, gpu)
    res = oracle.tolerance_check(H.d_float(d), oracle.fp4_gemm_nt_ref(pa, sa, pb, sb))
    assert res["ok"], res
    assert H.guard_untouched(flat, d.numel())


@pytest.mark.parametrize("m,n,kslabs", shapes("bf16", 8))
def test_random_bf16(gpu, m, n, kslabs):
    k = 64 * kslabs
    rng = np.random.default_rng(m + 3 * n)
    a = oracle_bf16_bits(rng.standard_normal((m, k)))
    b = oracle_bf16_bits(rng.standard_normal((n, k)))
    print(f"[case] random bf16 {m}x{n}x{k}", flush=True)
    d, flat = H.run_bf16(a, b, gpu)
    res = oracle.tolerance_check(H.d_float(d), oracle.bf16_gemm_nt_ref(a, b))
    assert res["ok"], res
    assert H.guard_untouched(flat, d.numel())


def oracle_bf16_bits(x):
    """bf16 bit patterns of fp32 values (round to nearest even), as inputs."""
    f = np.asarray(x, np.float32).view(np.uint32).astype(np.uint64)
    return ((f + 0x7FFF + ((f >> 16) & 1)) >> 16).astype(np.uint16)


@pytest.mark.parametrize("case", range(6))
def test_random_grouped(gpu, case):
    rng = np.random.default_rng(RNG_SEED + 100 + case)
    g = int(rng.integers(1, 6))
    n = int(rng.integers(1, 600))
    k = 128 * int(rng.integers(1, 6))
    # masked
    max_m = int(rng.integers(1, 400))
    mm = rng.integers(-2, max_m + 40, g).astype(np.int32)
    x = W.draw_masked(g, max_m, n, k, seed=case, masked_m=mm)
    qas = [oracle.quantize_a_1x128(x["a"][i]) for i in range(g)]
    qbs = [oracle.quantize_b_128x128(x["b"][i]) for i in range(g)]
    qa, sa = np.stack([q for q, _ in qas]), np.stack([s for _, s in qas])
    qb, sb = np.stack([q for q, _ in qbs]), np.stack([s for _, s in qbs])
    print(f"[case] random masked g={g} max_m={max_m} n={n} k={k} counts={mm.tolist()}", flush=True)
    d, flat = H.run_masked(qa, sa, qb, sb, mm, gpu)
    r, valid = oracle.grouped_masked_ref(qa, sa, qb, sb, mm)
    res = oracle.tolerance_check(H.d_float(d), r, valid[:, :, None])
    assert res["ok"], res
    assert np.all(H.d_bits(d)[~valid] == H.SENTINEL)
    assert H.guard_untouched(flat, d.numel())
    # contiguous (segments padded to 128 rows)
    rows = [int(v) for v in rng.integers(0, 300, g)]
    xc = W.draw_contiguous(rows, n, k, seed=case)
    qa_c, sa_c = oracle.quantize_a_1x128(xc["a"])
    qbs = [oracle.quantize_b_128x128(xc["b"][i]) for i in range(g)]
    qb_c, sb_c = np.stack([q for q, _ in qbs]), np.stack([s for _, s in qbs])
    idx = xc["m_indices"]
    print(f"[case] random contiguous rows={rows} n={n} k={k}", flush=True)
    d, flat = H.run_contiguous(qa_c, sa_c, qb_c, sb_c, idx, gpu)
    r, valid = oracle.grouped_contiguous_ref(qa_c, sa_c, qb_c, sb_c, idx)
    res = oracle.tolerance_check(H.d_float(d), r, valid[:, None])
    assert res["ok"], res
    assert np.all(H.d_bits(d)[~valid] == H.SENTINEL)
    assert H.guard_untouched(flat, d.numel())


@pytest.mark.parametrize("case", range(4))
def test_random_k_grouped(gpu, case):
    rng = np.random.default_rng(RNG_SEED + 200 + case)
    g = int(rng.integers(1, 5))
    m = int(rng.integers(1, 400))
    n = int(rng.integers(1, 400))
    sizes = [128 * int(v) for v in rng.integers(0, 4, g)]
    x = W.draw_kgrouped(sizes, m, n, seed=case, k_total=max(sum(sizes), 128))
    qa, sa = oracle.quantize_a_1x128(x["a"])
    qb, sb = oracle.quantize_b_128x128(x["b"])
    print(f"[case] random k-grouped m={m} n={n} sizes={sizes}", flush=True)
    d, flat = H.run_kgrouped(qa, sa, qb, sb, sizes, gpu)
    r = oracle.k_grouped_ref(qa, sa, qb, sb, sizes)
    res = oracle.tolerance_check(H.d_float(d), r)
    assert res["ok"], res
    assert H.guard_untouched(flat, d.numel())


@pytest.mark.parametrize("case", range(4))
def test_random_swiglu(gpu, case):
    from tests import test_gpu_swiglu as SW
    rng = np.random.default_rng(RNG_SEED + 300 + case)
    g = int(rng.integers(1, 5))
    max_m = int(rng.integers(1, 300))
    inter = 128 * int(rng.integers(1, 4))
    k = 128 * int(rng.integers(1, 5))
    mm = rng.integers(-1, max_m + 20, g).astype(np.int32)
    qa, sa, qb, sb, mm = SW.workload_case(g, max_m, inter, k, mm, seed=case)
    print(f"[case] random swiglu g={g} max_m={max_m} I={inter} k={k} counts={mm.tolist()}", flush=True)
    hq, hs, fq, fs = H.run_swiglu(qa, sa, qb, sb, mm, gpu)
    assert H.swiglu_guards_untouched(fq, fs, hq.size, hs.size)
    code_share, _ = SW.check_call(hq, hs, qa, sa, qb, sb, mm, SW.rule_tol, f"random swiglu {case}", 0.1)
    assert code_share >= 0.98, code_share
