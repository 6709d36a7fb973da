"""GPU parity of the FP4 (e2m1) path against the oracle.

* The FP4 quantisers, codes (packed two per byte) and scales bit for bit,
  including blocks whose scale is exactly 1 so that x / s falls on every
  rounding tie of the e2m1 grid.
* The FP4 GEMM element by element against oracle.fp4_gemm_nt_ref on
  oracle-quantised operands, every FP4 configuration, ragged M and N tails,
  forced split-K, under the acceptance rule |d - r| <= 8e-3 |r| + 1e-3 rms.
  (e2m1 products carry at most 3 significant bits and span a narrow range,
  so the MFMA's in-slab sums are exact; only the fp32 promotion and the bf16
  output round.)
* Closed form: all-ones operands with unit scales give exactly K.
* The FP4 workload at full size, quantised on the GPU, checked on sampled
  rows.
"""

import numpy as np
import pytest
import torch

import fp8_block_scaled_nt_amd as dg
import oracle
import workloads as W
from tests import gpu_harness as H

pytestmark = pytest.mark.gpu

FP4_CONFIGS = ["fp4_256x256_w8_s2", "fp4_128x128_w4_s2", "fp4_64x32_w4_s4", "fp4_64x64_w4_s3", "fp4_64x32_w4_s6_triple",
               "fp4_64x64_w4_s4_pair"]


def with_ties(x):
    """Make block (0, slab 0) have amax exactly 6 (scale 1) and put every
    e2m1 rounding tie and its neighbours in it."""
    ties = np.array([6.0, 0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, -0.25, -0.75, -1.25, -1.75, -2.5, -3.5, -5.0,
                     0.0, -0.0, 5.999, 0.2499, 0.7501, 1e-30], np.float32)
    x[0, :ties.size] = ties
    x[0, ties.size:128] = np.clip(x[0, ties.size:128], -5.9, 5.9)
    return x


@pytest.mark.parametrize("m,k", [(1, 128), (37, 384), (128, 1024), (64, 7168), (200, 256)])
def test_quant_a_fp4_bitexact(gpu, m, k):
    rng = np.random.default_rng(m * 3 + k)
    x = with_ties(rng.standard_normal((m, k), dtype=np.float32))
    print(f"[case] quant_a_fp4 {m}x{k}", flush=True)
    q, sfa = dg.quantize_a_1x128_fp4(H.f32_to_device(x, gpu))
    torch.cuda.synchronize()
    q_ref, s_ref = oracle.quantize_a_1x128_fp4(x)
    assert np.array_equal(q.cpu().numpy(), q_ref)
    s_dev = sfa.cpu().numpy()
    assert np.array_equal(H.slab_major_to_logical(s_dev, m), s_ref)
    assert s_ref[0, 0] == 1.0
    assert np.all(s_dev[:, m:] == 0)


@pytest.mark.parametrize("n,k", [(128, 128), (200, 384), (2112, 512), (1, 256)])
def test_quant_b_fp4_bitexact(gpu, n, k):
    rng = np.random.default_rng(n + 2 * k)
    x = rng.standard_normal((n, k), dtype=np.float32) * np.float32(0.02)
    print(f"[case] quant_b_fp4 {n}x{k}", flush=True)
    q, sfb = dg.quantize_b_128x128_fp4(H.f32_to_device(x, gpu))
    torch.cuda.synchronize()
    q_ref, s_ref = oracle.quantize_b_128x128_fp4(x)
    assert np.array_equal(q.cpu().numpy(), q_ref)
    assert np.array_equal(sfb.cpu().numpy(), s_ref)


def fp4_case(m, n, k, seed, b_std=1.0):
    x = W.draw_dense(m, n, k, seed=seed, b_std=b_std)
    pa, sa = oracle.quantize_a_1x128_fp4(x["a"])
    pb, sb = oracle.quantize_b_128x128_fp4(x["b"])
    return pa, sa, pb, sb


def check_fp4(gpu, pa, sa, pb, sb, label):
    print(f"[case] {label}", flush=True)
    d, flat = H.run_fp4(pa, sa, pb, sb, gpu)
    r = oracle.fp4_gemm_nt_ref(pa, sa, pb, sb)
    res = oracle.tolerance_check(H.d_float(d), r)
    assert res["ok"], (label, res)
    assert H.guard_untouched(flat, d.numel()), label
    return d, res


@pytest.mark.parametrize("m,n,k", [(128, 512, 1024), (1, 16, 256), (17, 40, 256), (200, 176, 512),
                                   (64, 2112, 512), (300, 520, 768), (513, 257, 256), (200, 2112, 1024),
                                   (384, 2112, 512),
                                   # each branch of the small-M tile rules: 64 x 32 at moderate N and
                                   # short K, 64 x 64 for wide N, long K or many tiles of short K
                                   (64, 3000, 2048), (64, 9000, 512), (64, 4200, 4096), (128, 5000, 2048),
                                   (100, 3000, 4096), (128, 17000, 512)])
def test_fp4_default_selection(gpu, m, n, k):
    check_fp4(gpu, *fp4_case(m, n, k, seed=m + n + k), label=f"fp4 {m}x{n}x{k}")


@pytest.mark.parametrize("cfg", FP4_CONFIGS)
@pytest.mark.parametrize("m,n,k", [(300, 520, 768), (64, 200, 512), (520, 300, 256)])
def test_fp4_every_config(gpu, cfg, m, n, k, monkeypatch):
    monkeypatch.setenv("DG_FORCE_CONFIG", cfg)
    check_fp4(gpu, *fp4_case(m, n, k, seed=3), label=f"{cfg} {m}x{n}x{k}")


@pytest.mark.parametrize("cfg", ["fp4_64x32_w4_s4", "fp4_64x32_w4_s6_triple"])
@pytest.mark.parametrize("splits", [2, 3, 5])
def test_fp4_forced_split_k(gpu, splits, cfg, monkeypatch):
    monkeypatch.setenv("DG_FORCE_CONFIG", cfg)
    monkeypatch.setenv("DG_SPLIT_K", str(splits))
    d, _ = check_fp4(gpu, *fp4_case(64, 200, 2560, seed=splits), label=f"fp4 split-K {splits}")
    d2, _ = H.run_fp4(*fp4_case(64, 200, 2560, seed=splits), gpu)
    assert np.array_equal(H.d_bits(d), H.d_bits(d2))  # deterministic fix-up


def test_fp4_unit_scale_exact_values(gpu):
    m, n, k = 96, 144, 1024
    ones_a = np.full((m, k // 2), 0x22, np.uint8)  # two codes 2 = 1.0 per byte
    ones_b = np.full((n, k // 2), 0x22, np.uint8)
    d, _ = H.run_fp4(ones_a, np.ones((m, k // 128), np.float32), ones_b, np.ones((2, k // 128), np.float32), gpu)
    assert np.all(H.d_float(d) == k)


def test_fp4_full_size_sampled(gpu):
    name = "fp4_dense_4096x7168x16384"
    s = W.WORKLOADS[name].shape
    m, n, k = s["m"], s["n"], s["k"]
    x = W.draw(name)
    print(f"[case] {name}: quantise + GEMM on GPU", flush=True)
    qa, sfa = dg.quantize_a_1x128_fp4(H.f32_to_device(x["a"], gpu))
    qb, sfb = dg.quantize_b_128x128_fp4(H.f32_to_device(x["b"], gpu))
    d, flat = H.sentinel_bf16((m, n), gpu, guard=4096)
    dg.fp4_gemm_nt((qa, sfa), (qb, sfb), d)
    torch.cuda.synchronize()
    assert H.guard_untouched(flat, d.numel())
    rng = np.random.default_rng(41)
    rows = np.unique(np.concatenate([[0, m - 1], rng.integers(0, m, 6)]))
    qa_r, sa_r = oracle.quantize_a_1x128_fp4(x["a"][rows])
    assert np.array_equal(qa.cpu().numpy()[rows], qa_r)
    qb_r, sb_r = oracle.quantize_b_128x128_fp4(x["b"])
    assert np.array_equal(qb.cpu().numpy(), qb_r)
    assert np.array_equal(sfb.cpu().numpy(), sb_r)
    r = oracle.fp4_gemm_nt_ref(qa_r, sa_r, qb_r, sb_r)
    got = d.float()[torch.from_numpy(rows).to(gpu)].cpu().numpy().astype(np.float64)
    res = oracle.tolerance_check(got, r)
    assert res["ok"], res
