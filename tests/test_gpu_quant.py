"""GPU quantisers against the oracle quantisers: codes and scales bit for bit.

The e4m3 code is an integer decided by floating point, so both sides decide
it the same way: fp32 amax, fp32 correctly rounded division, nearest-even
rounding onto the e4m3 grid with saturation.
"""

import numpy as np
import pytest
import torch

import fp8_block_scaled_nt_amd as dg
import oracle
import workloads as W
from tests import gpu_harness as H

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("m,k,std", [(1, 128, 1.0), (37, 384, 3.0), (128, 1024, 1.0), (64, 7168, 1.0),
                                     (5, 256, 1e-6)])
def test_quant_a_bitexact(gpu, m, k, std):
    rng = np.random.default_rng(m * 7 + k)
    x = (rng.standard_normal((m, k), dtype=np.float32) * np.float32(std))
    x[0, :5] = [0.0, -0.0, 448.0, 1e-30, -3.5]
    print(f"[case] quant_a {m}x{k}", flush=True)
    q, sfa = dg.quantize_a_1x128(H.f32_to_device(x, gpu))
    torch.cuda.synchronize()
    q_ref, s_ref = oracle.quantize_a_1x128(x)
    assert np.array_equal(q.view(torch.uint8).cpu().numpy(), q_ref)
    s_dev = sfa.cpu().numpy()
    assert np.array_equal(H.slab_major_to_logical(s_dev, m), s_ref)
    assert np.all(s_dev[:, m:] == 0)


@pytest.mark.parametrize("n,k,std", [(128, 128, 0.02), (200, 384, 0.02), (2112, 512, 0.02), (1, 256, 1.0)])
def test_quant_b_bitexact(gpu, n, k, std):
    rng = np.random.default_rng(n + k)
    x = rng.standard_normal((n, k), dtype=np.float32) * np.float32(std)
    print(f"[case] quant_b {n}x{k}", flush=True)
    q, sfb = dg.quantize_b_128x128(H.f32_to_device(x, gpu))
    torch.cuda.synchronize()
    q_ref, s_ref = oracle.quantize_b_128x128(x)
    assert np.array_equal(q.view(torch.uint8).cpu().numpy(), q_ref)
    assert np.array_equal(sfb.cpu().numpy(), s_ref)


def test_quant_then_gemm_small_workload(gpu):
    # the whole path on the GPU (quantise A and B, GEMM) against the oracle path
    x = W.draw("dense_128x512x1024")
    qa, sfa = dg.quantize_a_1x128(H.f32_to_device(x["a"], gpu))
    qb, sfb = dg.quantize_b_128x128(H.f32_to_device(x["b"], gpu))
    d, _ = H.sentinel_bf16((128, 512), gpu)
    dg.fp8_gemm_nt((qa, sfa), (qb, sfb), d)
    torch.cuda.synchronize()
    qa_r, sa_r = oracle.quantize_a_1x128(x["a"])
    qb_r, sb_r = oracle.quantize_b_128x128(x["b"])
    r = oracle.gemm_nt_ref(qa_r, sa_r, qb_r, sb_r)
    res = oracle.tolerance_check(H.d_float(d), r)
    assert res["ok"], res
