"""The allocation-free dense entry point (dg_fp8_gemm_nt_noalloc), called
through the C ABI, gives the same D as dg_fp8_gemm_nt and matches the oracle,
on two calls in a row (the second smaller, so stale scratch contents of the
first would show), for the skinny split-K kernel and the tiled split-K
kernel; a call that needs more scratch than the static array holds is
refused before anything is enqueued."""

import ctypes

import numpy as np
import pytest
import torch

import fp8_block_scaled_nt_amd as dg
import oracle
import workloads as W
from tests import gpu_harness as H

pytestmark = pytest.mark.gpu

DG_ERR_UNSUPPORTED_SHAPE = 2


def case(m, n, k, seed, b_std):
    x = W.draw_dense(m, n, k, seed=seed, b_std=b_std)
    qa, sa = oracle.quantize_a_1x128(x["a"])
    qb, sb = oracle.quantize_b_128x128(x["b"])
    return qa, sa, qb, sb


def run(entry, c, gpu):
    qa, sa, qb, sb = c
    m, k = qa.shape
    n = qb.shape[0]
    a = H.codes_to_device(qa, gpu)
    b = H.codes_to_device(qb, gpu)
    sfa = H.f32_to_device(H.slab_major(sa), gpu)
    sfb = H.f32_to_device(sb, gpu)
    d, flat = H.sentinel_bf16((m, n), gpu, 256)
    st = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    status = getattr(dg.lib(), entry)(H._ptr(a), H._ptr(sfa), H._ptr(b), H._ptr(sfb), H._ptr(d), m, n, k, st)
    torch.cuda.synchronize()
    return status, d, flat


SKINNY_TILE_BYTES = 64 * 32 * 4  # one fp32 partial tile of the skinny kernel


@pytest.mark.parametrize("shapes", [
    # the skinny split-K kernel (m <= 16, 14 and 12 K-slab units per run), then a smaller call
    [(8, 2112, 7168, 0.02), (5, 1800, 7168, 1.0)],
    # the tiled split-K kernel on the decode shape, then a smaller tiled call
    [(64, 2112, 7168, 0.02), (17, 520, 1280, 1.0)],
    # tiled split-K with 64 x 32 tiles on a small dense shape, then smaller
    [(128, 512, 1024, 1.0), (96, 200, 512, 1.0)],
], ids=["skinny", "tiled-decode", "tiled-small"])
def test_noalloc_matches_default_entry_point(gpu, shapes, monkeypatch):
    if shapes[0][0] <= 16:
        # the skinny split-K kernel, by name (the tiled kernel is the default
        # at these sizes): 66 and 57 tiles of 64 x 32, 5 and 6 partial slots each
        monkeypatch.setenv("DG_FORCE_CONFIG", "skinny_64x32_w16_stagea")
        assert dg.dense_workspace_size(8, 2112, 7168) == 66 * 5 * SKINNY_TILE_BYTES
        assert dg.dense_workspace_size(5, 1800, 7168) == 57 * 6 * SKINNY_TILE_BYTES
    for i, (m, n, k, b_std) in enumerate(shapes):
        c = case(m, n, k, seed=40 + i, b_std=b_std)
        print(f"[case] noalloc {m}x{n}x{k}", flush=True)
        s1, d1, f1 = run("dg_fp8_gemm_nt_noalloc", c, gpu)
        s0, d0, _ = run("dg_fp8_gemm_nt", c, gpu)
        assert s1 == 0 and s0 == 0, (s1, s0, dg.lib().dg_last_error_message())
        assert np.array_equal(H.d_bits(d1), H.d_bits(d0)), f"{m}x{n}x{k}: differs from dg_fp8_gemm_nt"
        res = oracle.tolerance_check(H.d_float(d1), oracle.gemm_nt_ref(*c))
        assert res["ok"], res
        assert H.guard_untouched(f1, d1.numel())


def test_noalloc_refuses_oversized_scratch(gpu):
    # 4096 x 896 x 2048: 224 tiles of 128 x 128 split 2 ways, 29 MiB of partials
    c = case(4096, 896, 2048, seed=50, b_std=1.0)
    status, d, _ = run("dg_fp8_gemm_nt_noalloc", c, gpu)
    assert status == DG_ERR_UNSUPPORTED_SHAPE
    assert b"static" in dg.lib().dg_last_error_message()
    assert np.all(H.d_bits(d) == H.SENTINEL)  # nothing was enqueued
