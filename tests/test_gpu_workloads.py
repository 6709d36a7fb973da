"""The named workloads at full size, run the way bench.py runs them:
fp32 inputs drawn by `workloads`, quantised on the GPU by the library, the
GEMM with the library's default tile choice.

The oracle cannot compute the full outputs in seconds, so it computes sampled
entries one by one: it quantises (on the CPU, from the same fp32 draws) the
A rows and B 128-row blocks those entries need, checks that the GPU's codes
and scales for them are bit-identical, and evaluates each sampled entry in
fp64.  The tolerance's rms term uses the sample's rms (the rms of the whole
output is not available without the whole output; over a sample of a few
hundred entries drawn from every tile row and column it is within a few
percent of it, and the term only matters for entries near zero).  The two
dense shapes the oracle finishes in seconds (128 x 512 x 1024 and the
64 x 2112 x 7168 decode shape) are compared in full instead.  Every output
element is checked on the device to have been written (no 0xFFFF sentinel
left) for the dense, contiguous and K-grouped workloads; for the masked
workload every row past masked_m is checked to hold the sentinel; for all of
them the guard band after D must be untouched.
"""

import numpy as np
import pytest
import torch

import fp8_block_scaled_nt_amd as dg
import oracle
import workloads as W
from tests import gpu_harness as H

pytestmark = pytest.mark.gpu


def pick(rng, hi, count):
    return np.unique(rng.integers(0, hi, count))


def plan_cols(rng, n, blocks, per_block):
    nb = (n + 127) // 128
    bsel = np.unique(np.concatenate([[nb - 1], rng.integers(0, nb, blocks)]))
    cols = []
    for b in bsel:
        lo, hi = b * 128, min(n, b * 128 + 128)
        cols.append(rng.integers(lo, hi, per_block))
    return bsel, np.concatenate(cols)


def oracle_b_block(xb, blk):
    """Oracle-quantised 128-row block blk of fp32 weights xb (rows, codes, scales)."""
    lo, hi = blk * 128, min(xb.shape[0], blk * 128 + 128)
    q, s = oracle.quantize_b_128x128(xb[lo:hi])
    return lo, hi, q, s[0]


def check_sampled(label, d_sel, qa_rows, sa_rows, b_codes, b_scales, rows_ix, cols_ix):
    """d_sel[i, j] is the GPU value at (row i, col j) of the sample grid."""
    ri, cj = np.meshgrid(np.arange(len(rows_ix)), np.arange(len(cols_ix)), indexing="ij")
    a_codes = qa_rows[ri.ravel()]
    a_sc = sa_rows[ri.ravel()]
    bq = b_codes[cj.ravel()]
    bs = b_scales[cj.ravel()]
    r = oracle.gemm._entries(a_codes, a_sc.astype(np.float64), bq, bs.astype(np.float64))
    res = oracle.tolerance_check(d_sel.ravel(), r)
    assert res["ok"], (label, res)
    return res


def dense_case(gpu, name, whole=False):
    """Full-size dense workload; with whole=True every output element is
    compared with the oracle (shapes the oracle finishes in seconds)."""
    w = W.WORKLOADS[name]
    m, n, k = w.shape["m"], w.shape["n"], w.shape["k"]
    x = W.draw(name)
    print(f"[case] {name}: quantise + GEMM on GPU", flush=True)
    qa, sfa = dg.quantize_a_1x128(H.f32_to_device(x["a"], gpu))
    qb, sfb = dg.quantize_b_128x128(H.f32_to_device(x["b"], gpu))
    d, flat = H.sentinel_bf16((m, n), gpu, guard=4096)
    dg.fp8_gemm_nt((qa, sfa), (qb, sfb), d)
    torch.cuda.synchronize()
    assert H.guard_untouched(flat, d.numel())
    # every element was written (results are finite, the 0xFFFF sentinel is a NaN)
    assert not bool((d.view(torch.int16) == -1).any())
    if whole:
        qa_r, sa_r = oracle.quantize_a_1x128(x["a"])
        qb_r, sb_r = oracle.quantize_b_128x128(x["b"])
        assert np.array_equal(qa.view(torch.uint8).cpu().numpy(), qa_r)
        assert np.array_equal(qb.view(torch.uint8).cpu().numpy(), qb_r)
        res = oracle.tolerance_check(H.d_float(d), oracle.gemm_nt_ref(qa_r, sa_r, qb_r, sb_r))
        assert res["ok"], (name, res)
        return res
    rng = np.random.default_rng(99)
    rows = np.unique(np.concatenate([[0, m - 1], pick(rng, m, 12)]))
    bsel, cols = plan_cols(rng, n, 3, 24)
    qa_r, sa_r = oracle.quantize_a_1x128(x["a"][rows])
    assert np.array_equal(qa.view(torch.uint8)[torch.from_numpy(rows).to(gpu)].cpu().numpy(), qa_r)
    sfa_dev = sfa.cpu().numpy()
    assert np.array_equal(sfa_dev[:, rows].T, sa_r)
    b_codes = np.zeros((len(cols), k), np.uint8)
    b_scales = np.zeros((len(cols), k // 128), np.float32)
    qb_host_rows = qb.view(torch.uint8)[torch.from_numpy(cols).to(gpu)].cpu().numpy()
    sfb_dev = sfb.cpu().numpy()
    for blk in bsel:
        lo, hi, q, s = oracle_b_block(x["b"], blk)
        sel = (cols >= lo) & (cols < hi)
        b_codes[sel] = q[cols[sel] - lo]
        b_scales[sel] = s
        assert np.array_equal(sfb_dev[blk], s)
    assert np.array_equal(qb_host_rows, b_codes)
    d_sel = d.float()[torch.from_numpy(rows).to(gpu)][:, torch.from_numpy(cols).to(gpu)].cpu().numpy()
    return check_sampled(name, d_sel.astype(np.float64), qa_r, sa_r, b_codes, b_scales, rows, cols)


def test_dense_small_full(gpu):
    dense_case(gpu, "dense_128x512x1024", whole=True)


def test_dense_decode_full(gpu):
    dense_case(gpu, "dense_decode_64x2112x7168", whole=True)


def test_dense_decode_small_batch_full(gpu):
    # m = 8: 64 x 32 tiles with 8 valid rows, split 7 ways
    assert dg.dense_workspace_size(8, 2112, 7168) == 66 * 7 * 64 * 32 * 4
    dense_case(gpu, "dense_decode_8x2112x7168", whole=True)


def test_dense_large_full(gpu):
    dense_case(gpu, "dense_large_4096x7168x16384")


def test_dense_shard_n_full(gpu):
    dense_case(gpu, "dense_shard_n_4096x896x16384")


def test_dense_shard_m_full(gpu):
    dense_case(gpu, "dense_shard_m_512x7168x16384")


def test_contiguous_full(gpu):
    name = "moe_contiguous_4x8192_n4096_k7168"
    w = W.WORKLOADS[name]
    n, k = w.shape["n"], w.shape["k"]
    x = W.draw(name)
    idx = x["m_indices"]
    m, g = idx.size, len(w.shape["group_rows"])
    print(f"[case] {name}: quantise + GEMM on GPU", flush=True)
    qa, sfa = dg.quantize_a_1x128(H.f32_to_device(x["a"], gpu))
    qb, sfb = dg.quantize_b_128x128(H.f32_to_device(x["b"], gpu))
    d, flat = H.sentinel_bf16((m, n), gpu, guard=4096)
    dg.m_grouped_fp8_gemm_nt_contiguous((qa, sfa), (qb, sfb), d, torch.from_numpy(idx).to(gpu))
    torch.cuda.synchronize()
    assert H.guard_untouched(flat, d.numel())
    assert not bool((d.view(torch.int16) == -1).any())  # no padding rows: every element written
    rng = np.random.default_rng(98)
    sfb_dev = sfb.cpu().numpy()
    for e in range(g):
        seg = np.nonzero(idx == e)[0]
        rows = np.unique(np.concatenate([[seg[0], seg[-1]], rng.choice(seg, 6)]))
        bsel, cols = plan_cols(rng, n, 2, 16)
        qa_r, sa_r = oracle.quantize_a_1x128(x["a"][rows])
        assert np.array_equal(qa.view(torch.uint8)[torch.from_numpy(rows).to(gpu)].cpu().numpy(), qa_r)
        b_codes = np.zeros((len(cols), k), np.uint8)
        b_scales = np.zeros((len(cols), k // 128), np.float32)
        for blk in bsel:
            lo, hi, q, s = oracle_b_block(x["b"][e], blk)
            sel = (cols >= lo) & (cols < hi)
            b_codes[sel] = q[cols[sel] - lo]
            b_scales[sel] = s
            assert np.array_equal(sfb_dev[e, blk], s)
        d_sel = d.float()[torch.from_numpy(rows).to(gpu)][:, torch.from_numpy(cols).to(gpu)].cpu().numpy()
        check_sampled(f"{name} expert {e}", d_sel.astype(np.float64), qa_r, sa_r, b_codes, b_scales, rows, cols)


@pytest.mark.parametrize("name,total", [("moe_masked_16x256_n4096_k7168", 2067),
                                        ("moe_masked_16x256_c64_n4096_k7168", 518)])
def test_masked_full(gpu, name, total):
    # the typical count passed as expected_m picks the ping-pong schedule for
    # the first workload (mean 129) and the 128-row tile for the second (32)
    w = W.WORKLOADS[name]
    g, max_m, n, k = w.shape["g"], w.shape["max_m"], w.shape["n"], w.shape["k"]
    x = W.draw(name)
    mm = x["masked_m"]
    assert int(mm.sum()) == total
    print(f"[case] {name}: quantise + GEMM on GPU", flush=True)
    qa, sfa = dg.quantize_a_1x128(H.f32_to_device(x["a"], gpu))
    qb, sfb = dg.quantize_b_128x128(H.f32_to_device(x["b"], gpu))
    d, flat = H.sentinel_bf16((g, max_m, n), gpu, guard=4096)
    expected = int(np.clip(mm, 0, max_m).mean())
    dg.m_grouped_fp8_gemm_nt_masked((qa, sfa), (qb, sfb), d, torch.from_numpy(mm).to(gpu), expected)
    torch.cuda.synchronize()
    assert H.guard_untouched(flat, d.numel())
    # every row past masked_m keeps the sentinel (checked on the device, bits only)
    valid = torch.arange(max_m, device=gpu)[None, :] < torch.from_numpy(mm).to(gpu)[:, None]
    bits = d.view(torch.int16)  # the 0xFFFF sentinel reads as -1
    assert bool((bits[~valid] == -1).all())
    assert not bool((bits[valid] == -1).any())
    rng = np.random.default_rng(97)
    sfb_dev = sfb.cpu().numpy()
    for e in [int(np.argmin(mm)), int(np.argmax(mm)), 5, 9]:
        cnt = int(mm[e])
        rows = np.unique(np.concatenate([[0, cnt - 1], rng.integers(0, cnt, 6)]))
        bsel, cols = plan_cols(rng, n, 2, 16)
        qa_r, sa_r = oracle.quantize_a_1x128(x["a"][e][rows])
        assert np.array_equal(qa[e].view(torch.uint8)[torch.from_numpy(rows).to(gpu)].cpu().numpy(), qa_r)
        b_codes = np.zeros((len(cols), k), np.uint8)
        b_scales = np.zeros((len(cols), k // 128), np.float32)
        for blk in bsel:
            lo, hi, q, s = oracle_b_block(x["b"][e], blk)
            sel = (cols >= lo) & (cols < hi)
            b_codes[sel] = q[cols[sel] - lo]
            b_scales[sel] = s
            assert np.array_equal(sfb_dev[e, blk], s)
        d_sel = d[e].float()[torch.from_numpy(rows).to(gpu)][:, torch.from_numpy(cols).to(gpu)].cpu().numpy()
        check_sampled(f"{name} expert {e}", d_sel.astype(np.float64), qa_r, sa_r, b_codes, b_scales, rows, cols)


def test_kgrouped_full(gpu):
    name = "kgrouped_4x8192_m4096_n7168"
    w = W.WORKLOADS[name]
    m, n = w.shape["m"], w.shape["n"]
    sizes = list(w.shape["k_sizes"])
    k = sum(sizes)
    x = W.draw(name)
    print(f"[case] {name}: quantise + GEMM on GPU", flush=True)
    qa, sfa = dg.quantize_a_1x128(H.f32_to_device(x["a"], gpu))
    qb, sfb = dg.quantize_b_128x128(H.f32_to_device(x["b"], gpu))
    d, flat = H.sentinel_bf16((len(sizes), m, n), gpu, guard=4096)
    dg.k_grouped_fp8_gemm_nt((qa, sfa), (qb, sfb), d, torch.from_numpy(x["k_sizes"]).to(gpu))
    torch.cuda.synchronize()
    assert H.guard_untouched(flat, d.numel())
    assert not bool((d.view(torch.int16) == -1).any())  # every element written
    rng = np.random.default_rng(96)
    rows = np.unique(np.concatenate([[0, m - 1], pick(rng, m, 8)]))
    bsel, cols = plan_cols(rng, n, 2, 16)
    qa_r, sa_r = oracle.quantize_a_1x128(x["a"][rows])
    assert np.array_equal(qa.view(torch.uint8)[torch.from_numpy(rows).to(gpu)].cpu().numpy(), qa_r)
    b_codes = np.zeros((len(cols), k), np.uint8)
    b_scales = np.zeros((len(cols), k // 128), np.float32)
    sfb_dev = sfb.cpu().numpy()
    for blk in bsel:
        lo, hi, q, s = oracle_b_block(x["b"], blk)
        sel = (cols >= lo) & (cols < hi)
        b_codes[sel] = q[cols[sel] - lo]
        b_scales[sel] = s
        assert np.array_equal(sfb_dev[blk], s)
    s0 = 0
    for g, size in enumerate(sizes):
        s1 = s0 + size // 128
        kc = slice(s0 * 128, s1 * 128)
        d_sel = d[g].float()[torch.from_numpy(rows).to(gpu)][:, torch.from_numpy(cols).to(gpu)].cpu().numpy()
        check_sampled(f"{name} group {g}", d_sel.astype(np.float64), qa_r[:, kc], sa_r[:, s0:s1],
                      b_codes[:, kc], b_scales[:, s0:s1], rows, cols)
        s0 = s1
