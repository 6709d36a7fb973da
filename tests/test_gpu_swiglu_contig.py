"""GPU parity of the fused MoE FC1 + SwiGLU + FP8 requantisation on the
contiguous layout against the oracle (oracle.contiguous_swiglu_ref and
oracle.contiguous_swiglu_quant_ref), with the interval checks of the masked
version (tests/test_gpu_swiglu.py): exact-arithmetic inputs, where almost
every code is fixed and must match, and workload-like inputs under the GEMM
acceptance rule carried through h, where at least 98 % of the codes must
equal the oracle's.  Padding rows, rows with an out-of-range tag, the scale
layout's padding entries and the guard bands keep their sentinels."""

import numpy as np
import pytest

import oracle
import workloads as W
from tests import gpu_harness as H
from tests.test_gpu_swiglu import T, check_rows, exact_tol, rms, rule_tol

pytestmark = pytest.mark.gpu

CONFIGS = ["swiglu_contig_128x256_w4_s2_sb", "swiglu_contig_128x256_w8_s3", "swiglu_contig_64x256_w4_s3"]


def tags_of(group_rows, bad_at=None):
    """Expert tags: each expert's rows padded to the 128-row alignment with
    -1; bad_at puts an out-of-range tag at that row of expert 0's block."""
    tags = []
    for e, r in enumerate(group_rows):
        tags += [e] * r + [-1] * ((-r) % 128)
    tags = np.array(tags, np.int32)
    if bad_at is not None:
        tags[bad_at] = 99
    return tags


def exact_case(tags, g, inter, k, seed):
    rng = np.random.default_rng(seed)

    def codes(*shape):
        e = rng.integers(6, 9, shape)
        m = rng.integers(0, 8, shape)
        sgn = rng.integers(0, 2, shape)
        return ((sgn << 7) | (e << 3) | m).astype(np.uint8)

    m = tags.size
    qa = codes(m, k)
    qb = codes(g, 2 * inter, k)
    sa = np.exp2(rng.integers(-5, -2, (m, k // 128))).astype(np.float32)
    sb = np.exp2(rng.integers(-3, 0, (g, 2 * inter // 128, k // 128))).astype(np.float32)
    return qa, sa, qb, sb


def workload_case(group_rows, inter, k, seed):
    x = W.draw_contiguous(group_rows, 2 * inter, k, seed=seed)
    qa, sa = oracle.quantize_a_1x128(x["a"])
    qbs = [oracle.quantize_b_128x128(x["b"][i]) for i in range(len(group_rows))]
    return qa, sa, np.stack([q for q, _ in qbs]), np.stack([s for _, s in qbs]), np.asarray(x["m_indices"], np.int32)


def check_call(hq, hs_bits, qa, sa, qb, sb, tags, tol_fn, label, min_fixed):
    inter = qb.shape[1] // 2
    r, valid = oracle.grouped_contiguous_ref(qa, sa, qb, sb, tags)
    gate, up = r[:, :inter], r[:, inter:]
    h, _ = oracle.contiguous_swiglu_ref(qa, sa, qb, sb, tags)
    hq_o, hs_o, _ = oracle.contiguous_swiglu_quant_ref(qa, sa, qb, sb, tags)
    m = tags.size
    assert np.all(hq[~valid] == H.SENTINEL_CODE), label
    assert np.all(hs_bits[:, :m][:, ~valid] == H.SENTINEL_SCALE), label
    assert np.all(hs_bits[:, m:] == H.SENTINEL_SCALE), label
    rows = np.nonzero(valid)[0]
    if rows.size == 0:
        return 1.0
    tol = tol_fn(gate[rows], up[rows], rms(gate[rows]), rms(up[rows]))
    s_bits = np.ascontiguousarray(hs_bits[:, rows].T)
    fixed, total = check_rows(hq[rows], s_bits, h[rows], tol, label)
    code_share = float(np.sum(T[hq[rows]] == T[hq_o[rows]])) / total
    scale_share = float(np.sum(s_bits.view(np.float32) == hs_o[rows])) / (total // 128)
    print(f"  fixed {fixed / total:.5f} same code as the oracle {code_share:.5f} same scale {scale_share:.5f}",
          flush=True)
    assert fixed / total >= min_fixed, (label, fixed / total)
    return code_share


@pytest.mark.parametrize("cfg", [None] + CONFIGS)
def test_exact_inputs(gpu, cfg, monkeypatch):
    if cfg:
        monkeypatch.setenv("DG_FORCE_CONFIG", cfg)
    g, inter, k = 5, 384, 512
    tags = tags_of([200, 0, 77, 128, 5], bad_at=7)  # ragged, empty, full, short; a bad tag
    qa, sa, qb, sb = exact_case(tags, g, inter, k, seed=61)
    print(f"[case] contiguous swiglu exact {cfg}", flush=True)
    hq, hs, fq, fs = H.run_contig_swiglu(qa, sa, qb, sb, tags, gpu)
    assert H.swiglu_guards_untouched(fq, fs, hq.size, hs.size)
    code_share = check_call(hq, hs, qa, sa, qb, sb, tags, exact_tol, f"exact {cfg}", 0.999)
    assert code_share >= 0.999


@pytest.mark.parametrize("cfg", [None] + CONFIGS)
def test_workload_like_inputs(gpu, cfg, monkeypatch):
    if cfg:
        monkeypatch.setenv("DG_FORCE_CONFIG", cfg)
    inter, k = 256, 640
    qa, sa, qb, sb, tags = workload_case([300, 1, 0, 130, 64], inter, k, seed=63)
    print(f"[case] contiguous swiglu workload-like {cfg}", flush=True)
    hq, hs, fq, fs = H.run_contig_swiglu(qa, sa, qb, sb, tags, gpu)
    assert H.swiglu_guards_untouched(fq, fs, hq.size, hs.size)
    code_share = check_call(hq, hs, qa, sa, qb, sb, tags, rule_tol, f"workload-like {cfg}", 0.15)
    assert code_share >= 0.98, code_share


def test_every_tile_gives_the_same_bits(gpu, monkeypatch):
    # no K split: every tile adds each output's slabs in the same order
    inter, k = 512, 384
    qa, sa, qb, sb, tags = workload_case([256, 40, 384, 0, 129], inter, k, seed=65)
    outs = []
    for cfg in CONFIGS:
        monkeypatch.setenv("DG_FORCE_CONFIG", cfg)
        print(f"[case] contiguous swiglu same bits {cfg}", flush=True)
        hq, hs, fq, fs = H.run_contig_swiglu(qa, sa, qb, sb, tags, gpu)
        assert H.swiglu_guards_untouched(fq, fs, hq.size, hs.size)
        outs.append((hq, hs))
    code_share = check_call(outs[0][0], outs[0][1], qa, sa, qb, sb, tags, rule_tol, "same bits", 0.15)
    assert code_share >= 0.98, code_share
    for hq, hs in outs[1:]:
        assert np.array_equal(hq, outs[0][0]) and np.array_equal(hs, outs[0][1])


def test_feeds_the_contiguous_gemm(gpu):
    """hq/hs are the contiguous GEMM's A operand as they stand: FC2 over the
    kernel's h, on the device, against FC2 over the oracle's h, within the
    GEMM rule plus one e4m3 step per code the oracle leaves open."""
    import torch
    import fp8_block_scaled_nt_amd as dg
    inter, k, n2 = 384, 512, 272
    qa, sa, qb, sb, tags = workload_case([130, 0, 64, 99], inter, k, seed=67)
    g = qb.shape[0]
    rng = np.random.default_rng(68)
    w2 = [oracle.quantize_b_128x128((rng.standard_normal((n2, inter)) * 0.02).astype(np.float32)) for _ in range(g)]
    q2 = np.stack([q for q, _ in w2])
    s2 = np.stack([s for _, s in w2])
    print("[case] contiguous swiglu -> contiguous GEMM chain", flush=True)
    hq, hs, _, _ = H.run_contig_swiglu(qa, sa, qb, sb, tags, gpu)
    hq_o, hs_o, valid = oracle.contiguous_swiglu_quant_ref(qa, sa, qb, sb, tags)
    a2 = torch.from_numpy(hq).to(gpu).view(torch.float8_e4m3fn)
    sfa2 = torch.from_numpy(hs.view(np.float32)).to(gpu)
    d2, _ = H.sentinel_bf16((tags.size, n2), gpu)
    dg.m_grouped_fp8_gemm_nt_contiguous((a2, sfa2), (H.codes_to_device(q2, gpu), H.f32_to_device(s2, gpu)), d2,
                                        torch.from_numpy(tags).to(gpu))
    torch.cuda.synchronize()
    d2 = H.d_float(d2)
    # oracle chain, bounded as in the masked version
    rows = np.nonzero(valid)[0]
    r2, _ = oracle.grouped_contiguous_ref(hq_o, np.nan_to_num(hs_o), q2, s2, tags)
    r, _ = oracle.grouped_contiguous_ref(qa, sa, qb, sb, tags)
    h, _ = oracle.contiguous_swiglu_ref(qa, sa, qb, sb, tags)
    rms_g, rms_u = rms(r[rows, :inter]), rms(r[rows, inter:])
    rms2 = rms(r2[rows])
    tol = rule_tol(r[rows, :inter], r[rows, inter:], rms_g, rms_u)
    hv = h[rows]
    s_o = np.repeat(hs_o[rows].astype(np.float64), 128, axis=1)
    step = np.maximum(np.abs(hv) * 2.0 ** -3, s_o * 2.0 ** -9)
    hb = tol.reshape(rows.size, -1, 128).max(axis=-1)
    s_rel = np.repeat(hb / (448.0 * hs_o[rows]), 128, axis=1) + 2.0 ** -23
    dh = step + 2 * tol + np.abs(hv) * 2 * s_rel
    for e in range(g):
        sel = tags[rows] == e
        if not sel.any():
            continue
        w = T[q2[e]].astype(np.float64) * np.repeat(s2[e], 128, axis=1)[np.arange(n2) // 128]
        bound = dh[sel] @ np.abs(w).T
        err = np.abs(d2[rows[sel]] - r2[rows[sel]])
        rule = oracle.check.REL_TOL * np.abs(r2[rows[sel]]) + oracle.check.ABS_TOL_RMS * rms2
        assert np.all(err <= rule + bound), (e, float(np.max(err - rule - bound)))
        res = oracle.tolerance_check(d2[rows[sel]], r2[rows[sel]], rms=rms2)
        print(f"  expert {e}: {res['n_bad']} of {res['n']} outside the plain GEMM rule", flush=True)


def test_full_size_sampled(gpu):
    """The contiguous FC1 workload (4 experts x 8192 rows, 2I = 4096, I = 2048,
    K = 7168), run as the benchmark runs it: quantised on the GPU by the
    library, the fused kernel at its default configuration.  Every h code and
    scale of the tagged rows is written (no row is padding here) and the guard
    bands keep their sentinels; for each expert the oracle re-quantises three
    of its A rows and its B on the CPU (the codes and scales must be
    bit-identical) and computes h for those rows."""
    import torch

    import fp8_block_scaled_nt_amd as dg
    name = "moe_swiglu_contig_4x8192_i2048_k7168"
    x = W.draw(name)
    s = W.WORKLOADS[name].shape
    inter, k, g = s["inter"], s["k"], len(s["group_rows"])
    idx = np.asarray(x["m_indices"], np.int32)
    m = idx.size
    print(f"[case] contiguous swiglu full size {name}", flush=True)
    qa, sfa = dg.quantize_a_1x128(H.f32_to_device(x["a"], gpu))
    qb, sfb = dg.quantize_b_128x128(H.f32_to_device(x["b"], gpu))
    ld = H.sfa_ld(m)
    nq, ns, guard = m * inter, (inter // 128) * ld, 4096
    fq = torch.full((nq + guard,), H.SENTINEL_CODE, dtype=torch.uint8, device=gpu)
    fs = torch.full((ns + guard,), H.SENTINEL_SCALE, dtype=torch.int32, device=gpu)
    hq_t = fq[:nq].view(m, inter)
    hs_t = fs[:ns].view(torch.float32).view(inter // 128, ld)
    dg.m_grouped_fp8_gemm_nt_contiguous_swiglu((qa, sfa), (qb, sfb), (hq_t.view(torch.float8_e4m3fn), hs_t),
                                               torch.from_numpy(idx).to(gpu))
    torch.cuda.synchronize()
    assert H.swiglu_guards_untouched(fq, fs, nq, ns)
    # no row is padding: every h code and every row's scales are written
    assert not bool((hq_t == H.SENTINEL_CODE).any())
    assert not bool((hs_t[:, :m].view(torch.int32) == H.SENTINEL_SCALE).any())
    hq = hq_t.cpu().numpy()
    hs = fs[:ns].view(inter // 128, ld).cpu().numpy().view(np.uint32)
    rng = np.random.default_rng(131)
    fixed, total, same = 0, 0, 0
    for e in range(g):
        seg = np.nonzero(idx == e)[0]
        rows = np.unique(np.concatenate([[seg[0], seg[-1]], rng.choice(seg, 1)]))
        qa_r, sa_r = oracle.quantize_a_1x128(x["a"][rows])
        assert np.array_equal(qa.view(torch.uint8)[torch.from_numpy(rows).to(gpu)].cpu().numpy(), qa_r)
        qb_e, sb_e = oracle.quantize_b_128x128(x["b"][e])
        assert np.array_equal(qb[e].view(torch.uint8).cpu().numpy(), qb_e)
        assert np.array_equal(sfb[e].cpu().numpy(), sb_e)
        sub = oracle.gemm_nt_ref(qa_r, sa_r, qb_e, sb_e)
        gate, up = sub[:, :inter], sub[:, inter:]
        h = oracle.silu(gate) * up
        f, t = check_rows(hq[rows], np.ascontiguousarray(hs[:, rows].T), h,
                          rule_tol(gate, up, rms(gate), rms(up)), f"{name} expert {e}")
        fixed, total = fixed + f, total + t
        hq_o, _ = oracle.quantize_a_1x128(h.astype(np.float32))
        same += int(np.sum(T[hq[rows]] == T[hq_o]))
    print(f"  fixed {fixed / max(total, 1):.5f} same code as the oracle {same / max(total, 1):.5f} of {total}",
          flush=True)
    assert fixed >= 0.1 * total and same >= 0.98 * total
