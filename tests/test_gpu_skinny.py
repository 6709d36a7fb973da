"""GPU parity of the skinny-M dense kernel (any m <= 64 when a skinny
configuration is forced; the default for m <= 16 where it is faster) and the
split-K workspace rules: per-stream workspaces, overlapping calls on two
streams, graph replays after the workspace has grown, and the status a
capture gets when the workspace would have to grow.

Every output element is compared with the oracle; elements without a result
must keep the 0xFFFF sentinel and the guard band past D stays untouched.
"""

import ctypes

import numpy as np
import pytest
import torch

import fp8_block_scaled_nt_amd as dg
import oracle
import workloads as W
from tests import gpu_harness as H

pytestmark = pytest.mark.gpu

SKINNY = ["skinny_64x32_w16_direct", "skinny_64x32_w16_stagea", "skinny_64x32_w8_u2_stage",
          "skinny_64x32_w8_u2_direct", "skinny_64x32_w12_stage", "skinny_64x16_w16_direct", "skinny_64x64_w8_stagea"]
DG_ERR_WORKSPACE = 7


def dense_case(m, n, k, seed, b_std=1.0):
    x = W.draw_dense(m, n, k, seed=seed, b_std=b_std)
    qa, sa = oracle.quantize_a_1x128(x["a"])
    qb, sb = oracle.quantize_b_128x128(x["b"])
    return qa, sa, qb, sb


def check(gpu, case, label):
    qa, sa, qb, sb = case
    print(f"[case] {label}", flush=True)
    d, flat = H.run_dense(qa, sa, qb, sb, gpu)
    r = oracle.gemm_nt_ref(qa, sa, qb, sb)
    res = oracle.tolerance_check(H.d_float(d), r)
    assert res["ok"], (label, res)
    assert H.guard_untouched(flat, d.numel()), label
    return d


@pytest.mark.parametrize("cfg", [None] + SKINNY)
def test_decode_shape_whole_output(gpu, cfg, monkeypatch):
    """The headline decode shape 64 x 2112 x 7168 (B ~ N(0, 0.02)), every
    output element, for the default and each skinny configuration; a second
    call repeats the first bit for bit."""
    if cfg:
        monkeypatch.setenv("DG_FORCE_CONFIG", cfg)
    case = dense_case(64, 2112, 7168, seed=0, b_std=0.02)
    d = check(gpu, case, f"decode 64x2112x7168 {cfg}")
    d2, _ = H.run_dense(*case, gpu)
    assert np.array_equal(H.d_bits(d), H.d_bits(d2)), "two calls differ"


@pytest.mark.parametrize("cfg", SKINNY)
@pytest.mark.parametrize("m,n,k", [
    (1, 16, 128),      # one row, one tile, one slab
    (5, 40, 256),      # ragged N inside the first tile
    (17, 200, 640),    # two A fragments, ragged N tail
    (33, 520, 1280),   # ragged M and N
    (64, 136, 7168),   # a partial 128-row B scale block
    (48, 2112, 1024),
    (64, 4096, 384),   # many tiles, short K: runs span several tiles
    (64, 96, 7680),    # long K over few tiles: 15-16 contributors per tile
])
def test_skinny_shapes(gpu, cfg, m, n, k, monkeypatch):
    monkeypatch.setenv("DG_FORCE_CONFIG", cfg)
    check(gpu, dense_case(m, n, k, seed=m * 7 + n + k), f"{cfg} {m}x{n}x{k}")


def test_skinny_rejects_tall_m(gpu, monkeypatch):
    monkeypatch.setenv("DG_FORCE_CONFIG", "skinny_64x32_w16_direct")
    qa, sa, qb, sb = dense_case(65, 64, 128, seed=1)
    with pytest.raises(dg.DGError, match="does not take"):
        H.run_dense(qa, sa, qb, sb, gpu)


def _device_operands(case, gpu):
    qa, sa, qb, sb = case
    return (H.codes_to_device(qa, gpu), H.f32_to_device(H.slab_major(sa), gpu),
            H.codes_to_device(qb, gpu), H.f32_to_device(sb, gpu))


@pytest.mark.parametrize("cfg", ["skinny_64x32_w16_stagea", "dense_64x32_w4_s4", "dense_64x32_w4_s6_triple"])
def test_two_streams_overlap(gpu, cfg, monkeypatch):
    """Two split-K calls of the decode shape enqueued on two streams with no
    synchronisation between them (each stream has its own workspace): both
    outputs match the oracle element by element, for the skinny kernel and
    for the tiled split-K kernel."""
    monkeypatch.setenv("DG_FORCE_CONFIG", cfg)
    cases = [dense_case(64, 2112, 7168, seed=s, b_std=0.02) for s in (11, 12)]
    refs = [oracle.gemm_nt_ref(*c) for c in cases]
    ops = [_device_operands(c, gpu) for c in cases]
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    outs = [H.sentinel_bf16((64, 2112), gpu)[0] for _ in range(2)]
    torch.cuda.synchronize()
    print(f"[case] two streams {cfg}", flush=True)
    for rep in range(3):
        for i in (0, 1):
            with torch.cuda.stream(streams[i]):
                for _ in range(4):  # several calls back to back keep both streams busy together
                    dg.fp8_gemm_nt((ops[i][0], ops[i][1]), (ops[i][2], ops[i][3]), outs[i])
        torch.cuda.synchronize()
        for i in (0, 1):
            res = oracle.tolerance_check(H.d_float(outs[i]), refs[i])
            assert res["ok"], (cfg, rep, i, res)


def test_graph_replay_after_workspace_growth(gpu):
    """A decode GEMM captured with a reserved workspace keeps replaying
    correctly after an eager call on the capture stream has grown that
    stream's workspace (the old block stays allocated)."""
    case = dense_case(64, 2112, 7168, seed=21, b_std=0.02)
    a, sfa, b, sfb = _device_operands(case, gpu)
    ref = oracle.gemm_nt_ref(*case)
    stream = torch.cuda.Stream()
    dg.reserve_workspace(dg.dense_workspace_size(64, 2112, 7168), stream)
    d = H.sentinel_bf16((64, 2112), gpu)[0]
    graph = torch.cuda.CUDAGraph()
    print("[case] capture decode GEMM", flush=True)
    with torch.cuda.stream(stream):
        with torch.cuda.graph(graph, stream=stream):
            dg.fp8_gemm_nt((a, sfa), (b, sfb), d)
    torch.cuda.synchronize()
    # an eager split-K call on the same stream that needs a larger workspace
    big = dense_case(4096, 896, 2048, seed=22)
    ba, bsfa, bb, bsfb = _device_operands(big, gpu)
    dbig = H.sentinel_bf16((4096, 896), gpu)[0]
    need_big = dg.dense_workspace_size(4096, 896, 2048)
    assert need_big > (4 << 20), need_big
    with torch.cuda.stream(stream):
        dg.fp8_gemm_nt((ba, bsfa), (bb, bsfb), dbig)
    torch.cuda.synchronize()
    rbig = oracle.gemm_nt_ref(*big)
    assert oracle.tolerance_check(H.d_float(dbig), rbig)["ok"]
    for rep in range(3):
        d.view(torch.uint16).fill_(H.SENTINEL)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        res = oracle.tolerance_check(H.d_float(d), ref)
        assert res["ok"], (rep, res)
        with torch.cuda.stream(stream):  # eager work on the grown workspace between replays
            dg.fp8_gemm_nt((ba, bsfa), (bb, bsfb), dbig)
        torch.cuda.synchronize()


def test_capture_needing_growth_returns_status(gpu):
    """A split-K call captured on a stream whose workspace is too small is
    refused with DG_ERR_WORKSPACE before anything is enqueued; reserving the
    workspace on that stream first makes the same capture succeed."""
    case = dense_case(64, 2112, 7168, seed=31, b_std=0.02)
    a, sfa, b, sfb = _device_operands(case, gpu)
    d = H.sentinel_bf16((64, 2112), gpu)[0]
    lib = dg.lib()
    stream = torch.cuda.Stream()
    graph = torch.cuda.CUDAGraph()
    st = ctypes.c_void_p(stream.cuda_stream)
    status = []
    print("[case] capture without a reserved workspace", flush=True)
    with torch.cuda.stream(stream):
        with torch.cuda.graph(graph, stream=stream):
            status.append(lib.dg_fp8_gemm_nt(H._ptr(a), H._ptr(sfa), H._ptr(b), H._ptr(sfb), H._ptr(d),
                                             64, 2112, 7168, st))
    torch.cuda.synchronize()
    assert status == [DG_ERR_WORKSPACE], status
    assert b"dg_reserve_workspace" in lib.dg_last_error_message()
    dg.reserve_workspace(dg.dense_workspace_size(64, 2112, 7168), stream)
    graph2 = torch.cuda.CUDAGraph()
    with torch.cuda.stream(stream):
        with torch.cuda.graph(graph2, stream=stream):
            dg.fp8_gemm_nt((a, sfa), (b, sfb), d)
    torch.cuda.synchronize()
    graph2.replay()
    torch.cuda.synchronize()
    assert oracle.tolerance_check(H.d_float(d), oracle.gemm_nt_ref(*case))["ok"]
