"""The hot path captured in a HIP graph (as bench.py times it) gives the
eager result on every replay, with eager work and synchronisation between
replays."""

import numpy as np
import pytest
import torch

import fp8_block_scaled_nt_amd as dg
import workloads as W
from tests import gpu_harness as H

pytestmark = pytest.mark.gpu


def test_graph_replays_match_eager(gpu):
    x = W.draw("dense_decode_64x2112x7168")
    xa = H.f32_to_device(x["a"], gpu)
    qb, sfb = dg.quantize_b_128x128(H.f32_to_device(x["b"], gpu))
    qa, sfa = dg.quantize_a_1x128(xa)
    d_eager = torch.empty((64, 2112), dtype=torch.bfloat16, device=gpu)
    dg.fp8_gemm_nt((qa, sfa), (qb, sfb), d_eager)
    torch.cuda.synchronize()
    ref = H.d_bits(d_eager)

    qa2 = torch.empty_like(qa)
    sfa2 = torch.empty_like(sfa)
    d = torch.empty_like(d_eager)
    stream = torch.cuda.Stream()
    dg.reserve_workspace(dg.dense_workspace_size(64, 2112, 7168), stream)  # the capture stream's workspace
    graph = torch.cuda.CUDAGraph()
    print("[case] graph capture of quantise A + GEMM (decode shape)", flush=True)
    with torch.cuda.stream(stream):
        with torch.cuda.graph(graph, stream=stream):
            dg.quantize_a_1x128(xa, qa2, sfa2)
            dg.fp8_gemm_nt((qa2, sfa2), (qb, sfb), d)
    torch.cuda.synchronize()
    for rep in range(4):
        d.fill_(float("nan"))
        qa2.view(torch.uint8).fill_(0)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert np.array_equal(H.d_bits(d), ref), f"replay {rep} differs from eager"
        # eager work between replays
        dg.fp8_gemm_nt((qa, sfa), (qb, sfb), d_eager)
        torch.cuda.synchronize()


def _replay_check(graph, outputs, refs, eager, label):
    for rep in range(4):
        for o in outputs:
            o.view(torch.uint8).fill_(0x7F)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for o, r in zip(outputs, refs):
            assert np.array_equal(o.view(torch.uint8).cpu().numpy(), r), f"{label}: replay {rep} differs from eager"
        eager()
        torch.cuda.synchronize()


def test_graph_swiglu_and_fp4(gpu):
    """The fused FC1 + SwiGLU (masked counts read on the device) and the FP4
    quantise + GEMM, captured together; the masked counts change between
    replays from the host side, and each replay must match an eager run
    with the counts it saw."""
    rng = np.random.default_rng(77)
    g, max_m, inter, k = 4, 96, 256, 512
    xa = torch.from_numpy(rng.standard_normal((g, max_m, k), dtype=np.float32)).to(gpu)
    xb = torch.from_numpy((rng.standard_normal((g, 2 * inter, k)) * 0.02).astype(np.float32)).to(gpu)
    qa, sfa = dg.quantize_a_1x128(xa)
    qb, sfb = dg.quantize_b_128x128(xb)
    mm = torch.tensor([96, 0, 33, 70], dtype=torch.int32, device=gpu)
    ld = dg.get_sfa_ld(max_m)
    hq = torch.empty((g, max_m, inter), dtype=torch.float8_e4m3fn, device=gpu)
    hs = torch.empty((g, inter // 128, ld), dtype=torch.float32, device=gpu)
    x4 = torch.from_numpy(rng.standard_normal((64, 1024), dtype=np.float32)).to(gpu)
    w4 = torch.from_numpy(rng.standard_normal((300, 1024), dtype=np.float32)).to(gpu)
    qb4, sfb4 = dg.quantize_b_128x128_fp4(w4)
    qa4 = torch.empty((64, 512), dtype=torch.uint8, device=gpu)
    sfa4 = dg.empty_sfa(64, 1024, None, gpu)
    d4 = torch.empty((64, 300), dtype=torch.bfloat16, device=gpu)
    stream = torch.cuda.Stream()
    dg.reserve_workspace(16 << 20, stream)  # the capture stream's split-K workspace

    def run():
        dg.m_grouped_fp8_gemm_nt_masked_swiglu((qa, sfa), (qb, sfb), (hq, hs), mm)
        dg.quantize_a_1x128_fp4(x4, qa4, sfa4)
        dg.fp4_gemm_nt((qa4, sfa4), (qb4, sfb4), d4)

    def eager_refs():
        for o in (hq, hs, d4):
            o.view(torch.uint8).fill_(0x7F)
        run()
        torch.cuda.synchronize()
        return [o.view(torch.uint8).cpu().numpy().copy() for o in (hq, hs, d4)]

    refs = eager_refs()
    graph = torch.cuda.CUDAGraph()
    print("[case] graph capture of FC1 + SwiGLU and FP4 quantise + GEMM", flush=True)
    with torch.cuda.stream(stream):
        with torch.cuda.graph(graph, stream=stream):
            run()
    torch.cuda.synchronize()
    _replay_check(graph, [hq, hs, d4], refs, run, "swiglu + fp4")
    # new counts, written on the device between replays: the replay follows them
    mm.copy_(torch.tensor([5, 96, 0, 64], dtype=torch.int32))
    torch.cuda.synchronize()
    refs = eager_refs()
    _replay_check(graph, [hq, hs, d4], refs, run, "swiglu + fp4, new counts")


def test_workspace_size_then_graph_of_mid_shape(gpu):
    """dense_workspace_size gives what a dense call's split-K takes (known
    figures on the decode, large and N-shard shapes); with that much
    reserved, a split-K call of a mid-sized shape captures and replays like
    its eager run."""
    tile = 64 * 32 * 4
    for dt in ("fp8", "bf16", "fp4"):
        assert dg.dense_workspace_size(64, 2112, 7168, dt) == 66 * 7 * tile, dt  # 7 splits of 64 x 32 tiles
    assert dg.dense_workspace_size(4096, 7168, 16384) == 0                       # 448 big tiles, no split
    assert dg.dense_workspace_size(4096, 896, 16384) == 224 * 2 * 128 * 128 * 4  # 128 x 128 tiles, 2 splits
    assert dg.dense_workspace_size(0, 896, 16384) == 0
    # m <= 16: the same tiled kernel, 64 x 32 tiles, 7 splits
    assert dg.dense_workspace_size(16, 2112, 7168) == 66 * 7 * tile
    m, n, k = 1024, 896, 2048  # 56 tiles of 128 x 128, 8 splits
    need = dg.dense_workspace_size(m, n, k)
    assert need == 56 * 8 * 128 * 128 * 4
    stream = torch.cuda.Stream()
    dg.reserve_workspace(need, stream)
    rng = np.random.default_rng(5)
    qa, sfa = dg.quantize_a_1x128(torch.from_numpy(rng.standard_normal((m, k), dtype=np.float32)).to(gpu))
    qb, sfb = dg.quantize_b_128x128(torch.from_numpy(rng.standard_normal((n, k), dtype=np.float32)).to(gpu))
    d_eager = torch.empty((m, n), dtype=torch.bfloat16, device=gpu)
    dg.fp8_gemm_nt((qa, sfa), (qb, sfb), d_eager)
    torch.cuda.synchronize()
    ref = d_eager.view(torch.uint8).cpu().numpy()
    d = torch.empty_like(d_eager)
    graph = torch.cuda.CUDAGraph()
    print("[case] graph capture of a split-K mid shape 1024x896x2048", flush=True)
    with torch.cuda.stream(stream):
        with torch.cuda.graph(graph, stream=stream):
            dg.fp8_gemm_nt((qa, sfa), (qb, sfb), d)
    torch.cuda.synchronize()
    _replay_check(graph, [d], [ref], lambda: dg.fp8_gemm_nt((qa, sfa), (qb, sfb), d_eager), "mid shape")
