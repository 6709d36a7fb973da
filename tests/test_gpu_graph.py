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
