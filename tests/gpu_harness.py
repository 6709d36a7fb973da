"""Helpers shared by the GPU parity tests: move oracle-quantised operands
into the library's device layouts, run the library, and read results back.

Nothing here computes the method: codes and scales come from the oracle's
quantisers (CPU), results from the library (GPU), expected values from the
oracle's GEMMs (CPU).
"""

import ctypes

import numpy as np
import torch

import fp8_block_scaled_nt_amd as dg

SENTINEL = 0xFFFF  # bf16 NaN pattern used to prefill D


def sfa_ld(m):
    return (m + 3) // 4 * 4


def slab_major(sfa_logical):
    """Logical [rows, K/128] scales -> the library's slab-major [K/128, ld(rows)]
    (padding entries zero)."""
    rows, kb = sfa_logical.shape
    out = np.zeros((kb, sfa_ld(rows)), dtype=np.float32)
    out[:, :rows] = sfa_logical.T
    return out


def slab_major_to_logical(sfa_dev, rows):
    """Inverse of slab_major for a downloaded buffer."""
    return np.ascontiguousarray(sfa_dev[:, :rows].T)


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr())


def codes_to_device(codes, dev):
    return torch.from_numpy(np.ascontiguousarray(codes, np.uint8)).to(dev).view(torch.float8_e4m3fn)


def f32_to_device(x, dev):
    return torch.from_numpy(np.ascontiguousarray(x, np.float32)).to(dev)


def sentinel_bf16(shape, dev, guard=0):
    """A bf16 buffer prefilled with the sentinel, with `guard` extra trailing
    elements; returns (view of the requested shape, the whole flat buffer)."""
    numel = int(np.prod(shape))
    flat = torch.full((numel + guard,), SENTINEL, dtype=torch.uint16, device=dev)
    view = flat[:numel].view(torch.bfloat16).view(*shape)
    return view, flat


def d_bits(d):
    return d.view(torch.uint16).cpu().numpy()


def d_float(d):
    return d.float().cpu().numpy().astype(np.float64)


def run_dense(qa, sa, qb, sb, dev, guard=256):
    m, k = qa.shape
    n = qb.shape[0]
    a = codes_to_device(qa, dev)
    b = codes_to_device(qb, dev)
    sfa = f32_to_device(slab_major(sa), dev)
    sfb = f32_to_device(sb, dev)
    d, flat = sentinel_bf16((m, n), dev, guard)
    dg.fp8_gemm_nt((a, sfa), (b, sfb), d)
    torch.cuda.synchronize()
    return d, flat


def run_contiguous(qa, sa, qb, sb, m_indices, dev, guard=256):
    m, k = qa.shape
    g, n, _ = qb.shape
    a = codes_to_device(qa, dev)
    b = codes_to_device(qb, dev)
    sfa = f32_to_device(slab_major(sa), dev)
    sfb = f32_to_device(sb, dev)
    idx = torch.from_numpy(np.asarray(m_indices, np.int32)).to(dev)
    d, flat = sentinel_bf16((m, n), dev, guard)
    dg.m_grouped_fp8_gemm_nt_contiguous((a, sfa), (b, sfb), d, idx)
    torch.cuda.synchronize()
    return d, flat


def run_masked(qa, sa, qb, sb, masked_m, dev, expected_m=0, guard=256):
    g, max_m, k = qa.shape
    n = qb.shape[1]
    a = codes_to_device(qa, dev)
    b = codes_to_device(qb, dev)
    sfa = f32_to_device(np.stack([slab_major(sa[i]) for i in range(g)]), dev)
    sfb = f32_to_device(sb, dev)
    mm = torch.from_numpy(np.asarray(masked_m, np.int32)).to(dev)
    d, flat = sentinel_bf16((g, max_m, n), dev, guard)
    dg.m_grouped_fp8_gemm_nt_masked((a, sfa), (b, sfb), d, mm, expected_m)
    torch.cuda.synchronize()
    return d, flat


def run_kgrouped(qa, sa, qb, sb, k_sizes, dev, guard=256):
    m, k = qa.shape
    n = qb.shape[0]
    g = len(k_sizes)
    a = codes_to_device(qa, dev)
    b = codes_to_device(qb, dev)
    sfa = f32_to_device(slab_major(sa), dev)
    sfb = f32_to_device(sb, dev)
    ks = torch.from_numpy(np.asarray(k_sizes, np.int32)).to(dev)
    d, flat = sentinel_bf16((g, m, n), dev, guard)
    dg.k_grouped_fp8_gemm_nt((a, sfa), (b, sfb), d, ks)
    torch.cuda.synchronize()
    return d, flat


def run_fp4(pa, sa, pb, sb, dev, guard=256):
    """FP4 GEMM on packed e2m1 operands (uint8 [m, k/2], [n, k/2])."""
    m = pa.shape[0]
    n = pb.shape[0]
    a = torch.from_numpy(np.ascontiguousarray(pa, np.uint8)).to(dev)
    b = torch.from_numpy(np.ascontiguousarray(pb, np.uint8)).to(dev)
    sfa = f32_to_device(slab_major(sa), dev)
    sfb = f32_to_device(sb, dev)
    d, flat = sentinel_bf16((m, n), dev, guard)
    dg.fp4_gemm_nt((a, sfa), (b, sfb), d)
    torch.cuda.synchronize()
    return d, flat


def run_bf16(a_bits, b_bits, dev, guard=256):
    m, k = a_bits.shape
    n = b_bits.shape[0]
    a = torch.from_numpy(np.ascontiguousarray(a_bits).view(np.int16)).to(dev).view(torch.bfloat16)
    b = torch.from_numpy(np.ascontiguousarray(b_bits).view(np.int16)).to(dev).view(torch.bfloat16)
    d, flat = sentinel_bf16((m, n), dev, guard)
    dg.bf16_gemm_nt(a, b, d)
    torch.cuda.synchronize()
    return d, flat


SENTINEL_CODE = 0x7F            # e4m3 NaN: never produced (codes saturate at 448)
SENTINEL_SCALE = 0x7FC0BEEF     # a NaN bit pattern for untouched fp32 scales


def run_swiglu(qa, sa, qb, sb, masked_m, dev, expected_m=0, guard=256):
    """Fused FC1 + SwiGLU + requantisation.  Returns (hq, hs, hq_flat,
    hs_flat): hq as uint8 [g][max_m][inter], hs as raw uint32 bits in the
    device layout [g][inter/128][ld], and the whole prefilled buffers."""
    g, max_m, k = qa.shape
    inter = qb.shape[1] // 2
    ld = sfa_ld(max_m)
    a = codes_to_device(qa, dev)
    b = codes_to_device(qb, dev)
    sfa = f32_to_device(np.stack([slab_major(sa[i]) for i in range(g)]), dev)
    sfb = f32_to_device(sb, dev)
    mm = torch.from_numpy(np.asarray(masked_m, np.int32)).to(dev)
    nq = g * max_m * inter
    ns = g * (inter // 128) * ld
    hq_flat = torch.full((nq + guard,), SENTINEL_CODE, dtype=torch.uint8, device=dev)
    hs_flat = torch.full((ns + guard,), SENTINEL_SCALE, dtype=torch.int32, device=dev)
    hq = hq_flat[:nq].view(g, max_m, inter)
    hs = hs_flat[:ns].view(torch.float32).view(g, inter // 128, ld)
    dg.m_grouped_fp8_gemm_nt_masked_swiglu((a, sfa), (b, sfb), (hq.view(torch.float8_e4m3fn), hs), mm, expected_m)
    torch.cuda.synchronize()
    return (hq.cpu().numpy(), hs_flat[:ns].view(g, inter // 128, ld).cpu().numpy().view(np.uint32),
            hq_flat, hs_flat)


def run_contig_swiglu(qa, sa, qb, sb, m_indices, dev, guard=256):
    """Fused FC1 + SwiGLU + requantisation on the contiguous layout.  Returns
    (hq, hs, hq_flat, hs_flat): hq as uint8 [m][inter], hs as raw uint32 bits
    in the device layout [inter/128][ld], and the whole prefilled buffers."""
    m, k = qa.shape
    inter = qb.shape[1] // 2
    ld = sfa_ld(m)
    a = codes_to_device(qa, dev)
    b = codes_to_device(qb, dev)
    sfa = f32_to_device(slab_major(sa), dev)
    sfb = f32_to_device(sb, dev)
    idx = torch.from_numpy(np.asarray(m_indices, np.int32)).to(dev)
    nq = m * inter
    ns = (inter // 128) * ld
    hq_flat = torch.full((nq + guard,), SENTINEL_CODE, dtype=torch.uint8, device=dev)
    hs_flat = torch.full((ns + guard,), SENTINEL_SCALE, dtype=torch.int32, device=dev)
    hq = hq_flat[:nq].view(m, inter)
    hs = hs_flat[:ns].view(torch.float32).view(inter // 128, ld)
    dg.m_grouped_fp8_gemm_nt_contiguous_swiglu((a, sfa), (b, sfb), (hq.view(torch.float8_e4m3fn), hs), idx)
    torch.cuda.synchronize()
    return (hq.cpu().numpy(), hs_flat[:ns].view(inter // 128, ld).cpu().numpy().view(np.uint32),
            hq_flat, hs_flat)


def swiglu_guards_untouched(hq_flat, hs_flat, nq, ns):
    tq = hq_flat[nq:].cpu().numpy()
    ts = hs_flat[ns:].cpu().numpy().view(np.uint32)
    return bool(np.all(tq == SENTINEL_CODE) and np.all(ts == SENTINEL_SCALE))


def guard_untouched(flat, numel):
    tail = flat[numel:].cpu().numpy()
    return bool(np.all(tail == SENTINEL))
