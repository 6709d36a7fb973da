"""Reference FP8 block-scaled NT GEMMs in fp64.  Test infrastructure only.

What is computed (D = A . B^T with block scales):

    D[m, n] = sum over K slabs kb of
              ( sum_{k in slab kb} a[m, k] * b[n, k] ) * sa[m, kb] * sb[n // 128, kb]

This is the plain definition of a block-dequantised matmul.  The pages reach
it through FP8 tensor-core sums per block followed by a higher-precision
second accumulation level ("DeepSeek open-source week day 3",
deepseek.csdn.net, "technical features", the two-level accumulation item);
the oracle writes the definition out directly, slab by slab:

* the per-slab dot products are taken in fp64 through a BLAS matmul.  They
  are exact in any summation order: each product of two e4m3 values is an
  integer multiple of 2^-18 below 2^17.6 in magnitude, so a 128-term sum
  stays far inside the 53-bit fp64 significand;
* the scale product sa * sb of two fp32 numbers is exact in fp64;
* one rounding happens per slab when the scaled slab sum is added.

So the result is the exact real-valued product to about (K/128) * 2^-53
relative, far below the bf16 output precision.

The grouped layouts follow the same page (MoE items):

* contiguous: the rows of all experts are stacked in one M x K matrix and
  each row carries an int32 expert index; row r uses expert m_indices[r]'s
  B.  An index outside [0, G) marks a padding row, which has no result.
* masked: A is G x max_m x K; expert g has masked_m[g] valid rows
  (clamped to [0, max_m]); rows at or past that count have no result.

Invalid entries are returned as NaN together with a boolean validity mask.

The K-grouped layout is named on "DeepGEMM: making LLM matrix
multiplication fly" (pomoai.com), "core functions", next to the M-grouped
one, for the irregular shapes of MoE training; the pages give no more than
the name.  The reading taken here: G groups are concatenated along K, group g
owning the k_sizes[g] consecutive K columns that follow the groups before it
(each size a multiple of 128, so every group is a run of whole scale slabs),
and D[g] = A[:, K_g] . B[:, K_g]^T with the same 1x128 / 128x128 scales as
the dense GEMM (the weight-gradient use: tokens on K).  An empty group's
result is the empty sum, zero.
"""

import numpy as np

from .e4m3 import decode_table

SLAB = 128


def _shapes(qa, sfa, qb, sfb):
    m, k = qa.shape
    n, k2 = qb.shape
    if k != k2 or k % SLAB:
        raise ValueError("A and B must share K, a multiple of 128")
    kb = k // SLAB
    nb = (n + SLAB - 1) // SLAB
    if sfa.shape != (m, kb) or sfb.shape != (nb, kb):
        raise ValueError(f"bad scale shapes {sfa.shape}, {sfb.shape}")
    return m, n, k, kb


def gemm_nt_ref(qa, sfa, qb, sfb):
    """Dense reference.  qa: M x K codes, sfa: M x K/128, qb: N x K codes,
    sfb: ceil(N/128) x K/128.  Returns the M x N fp64 result."""
    qa = np.asarray(qa, np.uint8)
    qb = np.asarray(qb, np.uint8)
    m, n, k, kb = _shapes(qa, sfa, qb, sfb)
    t = decode_table()
    sa = np.asarray(sfa, np.float64)
    sb = np.asarray(sfb, np.float64)
    block_of_col = np.arange(n) // SLAB
    r = np.zeros((m, n), dtype=np.float64)
    for s in range(kb):
        cols = slice(s * SLAB, (s + 1) * SLAB)
        a_dec = t[qa[:, cols]]
        b_dec = t[qb[:, cols]]
        p = a_dec @ b_dec.T  # exact slab sums
        scale = sa[:, s][:, None] * sb[block_of_col, s][None, :]
        r += p * scale
    return r


def _entries(a_codes, sa_rows, b_codes, sb_rows):
    """Element-wise results for paired rows: entry i is the dot of A row i
    with B row i under their slab scales (same slab order as gemm_nt_ref)."""
    t = decode_table()
    s_cnt, k = a_codes.shape
    kb = k // SLAB
    out = np.zeros(s_cnt, dtype=np.float64)
    chunk = max(1, (1 << 24) // max(k, 1))
    for c0 in range(0, s_cnt, chunk):
        c1 = min(s_cnt, c0 + chunk)
        prod = t[a_codes[c0:c1]] * t[b_codes[c0:c1]]
        p = prod.reshape(c1 - c0, kb, SLAB).sum(axis=2)  # exact slab sums
        acc = np.zeros(c1 - c0, dtype=np.float64)
        for s in range(kb):
            acc += p[:, s] * (np.float64(1) * sa_rows[c0:c1, s] * sb_rows[c0:c1, s])
        out[c0:c1] = acc
    return out


def gemm_nt_ref_at(qa, sfa, qb, sfb, rows, cols):
    """Dense reference at the given (rows[i], cols[i]) output positions."""
    rows = np.asarray(rows, np.int64)
    cols = np.asarray(cols, np.int64)
    sa = np.asarray(sfa, np.float64)
    sb = np.asarray(sfb, np.float64)
    return _entries(np.asarray(qa)[rows], sa[rows], np.asarray(qb)[cols], sb[cols // SLAB])


def grouped_contiguous_ref(qa, sfa, qb, sfb, m_indices):
    """Contiguous-layout grouped reference.

    qa: M x K, sfa: M x K/128, qb: G x N x K, sfb: G x ceil(N/128) x K/128,
    m_indices: M int32.  Returns (r, valid): r is M x N fp64 with NaN in
    rows whose index is outside [0, G); valid is the M-long row mask.
    """
    g_cnt, n, _ = qb.shape
    idx = np.asarray(m_indices, np.int64)
    m = qa.shape[0]
    r = np.full((m, n), np.nan, dtype=np.float64)
    valid = (idx >= 0) & (idx < g_cnt)
    for g in range(g_cnt):
        rows = np.nonzero(idx == g)[0]
        if rows.size:
            r[rows] = gemm_nt_ref(qa[rows], sfa[rows], qb[g], sfb[g])
    return r, valid


def grouped_contiguous_ref_at(qa, sfa, qb, sfb, m_indices, rows, cols):
    """Contiguous grouped reference at (rows[i], cols[i]); NaN where the row
    is a padding row."""
    g_cnt = qb.shape[0]
    rows = np.asarray(rows, np.int64)
    cols = np.asarray(cols, np.int64)
    g = np.asarray(m_indices, np.int64)[rows]
    ok = (g >= 0) & (g < g_cnt)
    out = np.full(rows.shape, np.nan)
    if ok.any():
        rr, cc, gg = rows[ok], cols[ok], g[ok]
        sa = np.asarray(sfa, np.float64)
        sb = np.asarray(sfb, np.float64)
        out[ok] = _entries(qa[rr], sa[rr], qb[gg, cc], sb[gg, cc // SLAB])
    return out


def _masked_counts(masked_m, max_m):
    return np.clip(np.asarray(masked_m, np.int64), 0, max_m)


def grouped_masked_ref(qa, sfa, qb, sfb, masked_m):
    """Masked-layout grouped reference.

    qa: G x max_m x K, sfa: G x max_m x K/128, qb: G x N x K,
    sfb: G x ceil(N/128) x K/128, masked_m: G int32.  Returns (r, valid):
    r is G x max_m x N fp64 with NaN in rows at or past min(masked_m[g], max_m).
    """
    g_cnt, max_m, _ = qa.shape
    n = qb.shape[1]
    cnt = _masked_counts(masked_m, max_m)
    r = np.full((g_cnt, max_m, n), np.nan, dtype=np.float64)
    valid = np.arange(max_m)[None, :] < cnt[:, None]
    for g in range(g_cnt):
        c = int(cnt[g])
        if c:
            r[g, :c] = gemm_nt_ref(qa[g, :c], sfa[g, :c], qb[g], sfb[g])
    return r, valid


def grouped_masked_ref_at(qa, sfa, qb, sfb, masked_m, groups, rows, cols):
    """Masked grouped reference at (groups[i], rows[i], cols[i]); NaN where
    the row is past the expert's valid count."""
    g_cnt, max_m, _ = qa.shape
    cnt = _masked_counts(masked_m, max_m)
    groups = np.asarray(groups, np.int64)
    rows = np.asarray(rows, np.int64)
    cols = np.asarray(cols, np.int64)
    ok = rows < cnt[groups]
    out = np.full(rows.shape, np.nan)
    if ok.any():
        gg, rr, cc = groups[ok], rows[ok], cols[ok]
        sa = np.asarray(sfa, np.float64)
        sb = np.asarray(sfb, np.float64)
        out[ok] = _entries(qa[gg, rr], sa[gg, rr], qb[gg, cc], sb[gg, cc // SLAB])
    return out


def _k_ranges(k_sizes, k_total):
    """Slab ranges [s0, s1) of the K groups; raises on sizes that are negative,
    not whole slabs, or past k_total."""
    sizes = np.asarray(k_sizes, np.int64)
    if np.any(sizes < 0) or np.any(sizes % SLAB):
        raise ValueError("k_sizes must be non-negative multiples of 128")
    ends = np.cumsum(sizes)
    if ends.size and ends[-1] > k_total:
        raise ValueError("k_sizes add up to more than K")
    starts = ends - sizes
    return [(int(a) // SLAB, int(b) // SLAB) for a, b in zip(starts, ends)]


def k_grouped_ref(qa, sfa, qb, sfb, k_sizes):
    """K-grouped reference.  qa: M x K, sfa: M x K/128, qb: N x K,
    sfb: ceil(N/128) x K/128, k_sizes: G group sizes along K.  Returns the
    G x M x N fp64 results, group g computed on its own K columns only."""
    qa = np.asarray(qa, np.uint8)
    qb = np.asarray(qb, np.uint8)
    m, n, k, _ = _shapes(qa, sfa, qb, sfb)
    ranges = _k_ranges(k_sizes, k)
    r = np.zeros((len(ranges), m, n), dtype=np.float64)
    for g, (s0, s1) in enumerate(ranges):
        if s1 > s0:
            cols = slice(s0 * SLAB, s1 * SLAB)
            r[g] = gemm_nt_ref(qa[:, cols], np.asarray(sfa)[:, s0:s1], qb[:, cols], np.asarray(sfb)[:, s0:s1])
    return r


def k_grouped_ref_at(qa, sfa, qb, sfb, k_sizes, groups, rows, cols):
    """K-grouped reference at (groups[i], rows[i], cols[i])."""
    qa = np.asarray(qa, np.uint8)
    qb = np.asarray(qb, np.uint8)
    ranges = _k_ranges(k_sizes, qa.shape[1])
    groups = np.asarray(groups, np.int64)
    rows = np.asarray(rows, np.int64)
    cols = np.asarray(cols, np.int64)
    sa = np.asarray(sfa, np.float64)
    sb = np.asarray(sfb, np.float64)
    out = np.zeros(rows.shape, dtype=np.float64)
    for g in np.unique(groups):
        s0, s1 = ranges[g]
        sel = np.nonzero(groups == g)[0]
        if s1 > s0:
            kc = slice(s0 * SLAB, s1 * SLAB)
            rr, cc = rows[sel], cols[sel]
            out[sel] = _entries(qa[rr, kc], sa[rr, s0:s1], qb[cc, kc], sb[cc // SLAB, s0:s1])
    return out


def bf16_to_f64(bits):
    """bf16 bit patterns (uint16) to float64, exactly: a bf16 value is the
    upper half of the fp32 with the same bits."""
    b = np.asarray(bits, np.uint16).astype(np.uint32) << 16
    return b.view(np.float32).astype(np.float64)


def bf16_gemm_nt_ref(a_bits, b_bits):
    """BF16 NT GEMM reference: D = A . B^T for bf16 A (M x K) and B (N x K),
    given as uint16 bit patterns, in fp64 (the BF16 family named on
    "DeepGEMM: making LLM matrix multiplication fly", pomoai.com, core
    functions).  No scales: bf16 keeps an 8-bit exponent, so the pages'
    fine-grained scaling is an FP8 device.  Each product of two bf16 values
    is exact in fp64 (8-bit significands); the sum over K is rounded to fp64."""
    a = bf16_to_f64(a_bits)
    b = bf16_to_f64(b_bits)
    if a.shape[1] != b.shape[1]:
        raise ValueError("A and B must share K")
    return a @ b.T


def silu(x):
    """SiLU (swish), x * sigmoid(x), in fp64 (exp overflows to inf for
    x < -709, where x / inf = -0 is the correctly rounded value)."""
    x = np.asarray(x, np.float64)
    with np.errstate(over="ignore"):
        return x / (1.0 + np.exp(-x))


def masked_swiglu_ref(qa, sfa, qb, sfb, masked_m):
    """FC1 of an MoE expert on the masked layout followed by SwiGLU, in fp64.

    The single-GPU slice of the fused MoE path (the popular-press article on
    DeepGEMM, yeyulingfeng.com, section 04 on Mega MoE: dispatch, the first
    GEMM, the SwiGLU activation and the second GEMM fused into one kernel).  Reading:
    B holds each expert's FC1 weight as [gate; up], 2I rows (I gate rows,
    then I up rows), and h = silu(A . gate^T) * (A . up^T).  Returns
    (h, valid): h is G x max_m x I with NaN in rows past masked_m[g]."""
    r, valid = grouped_masked_ref(qa, sfa, qb, sfb, masked_m)
    i = qb.shape[1] // 2
    if qb.shape[1] != 2 * i:
        raise ValueError("B must hold gate and up halves of equal size")
    return silu(r[..., :i]) * r[..., i:], valid


def masked_swiglu_quant_ref(qa, sfa, qb, sfb, masked_m):
    """FC1 + SwiGLU with h requantised as the second GEMM's A operand.

    Reading: the fused MoE path hands h to the second GEMM as FP8, so h is
    quantised with the activation rule (one fp32 scale per row and 128-wide
    slab of I; the scaling item of the DeepGEMM pages' technical features),
    exactly as quantize_a_1x128 does: the decision is taken in fp32 on
    fp32(h).  Returns (hq, hs, valid): hq is G x max_m x I e4m3 codes, hs is
    G x max_m x (I/128) fp32; rows past masked_m[g] hold code 0 and scale NaN.
    """
    from .quant import quantize_a_1x128

    h, valid = masked_swiglu_ref(qa, sfa, qb, sfb, masked_m)
    g, max_m, i = h.shape
    if i % 128 != 0:
        raise ValueError("I must be a multiple of 128")
    hq = np.zeros((g, max_m, i), np.uint8)
    hs = np.full((g, max_m, i // 128), np.nan, np.float32)
    for e in range(g):
        rows = int(valid[e].sum())
        if rows:
            hq[e, :rows], hs[e, :rows] = quantize_a_1x128(h[e, :rows].astype(np.float32))
    return hq, hs, valid


def contiguous_swiglu_ref(qa, sfa, qb, sfb, m_indices):
    """FC1 + SwiGLU on the contiguous layout (the prefill side of the same
    MoE path; the popular-press article's section on MoE pairs the
    contiguous layout with prefill and the masked one with decode), in fp64.
    Reading as for the masked layout: B holds each expert's FC1 weight as
    [gate; up], 2I rows, and h = silu(A . gate^T) * (A . up^T) for every row
    with a valid expert tag.  Returns (h, valid): h is M x I with NaN in
    padding rows."""
    r, valid = grouped_contiguous_ref(qa, sfa, qb, sfb, m_indices)
    i = qb.shape[1] // 2
    if qb.shape[1] != 2 * i:
        raise ValueError("B must hold gate and up halves of equal size")
    return silu(r[:, :i]) * r[:, i:], valid


def contiguous_swiglu_quant_ref(qa, sfa, qb, sfb, m_indices):
    """Contiguous FC1 + SwiGLU with h quantised by the activation rule, as
    the masked version does (one fp32 scale per row and 128-wide slab of I,
    the decision in fp32 on fp32(h)).  Returns (hq, hs, valid): hq is M x I
    e4m3 codes, hs is M x (I/128) fp32; padding rows hold code 0 and scale
    NaN."""
    from .quant import quantize_a_1x128

    h, valid = contiguous_swiglu_ref(qa, sfa, qb, sfb, m_indices)
    m, i = h.shape
    if i % 128 != 0:
        raise ValueError("I must be a multiple of 128")
    hq = np.zeros((m, i), np.uint8)
    hs = np.full((m, i // 128), np.nan, np.float32)
    rows = np.nonzero(valid)[0]
    if rows.size:
        hq[rows], hs[rows] = quantize_a_1x128(h[rows].astype(np.float32))
    return hq, hs, valid


def fp4_gemm_nt_ref(pa, sfa, pb, sfb):
    """FP4 (e2m1) block-scaled NT GEMM in fp64: the dense FP8 method with
    e2m1 operands (the pages name FP4 as a GEMM format, pomoai.com, core
    functions; readings: e2m1 values, packed two per byte, with the FP8
    scale layout: sfa M x K/128, sfb ceil(N/128) x K/128).

    r[m, n] = sum over slabs kb of
              (sum_{k in kb} a[m, k] b[n, k]) * sfa[m, kb] * sfb[n / 128, kb]
    """
    from .e2m1 import decode_packed
    a = decode_packed(pa)
    b = decode_packed(pb)
    m, k = a.shape
    n = b.shape[0]
    if b.shape[1] != k or k % SLAB:
        raise ValueError("bad operand shapes")
    kb = k // SLAB
    sa = np.asarray(sfa, np.float64)
    sb = np.asarray(sfb, np.float64)
    if sa.shape != (m, kb) or sb.shape != ((n + SLAB - 1) // SLAB, kb):
        raise ValueError("bad scale shapes")
    block_of_col = np.arange(n) // SLAB
    r = np.zeros((m, n))
    for s in range(kb):
        cols = slice(s * SLAB, (s + 1) * SLAB)
        r += (a[:, cols] @ b[:, cols].T) * (sa[:, s][:, None] * sb[block_of_col, s][None, :])
    return r
