"""Seeded synthetic inputs for the FP8 block-scaled NT GEMM.

This module draws the fp32 operands and the index arrays, and nothing else:
it holds none of the GEMM's or the quantiser's arithmetic.  Both the oracle
checks and the GPU runs take their inputs from here.

The workloads are the DeepSeek-V3/R1 layer shapes the pages benchmark
("DeepSeek open-source week day 3", deepseek.csdn.net, performance table;
PPIO's evaluation, juejin.cn, official speedup section).  No dataset or
weights are involved: activations are drawn N(0, 1), weights N(0, 0.02) where
the shape is a weight (decode and MoE shapes), all from
numpy.random.default_rng(seed) in a fixed order.
"""

import numpy as np

SLAB = 128
CONTIGUOUS_M_ALIGNMENT = 128


class Workload:
    """A named workload: its kind, sizes, and how to draw its inputs."""

    def __init__(self, name, kind, desc, **shape):
        self.name = name
        self.kind = kind  # "dense" | "contiguous" | "masked" | "kgrouped" | "bf16" | "swiglu" | "swiglu_contig" | "fp4"
        self.desc = desc
        self.shape = shape

    def __repr__(self):
        return f"Workload({self.name}, {self.kind}, {self.shape})"


WORKLOADS = {
    "dense_128x512x1024": Workload(
        "dense_128x512x1024", "dense", "dense FP8 NT GEMM, small (M=128 N=512 K=1024)",
        m=128, n=512, k=1024, b_std=1.0),
    "dense_decode_64x2112x7168": Workload(
        "dense_decode_64x2112x7168", "dense", "dense decode-shaped GEMM (M=64 N=2112 K=7168)",
        m=64, n=2112, k=7168, b_std=0.02),
    # The decode shape at a small batch (8 rows); an extra line beside the
    # pages' shapes, not one of them
    "dense_decode_8x2112x7168": Workload(
        "dense_decode_8x2112x7168", "dense", "dense decode-shaped GEMM, 8 rows (M=8 N=2112 K=7168)",
        m=8, n=2112, k=7168, b_std=0.02),
    "dense_large_4096x7168x16384": Workload(
        "dense_large_4096x7168x16384", "dense", "dense large GEMM (M=4096 N=7168 K=16384)",
        m=4096, n=7168, k=16384, b_std=1.0),
    # One GPU's share of the large GEMM sharded over 8 GPUs: split N (each
    # GPU holds 896 of B's 7168 rows) or split M (512 of A's 4096 rows),
    # drawn like the large shape
    "dense_shard_n_4096x896x16384": Workload(
        "dense_shard_n_4096x896x16384", "dense", "dense large GEMM, N/8 shard (M=4096 N=896 K=16384)",
        m=4096, n=896, k=16384, b_std=1.0),
    "dense_shard_m_512x7168x16384": Workload(
        "dense_shard_m_512x7168x16384", "dense", "dense large GEMM, M/8 shard (M=512 N=7168 K=16384)",
        m=512, n=7168, k=16384, b_std=1.0),
    "moe_contiguous_4x8192_n4096_k7168": Workload(
        "moe_contiguous_4x8192_n4096_k7168", "contiguous",
        "MoE grouped contiguous, 4 experts x 8192 rows, N=4096 K=7168",
        group_rows=(8192, 8192, 8192, 8192), n=4096, k=7168, b_std=0.02),
    "moe_masked_16x256_n4096_k7168": Workload(
        "moe_masked_16x256_n4096_k7168", "masked",
        "MoE grouped masked decode, 16 experts, max_m=256, N=4096 K=7168",
        g=16, max_m=256, n=4096, k=7168, b_std=0.02),
    # The masked decode shape with lighter experts: counts uniform on 0..64
    # (about 32 tokens per expert, the low-batch decode regime), same buffers
    "moe_masked_16x256_c64_n4096_k7168": Workload(
        "moe_masked_16x256_c64_n4096_k7168", "masked",
        "MoE grouped masked decode, 16 experts, max_m=256, counts U{0..64}, N=4096 K=7168",
        g=16, max_m=256, n=4096, k=7168, b_std=0.02, count_hi=64),
    # FP4 (e2m1) dense GEMM on the large dense shape, drawn as that shape
    "fp4_dense_4096x7168x16384": Workload(
        "fp4_dense_4096x7168x16384", "fp4", "FP4 dense GEMM (M=4096 N=7168 K=16384)",
        m=4096, n=7168, k=16384, b_std=1.0),
    # MoE FC1 + SwiGLU + FP8 requantisation on the masked decode layout: the
    # masked shape read as [gate; up] (2I = 4096 rows, I = 2048), drawn with
    # the same seed, so its inputs equal the masked workload's
    "moe_swiglu_16x256_i2048_k7168": Workload(
        "moe_swiglu_16x256_i2048_k7168", "swiglu",
        "MoE FC1 + SwiGLU + requantise, masked layout, 16 experts, max_m=256, I=2048 K=7168",
        g=16, max_m=256, inter=2048, k=7168, b_std=0.02),
    # the same with the light-expert counts (uniform on 0..64)
    "moe_swiglu_16x256_c64_i2048_k7168": Workload(
        "moe_swiglu_16x256_c64_i2048_k7168", "swiglu",
        "MoE FC1 + SwiGLU + requantise, masked layout, 16 experts, max_m=256, counts U{0..64}, I=2048 K=7168",
        g=16, max_m=256, inter=2048, k=7168, b_std=0.02, count_hi=64),
    # MoE FC1 + SwiGLU + FP8 requantisation on the contiguous (prefill)
    # layout: the contiguous shape read as [gate; up] (2I = 4096 rows,
    # I = 2048), drawn with the same seed, so its inputs equal the contiguous
    # workload's
    "moe_swiglu_contig_4x8192_i2048_k7168": Workload(
        "moe_swiglu_contig_4x8192_i2048_k7168", "swiglu_contig",
        "MoE FC1 + SwiGLU + requantise, contiguous layout, 4 experts x 8192 rows, I=2048 K=7168",
        group_rows=(8192, 8192, 8192, 8192), inter=2048, k=7168, b_std=0.02),
    # BF16 dense GEMM on the large dense shape (operands rounded to bf16 by
    # the caller from these fp32 draws)
    "bf16_dense_4096x7168x16384": Workload(
        "bf16_dense_4096x7168x16384", "bf16", "BF16 dense GEMM (M=4096 N=7168 K=16384)",
        m=4096, n=7168, k=16384, b_std=1.0),
    # K-grouped (MoE weight-gradient shape): 4 experts' 8192 tokens each on K,
    # M and N the expert FFN's output and input widths of the MoE shapes above
    "kgrouped_4x8192_m4096_n7168": Workload(
        "kgrouped_4x8192_m4096_n7168", "kgrouped",
        "K-grouped GEMM, 4 groups x 8192 K columns, M=4096 N=7168",
        k_sizes=(8192, 8192, 8192, 8192), m=4096, n=7168, b_std=1.0),
}


def _normal(rng, shape, std):
    x = rng.standard_normal(shape, dtype=np.float32)
    if std != 1.0:
        x *= np.float32(std)
    return x


def draw_dense(m, n, k, seed=0, b_std=1.0):
    """A (m x k) ~ N(0,1) then B (n x k) ~ N(0, b_std^2), both fp32."""
    rng = np.random.default_rng(seed)
    a = _normal(rng, (m, k), 1.0)
    b = _normal(rng, (n, k), b_std)
    return {"a": a, "b": b}


def contiguous_indices(group_rows, alignment=CONTIGUOUS_M_ALIGNMENT):
    """Row -> expert tags for the contiguous layout: each expert's rows are
    stacked in order and its segment is padded with -1 rows up to the
    alignment."""
    tags = []
    for g, cnt in enumerate(group_rows):
        padded = (cnt + alignment - 1) // alignment * alignment
        tags.append(np.full(cnt, g, dtype=np.int32))
        tags.append(np.full(padded - cnt, -1, dtype=np.int32))
    if not tags:
        return np.zeros(0, dtype=np.int32)
    return np.concatenate(tags)


def draw_contiguous(group_rows, n, k, seed=0, b_std=0.02):
    """m_indices from group_rows (padded to 128); then A (M x k) ~ N(0,1) for
    all M rows, padding rows included; then B (G x n x k) ~ N(0, b_std^2)."""
    rng = np.random.default_rng(seed)
    m_indices = contiguous_indices(group_rows)
    a = _normal(rng, (m_indices.size, k), 1.0)
    b = _normal(rng, (len(group_rows), n, k), b_std)
    return {"a": a, "b": b, "m_indices": m_indices}


def draw_masked(g, max_m, n, k, seed=0, b_std=0.02, masked_m=None, count_hi=None):
    """First masked_m ~ Uniform{0..count_hi} per expert (count_hi defaults to
    max_m; unless masked_m is given), then A (g x max_m x k) ~ N(0,1) with
    the invalid rows drawn too, then B (g x n x k) ~ N(0, b_std^2)."""
    rng = np.random.default_rng(seed)
    if masked_m is None:
        hi = max_m if count_hi is None else count_hi
        masked_m = rng.integers(0, hi + 1, g).astype(np.int32)
    else:
        masked_m = np.asarray(masked_m, dtype=np.int32)
    a = _normal(rng, (g, max_m, k), 1.0)
    b = _normal(rng, (g, n, k), b_std)
    return {"a": a, "b": b, "masked_m": masked_m}


def draw_kgrouped(k_sizes, m, n, seed=0, b_std=1.0, k_total=None):
    """A (m x K) ~ N(0,1) then B (n x K) ~ N(0, b_std^2), K = k_total or the
    sum of the group sizes (both operands hold activation-like data: output
    gradients and layer inputs, tokens along K)."""
    rng = np.random.default_rng(seed)
    k = int(sum(k_sizes)) if k_total is None else int(k_total)
    a = _normal(rng, (m, k), 1.0)
    b = _normal(rng, (n, k), b_std)
    return {"a": a, "b": b, "k_sizes": np.asarray(k_sizes, dtype=np.int32)}


def draw(name, seed=0):
    """Draw the named workload's inputs with its recipe."""
    w = WORKLOADS[name]
    s = w.shape
    if w.kind in ("dense", "bf16", "fp4"):
        return draw_dense(s["m"], s["n"], s["k"], seed, s["b_std"])
    if w.kind == "contiguous":
        return draw_contiguous(s["group_rows"], s["n"], s["k"], seed, s["b_std"])
    if w.kind == "swiglu_contig":
        return draw_contiguous(s["group_rows"], 2 * s["inter"], s["k"], seed, s["b_std"])
    if w.kind == "kgrouped":
        return draw_kgrouped(s["k_sizes"], s["m"], s["n"], seed, s["b_std"])
    if w.kind == "swiglu":
        return draw_masked(s["g"], s["max_m"], 2 * s["inter"], s["k"], seed, s["b_std"], count_hi=s.get("count_hi"))
    return draw_masked(s["g"], s["max_m"], s["n"], s["k"], seed, s["b_std"], count_hi=s.get("count_hi"))


def algorithmic_work(kind, **p):
    """Algorithmic flops and HBM bytes of one GEMM call.

    flops = 2 * (valid rows) * N * K.  Bytes count every operand once: the
    valid rows of A (1 byte per element) and their fp32 scales, B (1 byte per
    element) of every expert that has at least one valid row, its fp32 scales,
    the index array, and D (bf16, 2 bytes) for the valid rows.  This is the
    convention under which the pages' decode-shape pair (206 TFLOPS with
    1688 GB/s at M=64 N=2112 K=7168, "DeepSeek open-source week day 3",
    performance table) is self-consistent.
    """
    n, k = p["n"], p["k"]
    kb = k // SLAB
    nb = (n + SLAB - 1) // SLAB
    if kind == "dense":
        rows, experts, index_bytes = p["m"], 1, 0
    elif kind == "contiguous":
        m_indices = np.asarray(p["m_indices"])
        g = p["g"]
        ok = (m_indices >= 0) & (m_indices < g)
        rows = int(ok.sum())
        experts = int(np.unique(m_indices[ok]).size)
        index_bytes = 4 * m_indices.size
    elif kind == "masked":
        cnt = np.clip(np.asarray(p["masked_m"], np.int64), 0, p["max_m"])
        rows = int(cnt.sum())
        experts = int((cnt > 0).sum())
        index_bytes = 4 * cnt.size
    elif kind == "swiglu":
        # the masked FC1 GEMM with n = 2I, writing h as e4m3 codes (1 byte)
        # with one fp32 scale per 128 columns instead of D
        cnt = np.clip(np.asarray(p["masked_m"], np.int64), 0, p["max_m"])
        rows, experts = int(cnt.sum()), int((cnt > 0).sum())
        i = n // 2
        flops = 2.0 * rows * n * k
        nbytes = (rows * k + 4 * rows * kb + experts * (n * k + 4 * nb * kb) + 4 * cnt.size
                  + rows * i + 4 * rows * (i // SLAB))
        return flops, nbytes
    elif kind == "swiglu_contig":
        # the contiguous FC1 GEMM with n = 2I, writing h for the tagged rows
        # as e4m3 codes (1 byte) with one fp32 scale per 128 columns
        m_indices = np.asarray(p["m_indices"])
        g = p["g"]
        ok = (m_indices >= 0) & (m_indices < g)
        rows = int(ok.sum())
        experts = int(np.unique(m_indices[ok]).size)
        i = n // 2
        flops = 2.0 * rows * n * k
        nbytes = (rows * k + 4 * rows * kb + experts * (n * k + 4 * nb * kb) + 4 * m_indices.size
                  + rows * i + 4 * rows * (i // SLAB))
        return flops, nbytes
    elif kind == "fp4":
        # half a byte per element of A and B, their fp32 scales, bf16 D
        m = p["m"]
        return 2.0 * m * n * k, m * k // 2 + 4 * m * kb + n * k // 2 + 4 * nb * kb + 2 * m * n
    elif kind == "bf16":
        # two bytes per element of A, B and D; no scales
        m = p["m"]
        return 2.0 * m * n * k, 2 * (m * k + n * k + m * n)
    elif kind == "kgrouped":
        # every group reads its own K columns of A and B once and writes a
        # full M x N result (zeros for an empty group)
        sizes = np.maximum(np.asarray(p["k_sizes"], np.int64), 0)
        m, kk, g = p["m"], int(sizes.sum()), sizes.size
        kbb = kk // SLAB
        flops = 2.0 * m * n * kk
        nbytes = m * kk + 4 * m * kbb + n * kk + 4 * nb * kbb + 4 * g + 2 * g * m * n
        return flops, nbytes
    else:
        raise ValueError(kind)
    flops = 2.0 * rows * n * k
    nbytes = (rows * k + 4 * rows * kb + experts * (n * k + 4 * nb * kb)
              + index_bytes + 2 * rows * n)
    return flops, nbytes


def workload_work(name, inputs=None):
    """algorithmic_work for a named workload (inputs needed for the grouped
    kinds, whose valid-row counts come from the drawn index arrays)."""
    w = WORKLOADS[name]
    s = w.shape
    if w.kind == "dense":
        return algorithmic_work("dense", m=s["m"], n=s["n"], k=s["k"])
    if w.kind == "contiguous":
        mi = inputs["m_indices"] if inputs is not None else contiguous_indices(s["group_rows"])
        return algorithmic_work("contiguous", m_indices=mi, g=len(s["group_rows"]), n=s["n"], k=s["k"])
    if w.kind == "swiglu_contig":
        mi = inputs["m_indices"] if inputs is not None else contiguous_indices(s["group_rows"])
        return algorithmic_work("swiglu_contig", m_indices=mi, g=len(s["group_rows"]), n=2 * s["inter"], k=s["k"])
    if w.kind in ("bf16", "fp4"):
        return algorithmic_work(w.kind, m=s["m"], n=s["n"], k=s["k"])
    if w.kind == "kgrouped":
        return algorithmic_work("kgrouped", k_sizes=s["k_sizes"], m=s["m"], n=s["n"], k=int(sum(s["k_sizes"])))
    if w.kind == "swiglu":
        mm = inputs["masked_m"] if inputs is not None else np.random.default_rng(0).integers(0, s["max_m"] + 1, s["g"])
        return algorithmic_work("swiglu", masked_m=mm, max_m=s["max_m"], n=2 * s["inter"], k=s["k"])
    mm = inputs["masked_m"] if inputs is not None else np.random.default_rng(0).integers(0, s["max_m"] + 1, s["g"])
    return algorithmic_work("masked", masked_m=mm, max_m=s["max_m"], n=s["n"], k=s["k"])
