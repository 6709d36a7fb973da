"""Block quantisers (1x128 for A, 128x128 for B).  Test infrastructure only.

The pages describe the scaling only as "fine-grained" (deepseek.csdn.net,
"technical features", item on fine-grained dynamic scaling) and "block-wise,
each small block scaled independently" (pomoai.com, "core functions",
fourth point).  Readings taken:

* A (activations, M x K): one fp32 scale per row and per 128-wide K slab.
* B (weights, N x K): one fp32 scale per 128 x 128 block; the last row block
  may hold fewer than 128 rows when N is not a multiple of 128.
* For each block: amax = max |x| in fp32, floored at 1e-4 so an all-zero
  block does not divide by zero; s = fp32(amax / 448); each element is
  encoded as e4m3(fp32(x / s)) with nearest-even rounding and saturation at
  448.  Both divisions are IEEE fp32 divisions (correctly rounded), as numpy
  float32 division is.

The scales are returned in their logical shape: sfa is M x (K/128) and sfb is
ceil(N/128) x (K/128).  The GPU library's storage layout is not this module's
concern.
"""

import numpy as np

from .e4m3 import E4M3_MAX, encode

SLAB = 128
AMAX_FLOOR = np.float32(1e-4)
_F448 = np.float32(E4M3_MAX)


def _check_k(k):
    if k % SLAB != 0:
        raise ValueError(f"K must be a multiple of {SLAB}, got {k}")


def quantize_a_1x128(x):
    """Quantise an M x K fp32 matrix with one scale per 1 x 128 slice.

    Returns (q, sfa): q is M x K uint8 e4m3 codes, sfa is M x (K/128) fp32.
    """
    x = np.ascontiguousarray(x, dtype=np.float32)
    m, k = x.shape
    _check_k(k)
    kb = k // SLAB
    blocks = x.reshape(m, kb, SLAB)
    amax = np.max(np.abs(blocks), axis=2)  # exact in fp32
    amax = np.maximum(amax, AMAX_FLOOR)
    s = (amax / _F448).astype(np.float32)  # correctly rounded fp32 division
    scaled = (blocks / s[:, :, None]).astype(np.float32)
    q = encode(scaled).reshape(m, k)
    return q, s


def quantize_b_128x128(x):
    """Quantise an N x K fp32 matrix with one scale per 128 x 128 block.

    Returns (q, sfb): q is N x K uint8, sfb is ceil(N/128) x (K/128) fp32.
    The last row block may be partial.
    """
    x = np.ascontiguousarray(x, dtype=np.float32)
    n, k = x.shape
    _check_k(k)
    kb = k // SLAB
    nb = (n + SLAB - 1) // SLAB
    q = np.empty((n, k), dtype=np.uint8)
    sfb = np.empty((nb, kb), dtype=np.float32)
    for bi in range(nb):
        r0, r1 = bi * SLAB, min(n, (bi + 1) * SLAB)
        blk = x[r0:r1].reshape(r1 - r0, kb, SLAB)
        amax = np.max(np.abs(blk), axis=(0, 2))
        amax = np.maximum(amax, AMAX_FLOOR)
        s = (amax / _F448).astype(np.float32)
        sfb[bi] = s
        scaled = (blk / s[None, :, None]).astype(np.float32)
        q[r0:r1] = encode(scaled).reshape(r1 - r0, k)
    return q, sfb


# ---- FP4 (e2m1) quantisers: the same blocks and rule with the FP4 range

def _quant_fp4_blocks(blocks):
    """blocks [..., 128] fp32 -> (codes [..., 128] uint8, scale [...] fp32)
    with amax floored at 1e-4, s = fp32(amax / 6), code = e2m1(fp32(x / s))."""
    from .e2m1 import E2M1_MAX, encode as encode_e2m1
    amax = np.maximum(np.max(np.abs(blocks), axis=-1), AMAX_FLOOR)
    s = (amax / np.float32(E2M1_MAX)).astype(np.float32)
    scaled = (blocks / s[..., None]).astype(np.float32)
    return encode_e2m1(scaled), s


def quantize_a_1x128_fp4(x):
    """FP4 activations: as quantize_a_1x128 with the e2m1 range (6 instead of
    448).  Reading: the pages name FP4 without a scaling rule, so the FP8
    rule carries over.  Returns (packed, sfa): packed is M x K/2 bytes (low
    nibble first), sfa is M x K/128 fp32."""
    from .e2m1 import pack
    x = np.ascontiguousarray(x, dtype=np.float32)
    m, k = x.shape
    _check_k(k)
    codes, s = _quant_fp4_blocks(x.reshape(m, k // SLAB, SLAB))
    return pack(codes.reshape(m, k)), s


def quantize_b_128x128_fp4(x):
    """FP4 weights: as quantize_b_128x128 with the e2m1 range.  Returns
    (packed, sfb): packed is N x K/2 bytes, sfb is ceil(N/128) x K/128."""
    from .e2m1 import E2M1_MAX, encode as encode_e2m1, pack
    x = np.ascontiguousarray(x, dtype=np.float32)
    n, k = x.shape
    _check_k(k)
    kb = k // SLAB
    nb = (n + SLAB - 1) // SLAB
    codes = np.empty((n, k), dtype=np.uint8)
    sfb = np.empty((nb, kb), dtype=np.float32)
    for bi in range(nb):
        r0, r1 = bi * SLAB, min(n, (bi + 1) * SLAB)
        blk = x[r0:r1].reshape(r1 - r0, kb, SLAB)
        amax = np.maximum(np.max(np.abs(blk), axis=(0, 2)), AMAX_FLOOR)
        s = (amax / np.float32(E2M1_MAX)).astype(np.float32)
        sfb[bi] = s
        codes[r0:r1] = encode_e2m1((blk / s[None, :, None]).astype(np.float32)).reshape(r1 - r0, k)
    return pack(codes), sfb
